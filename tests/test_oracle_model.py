"""Pins for the oracle's decoder against an independent formulation built from library routines.

The reference here is written from the textbook definitions with other
primitives than the oracle uses: torch's scaled_dot_product_attention (GQA),
torch's rms_norm and silu, RoPE in complex form, and the closed-form sum for
linear attention. The bf16 roundings use torch's own float->bfloat16 cast.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from conftest import workload
from oracle.model import Model, lin_gammas
from oracle.spd import ar_decode
from spd_inputs import LINEAR, SOFTMAX

f64 = torch.float64


def _t(W, name):
    a = W[name]
    if a.dtype == np.uint16:
        return torch.from_numpy((a.astype(np.uint32) << 16).view(np.float32)).to(f64)
    return torch.from_numpy(a).to(f64)


def _bf(x):
    return x.to(torch.float32).to(torch.bfloat16).to(f64)


def _f32(x):
    return x.to(torch.float32).to(f64)


def _rope(x, pos, theta):
    hd = x.shape[-1]
    half = hd // 2
    w = theta ** (-2.0 * torch.arange(half, dtype=f64) / hd)
    ang = pos.to(f64)[:, None, None] * w
    z = torch.complex(x[..., :half], x[..., half:]) * torch.polar(torch.ones_like(ang), ang)
    return torch.cat([z.real, z.imag], dim=-1)


def _linear_closed_form(q, k, v, gam):
    """o_t = sum_{j<=t} gamma^(t-j) (qh_t . kh_j) v_j for every head (no recurrence)."""
    P = q.shape[0]
    qh = q / torch.sqrt((q * q).sum(-1, keepdim=True) + 1e-6)
    kh = k / torch.sqrt((k * k).sum(-1, keepdim=True) + 1e-6)
    t = torch.arange(P, dtype=f64)
    decay = gam[None, None, :] ** (t[:, None, None] - t[None, :, None])       # [t, j, h]
    decay = torch.where((t[:, None] >= t[None, :])[..., None], decay, torch.zeros_like(decay))
    s = torch.einsum("thd,jhd->tjh", qh, kh) * decay
    return torch.einsum("tjh,jhd->thd", s, v)


def torch_forward(cfg, W, tokens, round_gemm=False):
    """Whole-prompt forward; returns (final residual rows, logits of the last row)."""
    bf16 = cfg.dtype == "bf16"
    store = _bf if bf16 else _f32
    gin = _bf if (bf16 and round_gemm) else (lambda x: x)
    d, hq, hkv, hd = cfg.d_model, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    P = len(tokens)
    pos = torch.arange(P)
    H = _t(W, "embed")[torch.from_numpy(np.asarray(tokens, np.int64))]
    for l in range(cfg.n_layers):
        p = f"layers.{l}."
        a = F.rms_norm(H, (d,), _t(W, p + "attn_norm"), cfg.rms_eps)
        qkv = gin(a) @ _t(W, p + "w_qkv").T
        if cfg.kinds[l] == SOFTMAX:
            q = _rope(qkv[:, :hq * hd].reshape(P, hq, hd), pos, cfg.rope_theta)
            k = store(_rope(qkv[:, hq * hd:(hq + hkv) * hd].reshape(P, hkv, hd), pos, cfg.rope_theta))
            v = store(qkv[:, (hq + hkv) * hd:].reshape(P, hkv, hd))
            o = F.scaled_dot_product_attention(q.transpose(0, 1)[None], k.transpose(0, 1)[None],
                                               v.transpose(0, 1)[None], is_causal=True,
                                               enable_gqa=True)[0].transpose(0, 1)
        else:
            q = qkv[:, :hq * hd].reshape(P, hq, hd)
            k = qkv[:, hq * hd:2 * hq * hd].reshape(P, hq, hd)
            v = qkv[:, 2 * hq * hd:].reshape(P, hq, hd)
            o = _linear_closed_form(q, k, v, torch.from_numpy(lin_gammas(hq)))
        H = H + gin(o.reshape(P, -1)) @ _t(W, p + "w_o").T
        b = gin(F.rms_norm(H, (d,), _t(W, p + "ffn_norm"), cfg.rms_eps))
        act = F.silu(b @ _t(W, p + "w_gate").T) * (b @ _t(W, p + "w_up").T)
        H = H + gin(act) @ _t(W, p + "w_down").T
    z = _t(W, "lm_head") @ F.rms_norm(H[-1], (d,), _t(W, "final_norm"), cfg.rms_eps)
    return H.numpy(), z.numpy()


@pytest.mark.parametrize("name,plen,tol", [("tiny", 32, 1e-11), ("mid_bf16_L6_d384_n3", 40, 1e-9),
                                           ("mid_bf16_L4_d512_hd128_n4", 20, 1e-9),
                                           ("mid_hybrid_bf16_L8_d256_n4", 24, 1e-9)])
def test_prefill_matches_library_reference(name, plen, tol):
    cfg, W, prompt = workload(name)
    toks = prompt[:plen]
    m = Model(cfg, W)
    H = m.embed_many(toks)
    for l in range(cfg.n_layers):
        H = m.target.prefill_layer(l, H, 0)
    Href, zref = torch_forward(cfg, W, toks)
    np.testing.assert_allclose(H, Href, rtol=0, atol=tol * max(1.0, np.abs(Href).max()))
    np.testing.assert_allclose(m.logits(H[-1]), zref, rtol=0, atol=tol)


@pytest.mark.parametrize("name", ["tiny", "mid_bf16_L7_d256_n3_uneven", "mid_hybrid_bf16_L8_d256_n4"])
def test_decode_one_position_at_a_time_matches_reference(name):
    """Decode, one position at a time, equals the library forward over the whole prompt."""
    cfg, W, prompt = workload(name)
    toks = prompt[:20]
    m = Model(cfg, W)
    for pos, t in enumerate(toks):
        h = m.embed(t)
        for l in range(cfg.n_layers):
            h = m.target.decode_layer(l, h, pos)
    Href, zref = torch_forward(cfg, W, toks, round_gemm=False)
    np.testing.assert_allclose(h, Href[-1], rtol=0, atol=1e-9 * np.abs(Href).max())
    np.testing.assert_allclose(m.logits(h), zref, rtol=0, atol=1e-9)


@pytest.mark.parametrize("name", ["tiny", "mid_bf16_L6_d384_n3"])
def test_decode_equals_prefill(name):
    """The batched causal prefill and per-position decode agree (same roundings: the KV store)."""
    cfg, W, prompt = workload(name)
    prompt = prompt[:40]
    a, b = Model(cfg, W), Model(cfg, W)
    H = a.embed_many(prompt)
    for l in range(cfg.n_layers):
        H = a.target.prefill_layer(l, H, 0)
    for pos, t in enumerate(prompt):
        h = b.embed(t)
        for l in range(cfg.n_layers):
            h = b.target.decode_layer(l, h, pos)
        np.testing.assert_allclose(h, H[pos], rtol=0, atol=1e-9)
    for l in range(cfg.n_layers):
        np.testing.assert_allclose(a.target.K[l], b.target.K[l], atol=1e-9)


def test_gqa_head_mapping():
    """Query head i reads kv head i // (hq/hkv): zero all but one kv head's values."""
    cfg, W, prompt = workload("mid_bf16_L6_d384_n3")      # hq=6, hkv=2: group of 3
    m = Model(cfg, W)
    st = m.target
    hq, hkv, hd = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    rng = np.random.default_rng(0)
    qkv = rng.standard_normal((hq + 2 * hkv) * hd)
    qkv[(hq + hkv) * hd:(hq + hkv + 1) * hd] = 0.0          # kv head 0 values = 0
    qkv[(hq + hkv + 1) * hd:] = 1.0                          # kv head 1 values = 1
    o = st._attend_one(0, qkv, 0).reshape(hq, hd)
    np.testing.assert_array_equal(o[:3], 0.0)
    np.testing.assert_allclose(o[3:], 1.0)


def test_attention_over_one_key_returns_its_value():
    cfg, W, _ = workload("tiny")
    m = Model(cfg, W)
    hq, hd = cfg.n_q_heads, cfg.head_dim
    qkv = np.random.default_rng(1).standard_normal(3 * hq * hd)
    o = m.target._attend_one(0, qkv, 0)
    np.testing.assert_allclose(o, np.float32(qkv[2 * hq * hd:]).astype(np.float64), rtol=1e-15)


def test_linear_rollback_then_rerun_equals_clean_run():
    cfg, W, prompt = workload("mid_hybrid_bf16_L8_d256_n4")
    l = [i for i, k in enumerate(cfg.kinds) if k == LINEAR][0]
    rng = np.random.default_rng(2)
    good = [rng.standard_normal(cfg.d_model) for _ in range(8)]
    bad = [rng.standard_normal(cfg.d_model) for _ in range(3)]
    clean, dirty = Model(cfg, W).target, Model(cfg, W).target
    out_clean = [clean.decode_layer(l, h, p) for p, h in enumerate(good)]
    for p, h in enumerate(good[:5]):
        dirty.decode_layer(l, h, p)
    for j, h in enumerate(bad):
        dirty.decode_layer(l, h, 5 + j)
    dirty.truncate(5)
    out_dirty = [dirty.decode_layer(l, h, 5 + j) for j, h in enumerate(good[5:])]
    for a, b in zip(out_clean[5:], out_dirty):
        np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(clean.S[l], dirty.S[l])


def test_oracle_own_rounding_error_fp32_vs_fp64():
    """The oracle in float32 stays within 1e-5 of itself in float64 (tiny workload)."""
    cfg, W, prompt = workload("tiny")
    t64, z64 = ar_decode(cfg, W, prompt, G=24, return_logits=True)
    t32, z32 = ar_decode(cfg, W, prompt, G=24, ft=np.float32, return_logits=True)
    assert t64 == t32
    assert max(np.abs(a - b).max() for a, b in zip(z64, z32)) <= 1e-5
