"""Pins for the oracle's decoder against an independent formulation built from library routines.

The reference (tests/reference_torch.py) is written from the textbook definitions
with other primitives than the oracle uses: torch's scaled_dot_product_attention
(GQA), torch's rms_norm and silu, RoPE in complex form, and the closed-form sum for
linear attention. The bf16 roundings use torch's own float->bfloat16 cast.
"""
import numpy as np
import pytest

from conftest import workload
from oracle.model import Model
from oracle.spd import ar_decode
from reference_torch import torch_forward
from spd_inputs import LINEAR


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


def test_fp32_kv_cache_option_matches_reference():
    """kv_dtype "f32" on a bf16 model: the oracle stores K and V as fp32 (no bf16 rounding),
    and its prefill and per-position decode both match the reference with an fp32 store."""
    cfg, W, prompt = workload("mid_bf16_L4_d512_hd128_n4")
    cfg = cfg.with_(kv_dtype="f32")
    toks = prompt[:24]
    m = Model(cfg, W)
    H = m.embed_many(toks)
    for l in range(cfg.n_layers):
        H = m.target.prefill_layer(l, H, 0)
    Href, zref = torch_forward(cfg, W, toks)
    np.testing.assert_allclose(H, Href, rtol=0, atol=1e-9 * max(1.0, np.abs(Href).max()))
    # the stored keys are fp32 values, not all bf16 ones
    k = m.target.K[0][:24]
    assert np.array_equal(k, k.astype(np.float32).astype(np.float64))
    bits = k.astype(np.float32).view(np.uint32) & 0xFFFF
    assert bits.any()
