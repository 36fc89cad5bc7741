"""An independent formulation of the decoder, the PDM stack and the PDM's draft, for the
oracle's pins (CPU, float64).

It is written from the textbook definitions with other primitives than the oracle
uses: torch's scaled_dot_product_attention (GQA) over whole causal sequences, torch's
rms_norm and silu, RoPE in complex form, and the closed-form sum for linear attention.
The storage roundings use torch's own float->bfloat16 cast. Nothing here steps a
pipeline: the PDM's draft for a step is one causal forward of the PDM over the step's
feature rows, each row's feature taken from a causal forward of the target at the depth
the row has when the PDM reads it (pith.science review, "What carries the argument":
concatenate the hidden states at the deepest computed anchors, project, then the
speculation layers and the LM head).
"""
from __future__ import annotations

import numpy as np
import torch
import torch.nn.functional as F

from oracle.model import lin_gammas
from spd_inputs import SOFTMAX

f64 = torch.float64


def tensor(W, name):
    a = W[name]
    if a.dtype == np.uint16:
        return torch.from_numpy((a.astype(np.uint32) << 16).view(np.float32)).to(f64)
    return torch.from_numpy(np.asarray(a)).to(f64)


def bf(x):
    return x.to(torch.float32).to(torch.bfloat16).to(f64)


def f32(x):
    return x.to(torch.float32).to(f64)


def rope(x, pos, theta):
    hd = x.shape[-1]
    half = hd // 2
    w = theta ** (-2.0 * torch.arange(half, dtype=f64) / hd)
    ang = pos.to(f64)[:, None, None] * w
    z = torch.complex(x[..., :half], x[..., half:]) * torch.polar(torch.ones_like(ang), ang)
    return torch.cat([z.real, z.imag], dim=-1)


def linear_closed_form(q, k, v, gam):
    """o_t = sum_{j<=t} gamma^(t-j) (qh_t . kh_j) v_j for every head (no recurrence)."""
    P = q.shape[0]
    qh = q / torch.sqrt((q * q).sum(-1, keepdim=True) + 1e-6)
    kh = k / torch.sqrt((k * k).sum(-1, keepdim=True) + 1e-6)
    t = torch.arange(P, dtype=f64)
    decay = gam[None, None, :] ** (t[:, None, None] - t[None, :, None])       # [t, j, h]
    decay = torch.where((t[:, None] >= t[None, :])[..., None], decay, torch.zeros_like(decay))
    s = torch.einsum("thd,jhd->tjh", qh, kh) * decay
    return torch.einsum("tjh,jhd->thd", s, v)


def layer(cfg, W, prefix, kind, H, round_gemm=False):
    """One pre-norm decoder layer over the whole causal sequence H (positions 0..P-1).
    Returns (new H, stored K, stored V) with K, V as [P, hkv, hd] (None for linear)."""
    bf16 = cfg.dtype == "bf16"
    store = bf if (bf16 and cfg.kv_dtype != "f32") else f32
    gin = bf if (bf16 and round_gemm) else (lambda x: x)
    d, hq, hkv, hd = cfg.d_model, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    P = H.shape[0]
    pos = torch.arange(P)
    a = F.rms_norm(H, (d,), tensor(W, prefix + "attn_norm"), cfg.rms_eps)
    qkv = gin(a) @ tensor(W, prefix + "w_qkv").T
    K = V = None
    if kind == SOFTMAX:
        q = rope(qkv[:, :hq * hd].reshape(P, hq, hd), pos, cfg.rope_theta)
        K = store(rope(qkv[:, hq * hd:(hq + hkv) * hd].reshape(P, hkv, hd), pos, cfg.rope_theta))
        V = store(qkv[:, (hq + hkv) * hd:].reshape(P, hkv, hd))
        o = F.scaled_dot_product_attention(q.transpose(0, 1)[None], K.transpose(0, 1)[None],
                                           V.transpose(0, 1)[None], is_causal=True,
                                           enable_gqa=True)[0].transpose(0, 1)
    else:
        q = qkv[:, :hq * hd].reshape(P, hq, hd)
        k = qkv[:, hq * hd:2 * hq * hd].reshape(P, hq, hd)
        v = qkv[:, 2 * hq * hd:].reshape(P, hq, hd)
        o = linear_closed_form(q, k, v, torch.from_numpy(lin_gammas(hq)))
    H = H + gin(o.reshape(P, -1)) @ tensor(W, prefix + "w_o").T
    b = gin(F.rms_norm(H, (d,), tensor(W, prefix + "ffn_norm"), cfg.rms_eps))
    act = F.silu(b @ tensor(W, prefix + "w_gate").T) * (b @ tensor(W, prefix + "w_up").T)
    return H + gin(act) @ tensor(W, prefix + "w_down").T, K, V


def target_depths(cfg, W, tokens, round_gemm=False):
    """Residual rows after every depth 0..L of a causal forward over `tokens`:
    a list of L + 1 tensors [P, d] (depth 0 is the embedding)."""
    H = tensor(W, "embed")[torch.from_numpy(np.asarray(tokens, np.int64))]
    out = [H]
    for l in range(cfg.n_layers):
        H, _, _ = layer(cfg, W, f"layers.{l}.", cfg.kinds[l], H, round_gemm)
        out.append(H)
    return out


def torch_forward(cfg, W, tokens, round_gemm=False):
    """Whole-prompt forward; returns (final residual rows, logits of the last row)."""
    H = target_depths(cfg, W, tokens, round_gemm)[-1]
    z = tensor(W, "lm_head") @ F.rms_norm(H[-1], (cfg.d_model,), tensor(W, "final_norm"),
                                         cfg.rms_eps)
    return H.numpy(), z.numpy()


def features(cfg, depths_H, depth_of, anchors, fill="clamp"):
    """The PDM feature rows [P, k d]: row x concatenates, in ascending anchor order, the
    residual at each anchor b <= depth_of[x], and for an anchor not yet reached the deepest
    one that is (clamp) or zeros (zero fill)."""
    P = depths_H[0].shape[0]
    rows = []
    for x in range(P):
        dx = depth_of[x]
        reached = [b for b in anchors if b <= dx]
        parts = []
        for b in anchors:
            if b <= dx:
                parts.append(depths_H[b][x])
            elif fill == "clamp":
                parts.append(depths_H[reached[-1]][x])
            else:
                parts.append(torch.zeros_like(depths_H[0][x]))
        rows.append(torch.cat(parts))
    return torch.stack(rows)


def pdm_forward(cfg, W, X, Ls):
    """The PDM over feature rows X [P, k d] at positions 0..P-1: projection, Ls decoder
    layers (causal), the PDM's own final norm on the last row and the tied LM head.
    Returns (draft logits of the last row, [(K, V) per PDM layer])."""
    Z = X @ tensor(W, "pdm.proj").T
    kv = []
    for r in range(Ls):
        Z, K, V = layer(cfg, W, f"pdm.layers.{r}.", SOFTMAX, Z)
        kv.append((K, V))
    z = tensor(W, "lm_head") @ F.rms_norm(Z[-1], (cfg.d_model,), tensor(W, "pdm.final_norm"),
                                         cfg.rms_eps)
    return z.numpy(), kv
