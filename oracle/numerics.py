"""Scalar building blocks of the oracle: storage roundings and textbook layers.

The pages give no architecture; the workloads name a "dense decoder,
RMSNorm+RoPE, SwiGLU". These are the textbook forms:
  RMSNorm(x) = x / sqrt(mean(x^2) + eps) * g         (Zhang & Sennrich 2019)
  RoPE, rotate-half pairing (i, i + hd/2), angle pos * theta^(-2i/hd)
                                                      (Su et al. 2021)
  SwiGLU(b) = silu(b W_g^T) * (b W_u^T),  silu(x) = x / (1 + e^-x)
                                                      (Shazeer 2020)
"""
from __future__ import annotations

import numpy as np


def bf16_bits_to_float(bits: np.ndarray, dtype=np.float64) -> np.ndarray:
    """Exact value of bf16 bit patterns (uint16)."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(dtype)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Value after storing x as bfloat16.

    The GPU computes in float32 and stores with round-to-nearest-even, so the
    oracle first takes x to float32, then rounds the low 16 bits away with
    ties to even. Returns the result in x's dtype (a bf16 value exactly).
    """
    x = np.asarray(x)
    f = x.astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    keep = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + keep) >> np.uint64(16)) & np.uint64(0xFFFF)
    out = (r.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return out.astype(x.dtype if x.dtype.kind == "f" else np.float64)


def round_to_f32(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x)
    return x.astype(np.float32).astype(x.dtype)


def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * g over the last axis."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * g


def rope_angles(pos: np.ndarray, head_dim: int, theta: float) -> np.ndarray:
    """angle[p, i] = pos_p * theta^(-2i/hd) for i < hd/2, in float64."""
    half = head_dim // 2
    inv = theta ** (-(2.0 * np.arange(half, dtype=np.float64)) / head_dim)
    return np.asarray(pos, dtype=np.float64)[..., None] * inv


def apply_rope(x: np.ndarray, pos, theta: float) -> np.ndarray:
    """Rotate-half RoPE on x[..., heads, hd] at position(s) pos.

    pos is a scalar or an array broadcastable to x's leading axes (one entry
    per row). Pairs (i, i + hd/2) rotate by angle[pos, i].
    """
    hd = x.shape[-1]
    half = hd // 2
    ang = rope_angles(np.asarray(pos), hd, theta)      # [..., half]
    c = np.cos(ang)[..., None, :]
    s = np.sin(ang)[..., None, :]
    x1 = x[..., :half]
    x2 = x[..., half:]
    out = np.empty_like(x)
    out[..., :half] = x1 * c - x2 * s
    out[..., half:] = x1 * s + x2 * c
    return out


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


def softmax(x: np.ndarray, axis: int = -1) -> np.ndarray:
    m = np.max(x, axis=axis, keepdims=True)
    e = np.exp(x - m)
    return e / np.sum(e, axis=axis, keepdims=True)


def l2_normalize(x: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(sum(x^2) + eps) over the last axis (linear-attention q and k)."""
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)
