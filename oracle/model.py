"""The target decoder and the PDM decoder stack, one position at a time or batched.

Architecture (the pages name none; the workloads say "dense decoder,
RMSNorm+RoPE, SwiGLU", plus a hybrid with linear-attention layers). Layer l,
softmax kind, on residual h at position pos:
    a = RMSNorm(h) * g1
    q, k, v = split(W_qkv a)              q: hq heads, k and v: hkv heads, hd each
    q, k = RoPE(q, pos), RoPE(k, pos)
    K[pos], V[pos] = store(k), store(v)   (KV cache in the weight dtype)
    o_i = sum_j softmax_j(q_i . K_j / sqrt(hd)) V_j,  j <= pos, kv head i // (hq/hkv)
    h = h + W_o concat(o)
    b = RMSNorm(h) * g2
    h = h + W_down (silu(W_gate b) * (W_up b))
Linear kind (hybrid workload; a reading, since no page defines the layer):
    q, k, v = split(W_qkv a), hq heads each; qh = q/|q|, kh = k/|k| per head
    S_h = gamma_h S_h + kh_h v_h^T,  o_h = S_h^T qh_h,  gamma_h = 1 - 2^-(5 + h mod 8)
    no RoPE; S is snapshotted after every position so that a rejection can
    restore it.

Precision contract (a reading; the pages give none):
    * weights are the exact stored values (bf16 or f32);
    * activations, norms, softmax and accumulations: the oracle's float type;
    * the KV cache stores bf16 (bf16 workloads) or f32 (f32 workloads, or any workload
      whose kv_dtype is "f32");
    * prefill and decode both keep full-precision activations at every GEMM
      input (no bf16 rounding of activations): rounding them would turn
      last-bit differences between two correct implementations into logit
      differences of a few 1e-3, above the 1e-3 near-tie margin that the
      token comparison relies on.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence

import numpy as np

from spd_inputs.configs import LINEAR, SOFTMAX, ModelConfig
from .numerics import (apply_rope, bf16_bits_to_float, l2_normalize, rmsnorm,
                       round_to_bf16, round_to_f32, silu, softmax)

LIN_EPS = 1e-6


def lin_gammas(n_heads: int) -> np.ndarray:
    h = np.arange(n_heads)
    return 1.0 - 2.0 ** (-(5.0 + (h % 8)))


class Weights:
    """Read-only view of the generated tensors, upcast exactly to the oracle's float type."""

    def __init__(self, arrays: Dict[str, np.ndarray], ft=np.float64, cache: bool = True):
        self.arrays = arrays
        self.ft = ft
        self.cache = cache
        self._c: Dict[str, np.ndarray] = {}

    def __call__(self, name: str) -> np.ndarray:
        if name in self._c:
            return self._c[name]
        a = self.arrays[name]
        out = bf16_bits_to_float(a, self.ft) if a.dtype == np.uint16 else a.astype(self.ft)
        if self.cache:
            self._c[name] = out
        return out

    def row(self, name: str, idx: int) -> np.ndarray:
        a = self.arrays[name][idx]
        return bf16_bits_to_float(a, self.ft) if a.dtype == np.uint16 else a.astype(self.ft)


class Stack:
    """A list of decoder layers with their caches (target: L layers, PDM: Ls layers)."""

    def __init__(self, cfg: ModelConfig, W: Weights, prefix: str, kinds: Sequence[int]):
        self.cfg, self.W, self.prefix = cfg, W, prefix
        self.kinds = list(kinds)
        self.ft = W.ft
        # the KV cache is stored in the weight dtype unless the workload asks for fp32
        self.bf16 = cfg.dtype == "bf16" and cfg.kv_dtype != "f32"
        hkv, hd, T = cfg.n_kv_heads, cfg.head_dim, cfg.max_ctx
        self.K: List[Optional[np.ndarray]] = []
        self.V: List[Optional[np.ndarray]] = []
        self.S: List[Optional[np.ndarray]] = []
        self.snap: List[Dict[int, np.ndarray]] = []
        for kind in self.kinds:
            if kind == SOFTMAX:
                self.K.append(np.zeros((T, hkv, hd), self.ft))
                self.V.append(np.zeros((T, hkv, hd), self.ft))
                self.S.append(None)
            else:
                self.K.append(None)
                self.V.append(None)
                self.S.append(np.zeros((cfg.n_q_heads, hd, hd), self.ft))
            self.snap.append({})
        self.gam = lin_gammas(cfg.n_q_heads).astype(self.ft)
        # keys and values of sibling candidates: (layer, position, branch) -> (k, v)
        self.side: Dict[tuple, tuple] = {}

    # -- precision contract ------------------------------------------------
    def store(self, x: np.ndarray) -> np.ndarray:
        return round_to_bf16(x) if self.bf16 else round_to_f32(x)

    def gemm_in(self, x: np.ndarray) -> np.ndarray:
        """GEMM input in prefill: activations stay at full precision."""
        return x

    def w(self, i: int, t: str) -> np.ndarray:
        return self.W(f"{self.prefix}.{i}.{t}")

    # -- one position ------------------------------------------------------
    def decode_layer(self, i: int, h: np.ndarray, pos: int, branch: int = 0) -> np.ndarray:
        """Layer i on residual h at position pos. branch > 0: a sibling candidate of the
        token at pos (draft tree): its key and value go to a side entry, and it attends over
        the cached positions before pos and its own key, not the main token's."""
        c = self.cfg
        a = rmsnorm(h, self.w(i, "attn_norm"), c.rms_eps)
        qkv = self.w(i, "w_qkv") @ a
        if self.kinds[i] == SOFTMAX:
            o = self._attend_one(i, qkv, pos, branch)
        else:
            assert branch == 0, "sibling candidates need softmax layers"
            o = self._linear_one(i, qkv, pos)
        h = h + self.w(i, "w_o") @ o
        b = rmsnorm(h, self.w(i, "ffn_norm"), c.rms_eps)
        act = silu(self.w(i, "w_gate") @ b) * (self.w(i, "w_up") @ b)
        return h + self.w(i, "w_down") @ act

    def _attend_one(self, i: int, qkv: np.ndarray, pos: int, branch: int = 0) -> np.ndarray:
        c = self.cfg
        hq, hkv, hd = c.n_q_heads, c.n_kv_heads, c.head_dim
        q = qkv[: hq * hd].reshape(hq, hd)
        k = qkv[hq * hd:(hq + hkv) * hd].reshape(hkv, hd)
        v = qkv[(hq + hkv) * hd:].reshape(hkv, hd)
        q = apply_rope(q, pos, c.rope_theta)
        k = apply_rope(k, pos, c.rope_theta)
        if branch == 0:
            self.K[i][pos] = self.store(k)
            self.V[i][pos] = self.store(v)
            Ks, Vs = self.K[i][: pos + 1], self.V[i][: pos + 1]
        else:
            ks, vs = self.store(k), self.store(v)
            self.side[(i, pos, branch)] = (ks, vs)
            Ks = np.concatenate([self.K[i][:pos], ks[None]])
            Vs = np.concatenate([self.V[i][:pos], vs[None]])
        group = hq // hkv
        o = np.empty((hq, hd), self.ft)
        for head in range(hq):
            g = head // group
            s = (Ks[:, g, :] @ q[head]) / np.sqrt(hd)
            o[head] = softmax(s) @ Vs[:, g, :]
        return o.reshape(-1)

    def _linear_one(self, i: int, qkv: np.ndarray, pos: int) -> np.ndarray:
        c = self.cfg
        H, hd = c.n_q_heads, c.head_dim
        q = qkv[: H * hd].reshape(H, hd)
        k = qkv[H * hd: 2 * H * hd].reshape(H, hd)
        v = qkv[2 * H * hd:].reshape(H, hd)
        qh, kh = l2_normalize(q, LIN_EPS), l2_normalize(k, LIN_EPS)
        S = self.gam[:, None, None] * self.S[i] + kh[:, :, None] * v[:, None, :]
        self.S[i] = S
        self.snap[i][pos] = S.copy()
        for old in [p for p in self.snap[i] if p < pos - 4 * (self.cfg.n_stages + 2)]:
            del self.snap[i][old]
        return np.einsum("hij,hi->hj", S, qh).reshape(-1)

    # -- many positions (prefill) ---------------------------------------------
    def prefill_layer(self, i: int, H: np.ndarray, pos0: int) -> np.ndarray:
        c = self.cfg
        A = rmsnorm(H, self.w(i, "attn_norm"), c.rms_eps)
        QKV = self.gemm_in(A) @ self.w(i, "w_qkv").T
        if self.kinds[i] == SOFTMAX:
            O = self._attend_many(i, QKV, pos0)
        else:
            O = self._linear_many(i, QKV, pos0)
        H = H + self.gemm_in(O) @ self.w(i, "w_o").T
        B = self.gemm_in(rmsnorm(H, self.w(i, "ffn_norm"), c.rms_eps))
        act = silu(B @ self.w(i, "w_gate").T) * (B @ self.w(i, "w_up").T)
        return H + self.gemm_in(act) @ self.w(i, "w_down").T

    def _attend_many(self, i: int, QKV: np.ndarray, pos0: int) -> np.ndarray:
        c = self.cfg
        hq, hkv, hd = c.n_q_heads, c.n_kv_heads, c.head_dim
        P = QKV.shape[0]
        pos = pos0 + np.arange(P)
        q = apply_rope(QKV[:, : hq * hd].reshape(P, hq, hd), pos, c.rope_theta)
        k = apply_rope(QKV[:, hq * hd:(hq + hkv) * hd].reshape(P, hkv, hd), pos, c.rope_theta)
        v = QKV[:, (hq + hkv) * hd:].reshape(P, hkv, hd)
        self.K[i][pos] = self.store(k)
        self.V[i][pos] = self.store(v)
        T = pos0 + P
        Ks, Vs = self.K[i][:T], self.V[i][:T]
        future = np.arange(T)[None, :] > pos[:, None]          # causal mask
        group = hq // hkv
        O = np.empty((P, hq, hd), self.ft)
        for head in range(hq):
            g = head // group
            s = (q[:, head, :] @ Ks[:, g, :].T) / np.sqrt(hd)
            s[future] = -np.inf
            O[:, head, :] = softmax(s, axis=-1) @ Vs[:, g, :]
        return O.reshape(P, -1)

    def _linear_many(self, i: int, QKV: np.ndarray, pos0: int) -> np.ndarray:
        c = self.cfg
        H, hd = c.n_q_heads, c.head_dim
        P = QKV.shape[0]
        q = l2_normalize(QKV[:, : H * hd].reshape(P, H, hd), LIN_EPS)
        k = l2_normalize(QKV[:, H * hd: 2 * H * hd].reshape(P, H, hd), LIN_EPS)
        v = QKV[:, 2 * H * hd:].reshape(P, H, hd)
        O = np.empty((P, H, hd), self.ft)
        S = self.S[i]
        for r in range(P):
            S = self.gam[:, None, None] * S + k[r][:, :, None] * v[r][:, None, :]
            O[r] = np.einsum("hij,hi->hj", S, q[r])
        self.S[i] = S
        self.snap[i][pos0 + P - 1] = S.copy()
        return O.reshape(P, -1)

    # -- draft tree -----------------------------------------------------------------
    def adopt(self, pos: int, branch: int, layers: Sequence[int]) -> None:
        """The sibling `branch` at pos becomes the main token there: its keys and values of
        the given layers move into the cache at pos."""
        for i in layers:
            self.K[i][pos], self.V[i][pos] = self.side[(i, pos, branch)]

    def drop_side(self, keep) -> None:
        """Forget the sibling entries whose position fails keep(pos)."""
        for key in [k for k in self.side if not keep(k[1])]:
            del self.side[key]

    # -- rejection ---------------------------------------------------------------
    def truncate(self, length: int) -> None:
        """Drop every cached position >= length (KV rows zeroed, linear state restored)."""
        for i, kind in enumerate(self.kinds):
            if kind == SOFTMAX:
                self.K[i][length:] = 0.0
                self.V[i][length:] = 0.0
            elif any(p >= length for p in self.snap[i]):
                # the state absorbed dropped positions: go back to the one after length-1
                self.S[i] = self.snap[i][length - 1].copy()
                for p in [p for p in self.snap[i] if p >= length]:
                    del self.snap[i][p]


class Model:
    """Target decoder + PDM decoder sharing one weight table (the LM head is tied)."""

    def __init__(self, cfg: ModelConfig, arrays: Dict[str, np.ndarray], ft=np.float64,
                 cache: bool = True, weights: Optional[Weights] = None):
        self.cfg = cfg
        # a prebuilt Weights shares its upcast tensors between several runs of one model
        self.W = weights if weights is not None else Weights(arrays, ft, cache)
        self.ft = ft
        self.target = Stack(cfg, self.W, "layers", cfg.kinds)
        self.pdm = Stack(cfg, self.W, "pdm.layers", (SOFTMAX,) * cfg.pdm_layers)

    def embed(self, tok: int) -> np.ndarray:
        return self.W.row("embed", int(tok))

    def embed_many(self, toks: np.ndarray) -> np.ndarray:
        return np.stack([self.embed(t) for t in toks])

    def logits(self, h: np.ndarray, norm: str = "final_norm") -> np.ndarray:
        """LM head on the final-normed residual (the head is shared by target and PDM)."""
        x = rmsnorm(h, self.W(norm), self.cfg.rms_eps)
        return self.W("lm_head") @ x
