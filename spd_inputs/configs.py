"""Workload definitions: model shapes and SPD settings for every test and bench case.

This module only describes shapes and run settings. It holds none of the
method's arithmetic, so both the CPU oracle and the GPU path may import it.

Shapes follow the workloads that the speculative pipeline decoding pages
evaluate (a dense decoder split into n pipeline stages, anchors such as
[0, 8, 16, 24, 31], Ls = L/n speculation layers), at the sizes of the
synthetic stand-ins used here (random weights, uniform random prompts).
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import List, Optional, Tuple

SOFTMAX = 0
LINEAR = 1


@dataclass(frozen=True)
class ModelConfig:
    """A dense pre-norm decoder (RMSNorm, RoPE, GQA, SwiGLU) plus its SPD setup.

    Fields in the pages' notation: L = n_layers, n = n_stages, B = anchors,
    Ls = pdm_layers. Anchor b means "the residual stream after b target layers"
    (b = 0 is the token embedding, b = L the last layer's output before the
    final norm).
    """
    name: str
    n_layers: int
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    d_ffn: int
    vocab: int
    dtype: str                      # "f32" or "bf16": weight storage
    n_stages: int                   # n
    anchors: Tuple[int, ...]        # B, ascending, anchors[0] == 0
    pdm_layers: int                 # Ls
    prompt_len: int
    gen_len: int                    # G: generated tokens counting the prefill's first token
    max_ctx: int
    rope_theta: float = 10000.0
    rms_eps: float = 1e-6
    layer_kind: Tuple[int, ...] = ()   # per layer SOFTMAX / LINEAR; empty = all softmax
    stage_layers: Tuple[int, ...] = ()  # explicit stage sizes; empty = default split
    proj_init: str = "normal"        # "normal" or "select_deepest"
    weight_std: float = 0.02
    proj_noise_std: float = 0.05     # only for proj_init == "select_deepest"
    temperatures: Tuple[float, ...] = (0.0,)
    top_p: float = 1.0
    weight_seed: int = 0
    prompt_seed: int = 1
    kv_dtype: str = "auto"           # KV cache storage: "auto" (the weight dtype) or "f32"
    draft_width: int = 1             # W: draft candidates per position (1: a chain)

    @property
    def kinds(self) -> Tuple[int, ...]:
        return self.layer_kind if self.layer_kind else (SOFTMAX,) * self.n_layers

    @property
    def qkv_rows(self) -> int:
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim

    def lin_qkv_rows(self) -> int:
        return 3 * self.n_q_heads * self.head_dim

    def with_(self, **kw) -> "ModelConfig":
        return replace(self, **kw)


def hybrid_kinds(n_layers: int) -> Tuple[int, ...]:
    """3 linear-attention layers, then 1 softmax layer, repeated."""
    return tuple(SOFTMAX if (l % 4) == 3 else LINEAR for l in range(n_layers))


# ---- the five workloads -------------------------------------------------

TINY = ModelConfig(
    name="tiny_f32_L4_d64_n2",
    n_layers=4, d_model=64, n_q_heads=4, n_kv_heads=4, head_dim=16, d_ffn=256,
    vocab=512, dtype="f32", n_stages=2, anchors=(0, 2, 4), pdm_layers=1,
    prompt_len=32, gen_len=64, max_ctx=128, proj_init="select_deepest",
)

D2560_N4 = ModelConfig(
    name="dense_bf16_L32_d2560_n4",
    n_layers=32, d_model=2560, n_q_heads=32, n_kv_heads=8, head_dim=80, d_ffn=9728,
    vocab=151936, dtype="bf16", n_stages=4, anchors=(0, 8, 16, 24, 31), pdm_layers=2,
    prompt_len=512, gen_len=256, max_ctx=1024,
)

D2560_N8 = ModelConfig(
    name="dense_bf16_L32_d2560_n8_ctx2048",
    n_layers=32, d_model=2560, n_q_heads=32, n_kv_heads=8, head_dim=80, d_ffn=9728,
    vocab=151936, dtype="bf16", n_stages=8, anchors=(0, 8, 16, 24, 31), pdm_layers=4,
    prompt_len=1792, gen_len=256, max_ctx=2112, temperatures=(1.0, 0.0),
)

D4096_N8 = ModelConfig(
    name="dense_bf16_L36_d4096_n8_ctx4096",
    n_layers=36, d_model=4096, n_q_heads=32, n_kv_heads=8, head_dim=128, d_ffn=12288,
    vocab=151936, dtype="bf16", n_stages=8, anchors=(0, 9, 18, 27, 36), pdm_layers=4,
    prompt_len=3840, gen_len=256, max_ctx=4160, temperatures=(0.0, 1.0),
)

HYBRID_N16 = ModelConfig(
    name="hybrid_bf16_L32_d2560_n16_ctx8192",
    n_layers=32, d_model=2560, n_q_heads=32, n_kv_heads=8, head_dim=80, d_ffn=9728,
    vocab=151936, dtype="bf16", n_stages=16, anchors=(0, 8, 16, 24, 31), pdm_layers=2,
    prompt_len=7936, gen_len=256, max_ctx=8256, layer_kind=hybrid_kinds(32),
)

WORKLOADS = [TINY, D2560_N4, D2560_N8, D4096_N8, HYBRID_N16]

# ---- small cases the oracle finishes in seconds --------------------------
# They span several GEMV tiles, several attention splits and ragged tails
# (vocab and FFN widths that are not multiples of any tile), uneven stages,
# Ls > L/n, and both attention kinds.

MID_BF16 = ModelConfig(
    name="mid_bf16_L6_d384_n3",
    n_layers=6, d_model=384, n_q_heads=6, n_kv_heads=2, head_dim=64, d_ffn=1064,
    vocab=3001, dtype="bf16", n_stages=3, anchors=(0, 2, 4, 6), pdm_layers=2,
    prompt_len=300, gen_len=24, max_ctx=352,
)

MID_UNEVEN = ModelConfig(
    name="mid_bf16_L7_d256_n3_uneven",
    n_layers=7, d_model=256, n_q_heads=4, n_kv_heads=1, head_dim=64, d_ffn=712,
    vocab=2053, dtype="bf16", n_stages=3, anchors=(0, 3, 5, 7), pdm_layers=3,
    prompt_len=45, gen_len=20, max_ctx=96,
)

MID_F32_N1 = ModelConfig(
    name="mid_f32_L4_d128_n1",
    n_layers=4, d_model=128, n_q_heads=4, n_kv_heads=2, head_dim=32, d_ffn=344,
    vocab=1031, dtype="f32", n_stages=1, anchors=(0, 2, 4), pdm_layers=1,
    prompt_len=17, gen_len=16, max_ctx=48,
)

MID_HYBRID = ModelConfig(
    name="mid_hybrid_bf16_L8_d256_n4",
    n_layers=8, d_model=256, n_q_heads=4, n_kv_heads=2, head_dim=64, d_ffn=704,
    vocab=2003, dtype="bf16", n_stages=4, anchors=(0, 2, 4, 8), pdm_layers=2,
    prompt_len=70, gen_len=20, max_ctx=128, layer_kind=hybrid_kinds(8),
)

MID_D128 = ModelConfig(
    name="mid_bf16_L4_d512_hd128_n4",
    n_layers=4, d_model=512, n_q_heads=4, n_kv_heads=1, head_dim=128, d_ffn=1408,
    vocab=4099, dtype="bf16", n_stages=4, anchors=(0, 1, 2, 4), pdm_layers=1,
    prompt_len=130, gen_len=20, max_ctx=192,
)

SMALL_CASES = [MID_BF16, MID_UNEVEN, MID_F32_N1, MID_HYBRID, MID_D128]

BY_NAME = {c.name: c for c in WORKLOADS + SMALL_CASES}
ALIASES = {"tiny": TINY, "cfg1": TINY, "cfg2": D2560_N4, "cfg3": D2560_N8,
           "cfg4": D4096_N8, "cfg5": HYBRID_N16}


def get(name: str) -> ModelConfig:
    if name in ALIASES:
        return ALIASES[name]
    return BY_NAME[name]


def tensor_names(cfg: ModelConfig) -> List[str]:
    """Names of every weight tensor of a workload, in a stable order."""
    names = ["embed", "lm_head", "final_norm"]
    for l in range(cfg.n_layers):
        names += [f"layers.{l}.{t}" for t in LAYER_TENSORS]
    names.append("pdm.proj")
    for r in range(cfg.pdm_layers):
        names += [f"pdm.layers.{r}.{t}" for t in LAYER_TENSORS]
    names.append("pdm.final_norm")
    return names


LAYER_TENSORS = ("attn_norm", "w_qkv", "w_o", "ffn_norm", "w_gate", "w_up", "w_down")


def tensor_shape(cfg: ModelConfig, name: str) -> Tuple[int, ...]:
    d, V, F = cfg.d_model, cfg.vocab, cfg.d_ffn
    if name in ("embed", "lm_head"):
        return (V, d)
    if name in ("final_norm", "pdm.final_norm"):
        return (d,)
    if name == "pdm.proj":
        return (d, len(cfg.anchors) * d)
    parts = name.split(".")
    t = parts[-1]
    linear = parts[0] == "layers" and cfg.kinds[int(parts[1])] == LINEAR
    qo = cfg.n_q_heads * cfg.head_dim
    if t in ("attn_norm", "ffn_norm"):
        return (d,)
    if t == "w_qkv":
        return (cfg.lin_qkv_rows() if linear else cfg.qkv_rows, d)
    if t == "w_o":
        return (d, qo)
    if t in ("w_gate", "w_up"):
        return (F, d)
    if t == "w_down":
        return (d, F)
    raise KeyError(name)
