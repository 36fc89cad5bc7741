"""ctypes binding of libspd.so (include/spd.h): argument marshalling only.

Every step of the hot path runs in the HIP library. PyTorch only provides
device memory (weights, workspace) and the HIP stream. If the library is not
built, importing this module raises: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, List, Optional, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libspd.so")

SPD_OK, SPD_E_ARG, SPD_E_CONFIG, SPD_E_STATE, SPD_E_CAPACITY, SPD_E_DEVICE = 0, -1, -2, -3, -4, -5
SPD_F32, SPD_BF16 = 0, 1
SPD_FILL_CLAMP, SPD_FILL_ZERO = 0, 1
SPD_KV_AUTO, SPD_KV_F32 = 0, 1
DBG = {"target_logits": 1, "draft_logits": 2, "h_ring": 3, "anchors": 4, "pdm_rows": 5,
       "target_kv": 6, "pdm_kv": 7, "tokens": 8, "top_p": 9}
# launch kinds reported by spd_timing_read
OP_NAMES = ["embed", "gemv_proj", "gemv_qkv", "attention", "linear", "gemv_o", "gemv_gate_up",
            "gemv_down", "gemv_head", "vocab", "finalize", "residual", "pdm_qkv", "pdm_attention",
            "pdm_o", "pdm_gate_up", "pdm_down", "nucleus", "gather"]
TENSORS = ("attn_norm", "w_qkv", "w_o", "ffn_norm", "w_gate", "w_up", "w_down")


class SpdError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"spd error {code}: {msg}")
        self.code = code


class ModelConfig(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("d_model", ctypes.c_int32),
                ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("d_ffn", ctypes.c_int32), ("vocab", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("rope_theta", ctypes.c_float), ("rms_eps", ctypes.c_float),
                ("layer_kind", ctypes.POINTER(ctypes.c_uint8)), ("n_stages", ctypes.c_int32),
                ("stage_layers", ctypes.POINTER(ctypes.c_int32)), ("n_anchors", ctypes.c_int32),
                ("anchors", ctypes.POINTER(ctypes.c_int32)), ("pdm_layers", ctypes.c_int32),
                ("anchor_fill", ctypes.c_int32), ("max_ctx", ctypes.c_int32),
                ("speculate_from", ctypes.c_int32), ("kv_dtype", ctypes.c_int32),
                ("draft_width", ctypes.c_int32)]


class Weights(ctypes.Structure):
    _fields_ = [("embed", ctypes.c_void_p), ("lm_head", ctypes.c_void_p),
                ("final_norm", ctypes.c_void_p), ("layers", ctypes.POINTER(ctypes.c_void_p)),
                ("pdm_proj", ctypes.c_void_p), ("pdm_layers", ctypes.POINTER(ctypes.c_void_p)),
                ("pdm_final_norm", ctypes.c_void_p)]


class Sampling(ctypes.Structure):
    _fields_ = [("temperature", ctypes.c_float), ("top_p", ctypes.c_float),
                ("seed", ctypes.c_uint64), ("forced_mode", ctypes.c_int32),
                ("forced_p", ctypes.c_float), ("forced_ref", ctypes.POINTER(ctypes.c_int32)),
                ("forced_ref_len", ctypes.c_int32)]


class Commit(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("verified", "position", "token", "accepted",
                                              "draft_token", "flags", "committed_total",
                                              "inflight", "new_draft", "newest",
                                              "accepted_index")]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


class Stats(ctypes.Structure):
    _fields_ = [("K", ctypes.c_int64), ("N", ctypes.c_int64), ("accepted", ctypes.c_int64),
                ("rejected", ctypes.c_int64), ("alpha", ctypes.c_double), ("s0", ctypes.c_double)]


SYMBOLS = ["spd_workspace_bytes", "spd_init", "spd_init_error", "spd_prefill", "spd_step",
           "spd_verify_commit", "spd_get_stats", "spd_get_kv_lens", "spd_debug_size",
           "spd_debug_copy", "spd_reset", "spd_last_error", "spd_destroy", "spd_lookahead",
           "spd_timing_enable",
           "spd_timing_read", "spd_timing_read_layers", "spd_balance_stages",
           "spd_prefill_static_scratch"]

_lib = None


def load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m speculative_pipeline_decoding_amd.build` (no fallback exists)")
    # One HIP runtime per process: torch ships its own libamdhip64.so.7, and libspd.so needs a
    # library of that name. Loaded first, libspd.so would pull in the system copy, and torch
    # imported later would bind to it instead of its own (its GPU ops then crash). Importing
    # torch first makes libspd.so use torch's copy.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    L = ctypes.CDLL(LIB_PATH)
    P, I, VP = ctypes.POINTER, ctypes.c_int, ctypes.c_void_p
    L.spd_workspace_bytes.argtypes = [P(ModelConfig)]
    L.spd_workspace_bytes.restype = ctypes.c_size_t
    L.spd_init.argtypes = [P(ModelConfig), P(Weights), P(Sampling), VP, ctypes.c_size_t, VP, P(VP)]
    L.spd_init_error.restype = ctypes.c_char_p
    L.spd_prefill.argtypes = [VP, P(ctypes.c_int32), ctypes.c_int32, P(ctypes.c_int32)]
    L.spd_prefill_static_scratch.argtypes = [VP, P(ctypes.c_int32), ctypes.c_int32,
                                             P(ctypes.c_int32)]
    L.spd_step.argtypes = [VP]
    L.spd_verify_commit.argtypes = [VP, P(Commit)]
    L.spd_get_stats.argtypes = [VP, P(Stats)]
    L.spd_get_kv_lens.argtypes = [VP, P(ctypes.c_int32), P(ctypes.c_int32)]
    L.spd_debug_size.argtypes = [VP, ctypes.c_int32]
    L.spd_debug_size.restype = ctypes.c_size_t
    L.spd_debug_copy.argtypes = [VP, ctypes.c_int32, VP, ctypes.c_size_t]
    L.spd_reset.argtypes = [VP]
    L.spd_last_error.argtypes = [VP]
    L.spd_last_error.restype = ctypes.c_char_p
    L.spd_destroy.argtypes = [VP]
    L.spd_destroy.restype = None
    L.spd_lookahead.argtypes = [VP, I]
    L.spd_lookahead.restype = I
    L.spd_timing_enable.argtypes = [VP, I]
    L.spd_timing_read.argtypes = [VP, ctypes.c_int32, P(ctypes.c_int64), P(ctypes.c_double),
                                  P(ctypes.c_double)]
    L.spd_timing_read_layers.argtypes = [VP, P(ctypes.c_double), P(ctypes.c_int64)]
    L.spd_balance_stages.argtypes = [ctypes.c_int32, P(ctypes.c_float), ctypes.c_int32,
                                     P(ctypes.c_int32)]
    for name in ("spd_init", "spd_prefill", "spd_step", "spd_verify_commit", "spd_get_stats",
                 "spd_get_kv_lens", "spd_debug_copy", "spd_reset", "spd_timing_enable",
                 "spd_timing_read", "spd_timing_read_layers", "spd_balance_stages"):
        getattr(L, name).restype = I
    _lib = L
    return L


def balance_stages(layer_cost: Sequence[float], n: int) -> List[int]:
    """Stage sizes from per-layer costs (spd_balance_stages); host only."""
    L = load()
    cost = np.ascontiguousarray(layer_cost, dtype=np.float32)
    out = (ctypes.c_int32 * n)()
    rc = L.spd_balance_stages(cost.size, cost.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), n, out)
    if rc != SPD_OK:
        raise SpdError(rc, "spd_balance_stages: bad arguments")
    return list(out)


def _i32(vals) -> ctypes.Array:
    vals = [int(v) for v in vals]
    return (ctypes.c_int32 * max(1, len(vals)))(*vals)


def make_config(cfg, n: Optional[int] = None, anchors: Optional[Sequence[int]] = None,
                Ls: Optional[int] = None, fill: str = "clamp", speculate_from: str = "input",
                draft_width: Optional[int] = None):
    """spd_model_config from a workload description; returns (struct, keep-alive list)."""
    n = cfg.n_stages if n is None else n
    anchors = list(cfg.anchors if anchors is None else anchors)
    Ls = cfg.pdm_layers if Ls is None else Ls
    keep = []
    c = ModelConfig()
    c.n_layers, c.d_model = cfg.n_layers, cfg.d_model
    c.n_q_heads, c.n_kv_heads, c.head_dim = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    c.d_ffn, c.vocab = cfg.d_ffn, cfg.vocab
    c.dtype = SPD_BF16 if cfg.dtype == "bf16" else SPD_F32
    c.rope_theta, c.rms_eps = cfg.rope_theta, cfg.rms_eps
    kinds = (ctypes.c_uint8 * cfg.n_layers)(*cfg.kinds)
    keep.append(kinds)
    c.layer_kind = ctypes.cast(kinds, ctypes.POINTER(ctypes.c_uint8))
    c.n_stages = n
    if cfg.stage_layers and n == cfg.n_stages:
        sl = _i32(cfg.stage_layers)
        keep.append(sl)
        c.stage_layers = ctypes.cast(sl, ctypes.POINTER(ctypes.c_int32))
    a = _i32(anchors)
    keep.append(a)
    c.n_anchors = len(anchors)
    c.anchors = ctypes.cast(a, ctypes.POINTER(ctypes.c_int32))
    c.pdm_layers = Ls
    c.anchor_fill = SPD_FILL_ZERO if fill == "zero" else SPD_FILL_CLAMP
    c.max_ctx = cfg.max_ctx
    c.speculate_from = {"input": 0, "output": 1}[speculate_from]
    c.kv_dtype = {"auto": SPD_KV_AUTO, "f32": SPD_KV_F32}[getattr(cfg, "kv_dtype", "auto")]
    c.draft_width = getattr(cfg, "draft_width", 1) if draft_width is None else draft_width
    return c, keep


def upload_weights(cfg, arrays: Dict[str, np.ndarray], device="cuda"):
    """Copy generated numpy tensors to device tensors (bf16 bit patterns become torch.bfloat16)."""
    import torch
    out = {}
    for name, a in arrays.items():
        if a.dtype == np.uint16:
            t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
        else:
            t = torch.from_numpy(np.ascontiguousarray(a))
        out[name] = t.to(device)
    return out


class SPD:
    """One decoding session on one sequence: spd_init / spd_prefill / spd_step / spd_verify_commit."""

    def __init__(self, cfg, weights, temperature: float = 0.0, top_p: float = 1.0, seed: int = 0,
                 forced_p: Optional[float] = None, forced_ref: Optional[Sequence[int]] = None,
                 n: Optional[int] = None, anchors: Optional[Sequence[int]] = None,
                 Ls: Optional[int] = None, fill: str = "clamp", stream=None,
                 speculate_from: str = "input", draft_width: Optional[int] = None):
        import torch
        self.L = load()
        self.cfg = cfg
        self._keep = []
        self.c, keep = make_config(cfg, n, anchors, Ls, fill, speculate_from, draft_width)
        self.W = self.c.draft_width
        self._keep += keep
        self.n = self.c.n_stages
        self.Ls = self.c.pdm_layers
        self.weights = weights
        ptr = lambda name: ctypes.c_void_p(weights[name].data_ptr())
        lay = (ctypes.c_void_p * (7 * cfg.n_layers))(
            *[weights[f"layers.{l}.{t}"].data_ptr() for l in range(cfg.n_layers) for t in TENSORS])
        pl = (ctypes.c_void_p * (7 * self.Ls))(
            *[weights[f"pdm.layers.{r}.{t}"].data_ptr() for r in range(self.Ls) for t in TENSORS])
        self._keep += [lay, pl]
        w = Weights()
        w.embed, w.lm_head, w.final_norm = ptr("embed").value, ptr("lm_head").value, ptr("final_norm").value
        w.layers = ctypes.cast(lay, ctypes.POINTER(ctypes.c_void_p))
        w.pdm_proj = ptr("pdm.proj").value
        w.pdm_layers = ctypes.cast(pl, ctypes.POINTER(ctypes.c_void_p))
        w.pdm_final_norm = ptr("pdm.final_norm").value
        s = Sampling()
        s.temperature, s.top_p, s.seed = temperature, top_p, seed
        if forced_p is not None:
            ref = _i32(forced_ref)
            self._keep.append(ref)
            s.forced_mode, s.forced_p = 1, forced_p
            s.forced_ref = ctypes.cast(ref, ctypes.POINTER(ctypes.c_int32))
            s.forced_ref_len = len(forced_ref)
        nbytes = self.L.spd_workspace_bytes(ctypes.byref(self.c))
        if nbytes == 0:
            raise SpdError(SPD_E_CONFIG, "invalid configuration")
        dev = weights["embed"].device
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        self.stream = stream if stream is not None else torch.cuda.current_stream(dev)
        h = ctypes.c_void_p()
        rc = self.L.spd_init(ctypes.byref(self.c), ctypes.byref(w), ctypes.byref(s),
                             ctypes.c_void_p(self.workspace.data_ptr()), nbytes,
                             ctypes.c_void_p(self.stream.cuda_stream), ctypes.byref(h))
        if rc != SPD_OK:
            raise SpdError(rc, self.L.spd_init_error().decode())
        self.h = h

    def _chk(self, rc):
        if rc != SPD_OK:
            raise SpdError(rc, self.L.spd_last_error(self.h).decode())

    def prefill(self, prompt) -> int:
        arr = _i32(prompt)
        first = ctypes.c_int32()
        self._chk(self.L.spd_prefill(self.h, arr, len(prompt), ctypes.byref(first)))
        return first.value

    def prefill_static_scratch(self, prompt) -> int:
        """spd_prefill with its chunk buffers in the library's static device array."""
        arr = _i32(prompt)
        first = ctypes.c_int32()
        self._chk(self.L.spd_prefill_static_scratch(self.h, arr, len(prompt), ctypes.byref(first)))
        return first.value

    def step(self) -> None:
        self._chk(self.L.spd_step(self.h))

    def verify_commit(self) -> Commit:
        c = Commit()
        self._chk(self.L.spd_verify_commit(self.h, ctypes.byref(c)))
        return c

    def stats(self) -> Stats:
        s = Stats()
        self._chk(self.L.spd_get_stats(self.h, ctypes.byref(s)))
        return s

    def kv_lens(self):
        per = (ctypes.c_int32 * self.cfg.n_layers)()
        pl = ctypes.c_int32()
        self._chk(self.L.spd_get_kv_lens(self.h, per, ctypes.byref(pl)))
        return list(per), pl.value

    def debug(self, what: str) -> np.ndarray:
        code = DBG[what]
        nb = self.L.spd_debug_size(self.h, code)
        if what in ("target_kv", "pdm_kv"):
            kv16 = self.cfg.dtype == "bf16" and getattr(self.cfg, "kv_dtype", "auto") == "auto"
            dt = np.uint16 if kv16 else np.float32
        elif what == "tokens":
            dt = np.int32
        elif what == "top_p":
            dt = np.dtype([("zb", np.float32), ("id_cut", np.int32), ("lse", np.float32),
                           ("pad", np.int32)])
        else:
            dt = np.float32
        out = np.empty(nb // np.dtype(dt).itemsize, dtype=dt)
        self._chk(self.L.spd_debug_copy(self.h, code, out.ctypes.data, nb))
        return out

    def reset(self):
        self._chk(self.L.spd_reset(self.h))

    def lookahead(self, on: bool = True):
        """Enqueue the step after a refill step together with it (spd_lookahead)."""
        self._chk(self.L.spd_lookahead(self.h, 1 if on else 0))

    def timing(self, on, serial: bool = False):
        """Per-launch timing on or off; serial also puts the PDM chain on the caller's stream."""
        self._chk(self.L.spd_timing_enable(self.h, (2 if serial else 1) if on else 0))

    def timing_read(self):
        out = {}
        for k, name in enumerate(OP_NAMES):
            c, ms, b = ctypes.c_int64(), ctypes.c_double(), ctypes.c_double()
            self._chk(self.L.spd_timing_read(self.h, k, ctypes.byref(c), ctypes.byref(ms), ctypes.byref(b)))
            out[name] = {"count": c.value, "ms": ms.value, "bytes": b.value}
        return out

    def timing_read_layers(self):
        """Per target layer: (total kernel ms, single-token passes)."""
        ms = (ctypes.c_double * self.cfg.n_layers)()
        passes = (ctypes.c_int64 * self.cfg.n_layers)()
        self._chk(self.L.spd_timing_read_layers(self.h, ms, passes))
        return np.array(ms[:]), np.array(passes[:])

    def close(self):
        if getattr(self, "h", None):
            self.L.spd_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def generate(self, prompt, G: int):
        """prefill, then (step, verify_commit) until G tokens (first included) are committed."""
        toks = [self.prefill(prompt)]
        recs = []
        while len(toks) < G:
            self.step()
            c = self.verify_commit()
            recs.append(c.as_dict())
            if c.verified:
                toks.append(c.token)
        return toks, recs
