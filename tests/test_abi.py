"""The C-ABI library loads and exports every function include/spd.h declares (no GPU needed).

Only error paths that return before any HIP call are exercised here.
"""
import ctypes
import os
import re

import pytest

from spd_inputs import get, SMALL_CASES, WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "spd.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = set(re.findall(r"\b(spd_[a-z_]+)\s*\(", src))
    return sorted(names)


def _lib():
    from speculative_pipeline_decoding_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        from speculative_pipeline_decoding_amd.build import build
        build()
    return binding, binding.load()


def test_every_declared_symbol_is_exported():
    binding, L = _lib()
    declared = _declared()
    assert len(declared) >= 14
    for name in declared:
        assert hasattr(L, name), name
    assert set(declared) <= set(binding.SYMBOLS)


def test_workspace_bytes_and_config_errors():
    binding, L = _lib()
    for cfg in WORKLOADS + SMALL_CASES:
        c, keep = binding.make_config(cfg)
        nb = L.spd_workspace_bytes(ctypes.byref(c))
        if any(cfg.kinds):
            continue
        assert nb > 0, cfg.name
    cfg = get("tiny")
    for bad in (dict(anchors=(1, 2, 4)), dict(anchors=(0, 3, 2)), dict(anchors=(0, 2, 5)),
                dict(n=5), dict(Ls=0)):
        c, keep = binding.make_config(cfg, **bad)
        assert L.spd_workspace_bytes(ctypes.byref(c)) == 0, bad


def test_init_rejects_bad_arguments_without_a_gpu():
    binding, L = _lib()
    cfg = get("tiny")
    c, keep = binding.make_config(cfg)
    w = binding.Weights()
    s = binding.Sampling()
    s.top_p = 1.0
    h = ctypes.c_void_p()
    nb = L.spd_workspace_bytes(ctypes.byref(c))
    # null workspace
    assert L.spd_init(ctypes.byref(c), ctypes.byref(w), ctypes.byref(s), None, nb, None,
                      ctypes.byref(h)) == binding.SPD_E_ARG
    fake = ctypes.c_void_p(0x1000)
    # workspace too small
    assert L.spd_init(ctypes.byref(c), ctypes.byref(w), ctypes.byref(s), fake, nb - 1, None,
                      ctypes.byref(h)) == binding.SPD_E_CAPACITY
    assert b"workspace" in L.spd_init_error()
    # top_p must be > 0 (and not NaN)
    for bad in (0.0, -0.5, float("nan")):
        s.top_p = bad
        assert L.spd_init(ctypes.byref(c), ctypes.byref(w), ctypes.byref(s), fake, nb, None,
                          ctypes.byref(h)) == binding.SPD_E_ARG
        assert b"top_p" in L.spd_init_error()
    s.top_p = 1.0
    # forced mode needs T = 0
    s.temperature, s.forced_mode = 1.0, 1
    assert L.spd_init(ctypes.byref(c), ctypes.byref(w), ctypes.byref(s), fake, nb, None,
                      ctypes.byref(h)) == binding.SPD_E_CONFIG
    s.temperature, s.forced_mode = 0.0, 0
    # null weights
    assert L.spd_init(ctypes.byref(c), ctypes.byref(w), ctypes.byref(s), fake, nb, None,
                      ctypes.byref(h)) == binding.SPD_E_ARG
    assert not h.value


def test_null_handle_calls():
    binding, L = _lib()
    assert L.spd_step(None) == binding.SPD_E_ARG
    assert L.spd_verify_commit(None, None) == binding.SPD_E_ARG
    assert L.spd_prefill(None, None, 0, None) == binding.SPD_E_ARG
    L.spd_destroy(None)
