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
    # forced_ref ids must lie in [0, V): checked before any device call
    fake_layers = (ctypes.c_void_p * (7 * cfg.n_layers))(*([0x1000] * (7 * cfg.n_layers)))
    fake_pdm = (ctypes.c_void_p * (7 * cfg.pdm_layers))(*([0x1000] * (7 * cfg.pdm_layers)))
    wf = binding.Weights(0x1000, 0x1000, 0x1000, fake_layers, 0x1000, fake_pdm, 0x1000)
    for bad in (-1, cfg.vocab, 1 << 30):
        ref = (ctypes.c_int32 * 4)(1, 2, bad, 3)
        sf = binding.Sampling(0.0, 1.0, 0, 1, 0.5, ref, 4)
        assert L.spd_init(ctypes.byref(c), ctypes.byref(wf), ctypes.byref(sf), fake, nb, None,
                          ctypes.byref(h)) == binding.SPD_E_ARG
        assert b"forced_ref" in L.spd_init_error()
    # null weights
    assert L.spd_init(ctypes.byref(c), ctypes.byref(w), ctypes.byref(s), fake, nb, None,
                      ctypes.byref(h)) == binding.SPD_E_ARG
    assert not h.value


def test_draft_width_limits():
    binding, L = _lib()
    cfg = get("tiny")
    for w in (0, 1, 2, 4):
        c, keep = binding.make_config(cfg, draft_width=w)
        assert L.spd_workspace_bytes(ctypes.byref(c)) > 0, w
    # the side caches and the candidate rows grow the workspace
    c1, k1 = binding.make_config(cfg, draft_width=1)
    c4, k4 = binding.make_config(cfg, draft_width=4)
    assert L.spd_workspace_bytes(ctypes.byref(c4)) > L.spd_workspace_bytes(ctypes.byref(c1))
    for bad in (dict(draft_width=5), dict(draft_width=-1),
                dict(draft_width=2, speculate_from="output")):
        c, keep = binding.make_config(cfg, **bad)
        assert L.spd_workspace_bytes(ctypes.byref(c)) == 0, bad
    c, keep = binding.make_config(get("mid_hybrid_bf16_L8_d256_n4"), draft_width=2)
    assert L.spd_workspace_bytes(ctypes.byref(c)) == 0     # linear layers
    # top_p < 1 and forced mode are refused with W > 1, before any device call
    c, keep = binding.make_config(cfg, draft_width=2)
    nb = L.spd_workspace_bytes(ctypes.byref(c))
    fake = ctypes.c_void_p(0x1000)
    h = ctypes.c_void_p()
    w = binding.Weights()
    for s in (binding.Sampling(1.0, 0.9, 0, 0, 0.0, None, 0),
              binding.Sampling(0.0, 1.0, 0, 1, 0.5, None, 0)):
        assert L.spd_init(ctypes.byref(c), ctypes.byref(w), ctypes.byref(s), fake, nb, None,
                          ctypes.byref(h)) == binding.SPD_E_CONFIG
        assert b"draft" in L.spd_init_error()


def test_null_handle_calls():
    binding, L = _lib()
    assert L.spd_step(None) == binding.SPD_E_ARG
    assert L.spd_verify_commit(None, None) == binding.SPD_E_ARG
    assert L.spd_prefill(None, None, 0, None) == binding.SPD_E_ARG
    assert L.spd_prefill_static_scratch(None, None, 0, None) == binding.SPD_E_ARG
    assert L.spd_lookahead(None, 1) == binding.SPD_E_ARG
    assert L.spd_reset(None) == binding.SPD_E_ARG
    L.spd_destroy(None)


def test_stage_planner_matches_the_oracle_bit_for_bit():
    """spd_balance_stages is host code: it runs here. Same sizes as the oracle's planner."""
    import numpy as np
    from oracle.plan import balance_stages as oracle_plan
    binding, L = _lib()
    rng = np.random.default_rng(17)
    cases = [([1.0] * 36, 8), ([1.0] * 32, 16), ([3, 1, 1, 1, 2, 2, 1, 1], 4)]
    # the hybrid's pattern (three linear layers, then one softmax layer) at two costs
    cases += [([1.1, 1.1, 1.1, 1.0] * 8, n) for n in (4, 8, 16)]
    for _ in range(60):
        Ln = int(rng.integers(1, 40))
        n = int(rng.integers(1, min(Ln, 16) + 1))
        costs = rng.choice([rng.uniform(0.5, 1.5, Ln), rng.integers(0, 5, Ln).astype(float)])
        cases.append((list(costs), n))
    for costs, n in cases:
        assert binding.balance_stages(costs, n) == oracle_plan(costs, n), (costs, n)


def test_stage_planner_rejects_bad_arguments():
    binding, L = _lib()
    for costs, n in [([1.0, 2.0], 3), ([1.0, 2.0], 0), ([1.0, float("nan")], 1),
                     ([1.0, -1.0], 1), ([1.0, float("inf")], 2)]:
        with pytest.raises(binding.SpdError):
            binding.balance_stages(costs, n)


def test_explicit_stage_splits():
    binding, L = _lib()
    import dataclasses
    base = get("mid_hybrid_bf16_L8_d256_n4")
    for ok in [(2, 3, 1, 2), (3, 2, 2, 1), (1, 1, 1, 5)]:
        c, keep = binding.make_config(dataclasses.replace(base, stage_layers=ok))
        assert L.spd_workspace_bytes(ctypes.byref(c)) > 0, ok
    for bad in [(2, 3, 1, 1), (0, 4, 2, 2), (2, 2, 2, 3)]:
        c, keep = binding.make_config(dataclasses.replace(base, stage_layers=bad))
        assert L.spd_workspace_bytes(ctypes.byref(c)) == 0, bad


def test_binding_loads_torch_before_the_library():
    """libspd.so must bind to the HIP runtime torch already loaded (one per process)."""
    import subprocess
    import sys
    code = ("import sys; sys.path.insert(0, %r)\n"
            "from speculative_pipeline_decoding_amd import binding\n"
            "binding.load()\n"
            "assert 'torch' in sys.modules\n") % ROOT
    subprocess.run([sys.executable, "-c", code], check=True, timeout=300)
