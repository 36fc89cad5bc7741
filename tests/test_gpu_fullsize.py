"""Full-size checks at the real model shapes (MI355X; up to ~90 GB of host memory).

For each of the four large workloads (the n=4 d2560 model with its 512-token prompt, the
n=8 d2560 model the benchmark runs, the n=8 d4096 / head_dim 128 model, and the n=16
hybrid with 24 linear-attention layers):
  * lockstep with the oracle on the model itself: every kernel runs at its benchmark
    launch shape, on a short prompt so that the fp64 oracle finishes in about a minute;
  * at the workload's own context (its full prompt), properties that hold at any size:
      - lossless at T=0: the n-stage stream equals the same model decoded
        autoregressively (the library at n=1), up to the first decision either run
        flags as a near-tie;
      - the scheduler's counting identity K = N + (n-1)(1 + R') and S0 = alpha n at T=1,
        with KV lengths non-increasing over layers after every step;
      - at T=1, top_p=0.875: every top-p set the library reports is the top-p set of its
        own logit row over the full vocabulary (parity.check_top_p_set), and every
        draft lies in its set.
  * lockstep with the oracle at the workload's own prompt (the benchmark's context),
    capped at 8 commits: by default for the n=4 model (T=0, and forced acceptance
    p = 0.7 against the oracle's own greedy stream) and for the benchmark's n=8 model at
    T=1; the other cases (and 32 commits) with SPD_FULL_CONTEXT_LOCKSTEP=1.
One workload's weights are resident at a time (host and device).
"""
import json
import os

import numpy as np
import pytest

import conftest
from conftest import workload
from parity import check_top_p_set, run_parity

pytestmark = pytest.mark.gpu

NAMES = ["dense_bf16_L32_d2560_n4", "dense_bf16_L32_d2560_n8_ctx2048",
         "dense_bf16_L36_d4096_n8_ctx4096", "hybrid_bf16_L32_d2560_n16_ctx8192"]
# full-context lockstep cases that run by default: the fp64 oracle's prefill of the prompt
# and 8 commits take about a minute each on the host
DEFAULT_FULL_CONTEXT = {("dense_bf16_L32_d2560_n4", "T0"), ("dense_bf16_L32_d2560_n4", "forced"),
                        ("dense_bf16_L32_d2560_n8_ctx2048", "T1")}
_state = {}


def deselect(item) -> bool:
    """Cases this module does not run (conftest deselects them at collection): the
    full-context lockstep beyond its defaults (minutes of fp64 oracle work each; set
    SPD_FULL_CONTEXT_LOCKSTEP=1 to run every case), the draft-tree lockstep on any model but
    the benchmark's (the oracle runs every candidate), and draft trees on the hybrid model
    (trees need softmax layers only)."""
    cs = getattr(item, "callspec", None)
    if cs is None or "wl" not in cs.params:
        return False
    name, fn = cs.params["wl"], item.originalname
    if fn == "test_fullsize_lockstep_at_full_context":
        return (os.environ.get("SPD_FULL_CONTEXT_LOCKSTEP") != "1"
                and (name, cs.params["mode"]) not in DEFAULT_FULL_CONTEXT)
    if fn == "test_fullsize_draft_tree_lockstep":
        return name != "dense_bf16_L32_d2560_n8_ctx2048"
    if fn == "test_fullsize_draft_tree_lossless":
        return name.startswith("hybrid")
    return False


@pytest.fixture(scope="module", params=NAMES)
def wl(request):
    """(name, device weights, oracle weights) of one workload; the previous one is dropped."""
    import torch
    from oracle.model import Weights
    from speculative_pipeline_decoding_amd import upload_weights
    name = request.param
    if _state.get("name") != name:
        _state.clear()
        for k in [k for k in conftest._cache if k in NAMES and k != name]:
            del conftest._cache[k]
        torch.cuda.empty_cache()
        cfg, W, _ = workload(name)
        _state.update(name=name, dW=upload_weights(cfg, W), oW=Weights(W, np.float64, cache=True))
    return name, _state["dW"], _state["oW"]


def logit_tolerance(name, T):
    """5e-2 (bf16 bound), or twice the oracle's own fp32-vs-fp64 logit gap on this lockstep
    where that floor is higher (tests/golden/fp32_sensitivity.py: bf16 KV rounding makes a
    deep, wide model's logits sensitive at the fp32 level; no fp32 path can beat the floor)."""
    with open(os.path.join(os.path.dirname(__file__), "golden", "fp32_sensitivity.json")) as f:
        gaps = json.load(f)["gaps"]
    if name not in gaps:
        return 5e-2
    return max(5e-2, 2.0 * gaps[name][f"T{T:g}"])


@pytest.mark.parametrize("T,seed", [(0.0, 0), (1.0, 11)])
def test_fullsize_lockstep_with_oracle(wl, T, seed):
    name, dW, oW = wl
    cfg, W, prompt = workload(name)
    tol = logit_tolerance(name, T)
    print(f"[fullsize] lockstep {name} T={T} logit tolerance {tol:.3g}", flush=True)
    rep = run_parity(cfg, W, dW, prompt[:40], T=T, seed=seed, max_steps=cfg.n_stages + 6,
                     oracle_weights=oW, tol_logits=tol)
    print(f"[fullsize] -> {rep}", flush=True)
    assert rep["steps"] >= cfg.n_stages or rep["stopped_at_near_tie"] is not None


@pytest.mark.parametrize("T,seed", [(0.0, 0), (1.0, 11)])
def test_fullsize_lockstep_fp32_kv(wl, T, seed):
    """The fp32 KV cache option (kv_dtype "f32"): with no bf16 rounding of K and V, the
    library and the oracle (which stores fp32 then too) agree within the fixed 5e-2 logit
    bound on every workload, the d4096 model included."""
    name, dW, oW = wl
    cfg, W, prompt = workload(name)
    cfg = cfg.with_(kv_dtype="f32")
    print(f"[fullsize] lockstep {name} kv f32 T={T}", flush=True)
    rep = run_parity(cfg, W, dW, prompt[:40], T=T, seed=seed, max_steps=cfg.n_stages + 6,
                     oracle_weights=oW, tol_logits=5e-2)
    print(f"[fullsize] -> {rep}", flush=True)
    assert rep["steps"] >= cfg.n_stages or rep["stopped_at_near_tie"] is not None


def _stream(name, dW, n, T, G, seed=0, speculate_from="input", lookahead=False, draft_width=1):
    from speculative_pipeline_decoding_amd import SPD
    cfg, _, prompt = workload(name)
    gpu = SPD(cfg, dW, temperature=T, seed=seed, n=n, speculate_from=speculate_from,
              draft_width=draft_width)
    gpu.lookahead(lookahead)
    toks = [(gpu.prefill(prompt), 0)]
    steps = []
    while len(toks) < G:
        gpu.step()
        c = gpu.verify_commit()
        kv, pl = gpu.kv_lens()
        steps.append((bool(c.verified), bool(c.accepted), kv, pl))
        if c.verified:
            toks.append((c.token, c.flags & 1))
    st = gpu.stats()
    gpu.close()
    return toks, steps, st


def test_fullsize_lossless_matches_autoregressive(wl):
    name, dW, _ = wl
    cfg, _, prompt = workload(name)
    print(f"[fullsize] lossless n={cfg.n_stages} vs n=1 on the {len(prompt)}-token prompt "
          f"of {name}", flush=True)
    # the n-stage run launches each refill step's successor with it (as the benchmark does)
    a, _, _ = _stream(name, dW, cfg.n_stages, 0.0, 32, lookahead=True)
    b, _, sb = _stream(name, dW, 1, 0.0, 32)
    assert sb.N == sb.K and abs(sb.alpha - 1.0) < 1e-12   # n=1: every step commits
    for i, ((ta, fa), (tb, fb)) in enumerate(zip(a, b)):
        if fa or fb:
            print(f"[fullsize] near-tie flagged at commit {i}; compared {i} tokens", flush=True)
            break
        assert ta == tb, f"commit {i}: n={cfg.n_stages} gives {ta}, n=1 gives {tb}"


def test_fullsize_counting_identity_and_kv_invariants(wl):
    name, dW, _ = wl
    cfg, _, _ = workload(name)
    n = cfg.n_stages
    toks, steps, st = _stream(name, dW, n, 1.0, 24, seed=5, lookahead=True)
    rejects = [i for i, (v, acc, _, _) in enumerate(steps) if v and not acc]
    # the run ends on a verification step; a rejection there has no refill inside the run
    r_prime = len(rejects) - (1 if rejects and rejects[-1] == len(steps) - 1 else 0)
    N = sum(1 for v, _, _, _ in steps if v)
    K = len(steps)
    assert K == N + (n - 1) * (1 + r_prime), (K, N, r_prime)
    assert abs(st.s0 - st.alpha * n) < 1e-12 and abs(st.alpha - st.N / st.K) < 1e-12
    for v, acc, kv, pl in steps:
        assert all(x >= y for x, y in zip(kv, kv[1:])), kv   # deeper layers never ahead
        assert pl <= kv[-1]                                   # the PDM keeps exited rows only
        if v and not acc:
            assert len(set(kv)) == 1, kv                      # a reject truncates every layer to v


def test_fullsize_top_p_sets(wl):
    from speculative_pipeline_decoding_amd import SPD
    name, dW, _ = wl
    cfg, _, prompt = workload(name)
    top_p = 0.875
    print(f"[fullsize] top-p sets of {name} at top_p={top_p}", flush=True)
    gpu = SPD(cfg, dW, temperature=1.0, top_p=top_p, seed=13)
    ring = gpu.n + 1
    t0 = gpu.prefill(prompt)
    keep, _ = check_top_p_set(gpu.debug("target_logits"), gpu.debug("top_p")[0], 1.0, top_p,
                              "prefill")
    assert keep[t0]
    sizes = []
    for k in range(2 * cfg.n_stages):
        gpu.step()
        c = gpu.verify_commit()
        cuts = gpu.debug("top_p")
        dpos = c.newest + 1
        keep, _ = check_top_p_set(gpu.debug("draft_logits"), cuts[1 + dpos % ring], 1.0, top_p,
                                  f"step {k} draft")
        assert keep[c.new_draft], f"step {k}: draft {c.new_draft} outside its top-p set"
        sizes.append(int(keep.sum()))
        if c.verified:
            keep, _ = check_top_p_set(gpu.debug("target_logits"), cuts[0], 1.0, top_p,
                                      f"step {k} target")
            assert keep[c.token], f"step {k}: committed {c.token} outside the target's set"
    gpu.close()
    print(f"[fullsize] draft set sizes {sizes[:4]} ... of V={cfg.vocab}", flush=True)


def test_fullsize_output_states_lossless(wl):
    """Output-state speculation at full size: the T=0 stream still equals autoregressive
    decoding (the library at n = 1), and the counting identity holds at T=1."""
    name, dW, _ = wl
    cfg, _, _ = workload(name)
    n = cfg.n_stages
    print(f"[fullsize] output states, {name}", flush=True)
    a, _, _ = _stream(name, dW, n, 0.0, 32, speculate_from="output")
    b, _, _ = _stream(name, dW, 1, 0.0, 32)
    for i, ((ta, fa), (tb, fb)) in enumerate(zip(a, b)):
        if fa or fb:
            print(f"[fullsize] near-tie flagged at commit {i}; compared {i} tokens", flush=True)
            break
        assert ta == tb, f"commit {i}: output states give {ta}, n=1 gives {tb}"
    toks, steps, st = _stream(name, dW, n, 1.0, 16, seed=5, speculate_from="output")
    rejects = [i for i, (v, acc, _, _) in enumerate(steps) if v and not acc]
    r_prime = len(rejects) - (1 if rejects and rejects[-1] == len(steps) - 1 else 0)
    N = sum(1 for v, _, _, _ in steps if v)
    assert len(steps) == N + (n - 1) * (1 + r_prime)
    for v, acc, kv, pl in steps:
        assert all(x >= y for x, y in zip(kv, kv[1:]))
        assert pl <= kv[-1]


@pytest.mark.parametrize("mode", ["T0", "T1", "forced"])
def test_fullsize_lockstep_at_full_context(wl, mode):
    """Lockstep with the oracle at the workload's own prompt (the benchmark's context):
    8 commits for the default cases, 32 with SPD_FULL_CONTEXT_LOCKSTEP=1 (every case), or
    until the first flagged near-tie."""
    from oracle.model import Model
    from oracle.spd import ar_decode
    name, dW, oW = wl
    everything = os.environ.get("SPD_FULL_CONTEXT_LOCKSTEP") == "1"
    cfg, W, prompt = workload(name)
    G = 33 if everything else 9
    T, seed = (1.0, 11) if mode == "T1" else (0.0, 0)
    kw = {}
    if mode == "forced":
        print(f"[fullsize] oracle greedy reference over the {len(prompt)}-token prompt of "
              f"{name}", flush=True)
        ref = ar_decode(cfg, W, prompt, G=G + cfg.n_stages + 2, model=Model(cfg, W, weights=oW))
        kw = dict(forced_p=0.7, forced_ref=ref, seed=5)
    print(f"[fullsize] full-context lockstep {name}: {len(prompt)}-token prompt, {mode}, "
          f"{G - 1} commits", flush=True)
    rep = run_parity(cfg, W, dW, prompt, G=G, T=T, seed=kw.pop("seed", seed), oracle_weights=oW,
                     tol_logits=logit_tolerance(name, T), progress_every=8, **kw)
    print(f"[fullsize] -> { {k: v for k, v in rep.items() if k != 'tokens_match'} }", flush=True)
    assert rep["steps"] > 0
    if rep["stopped_at_near_tie"] is None:
        assert rep["N"] == G - 1
    if mode == "forced" and rep["stopped_at_near_tie"] is None:
        assert rep["rejected"] > 0 and rep["N"] > rep["rejected"]


@pytest.mark.parametrize("T,seed", [(1.0, 1), (1.0, 10)])
def test_fullsize_draft_tree_lockstep(wl, T, seed):
    """Draft trees (W = 4) on the benchmark's n=8 model in lockstep with the oracle: every
    candidate, the accepted rank, the siblings' states and their adoption, at the
    benchmark's launch shapes on a short prompt."""
    name, dW, oW = wl
    cfg, W, prompt = workload(name)
    print(f"[fullsize] draft tree lockstep {name} W=4 T={T}", flush=True)
    rep = run_parity(cfg, W, dW, prompt[:40], T=T, seed=seed, max_steps=cfg.n_stages + 12,
                     oracle_weights=oW, tol_logits=logit_tolerance(name, T), width=4)
    print(f"[fullsize] -> {rep}", flush=True)
    # both seeds reach an accepted sibling (adopted) within these steps in the oracle
    assert rep["stopped_at_near_tie"] is not None or rep["adoptions"] > 0


def test_fullsize_draft_tree_lossless(wl):
    """At T = 0 a draft tree changes only which positions are accepted: the committed
    stream still equals autoregressive decoding (the library at n = 1)."""
    name, dW, _ = wl
    cfg, _, _ = workload(name)
    assert not any(cfg.kinds)
    G = 24
    ref, _, _ = _stream(name, dW, 1, 0.0, G)
    got, steps, st = _stream(name, dW, cfg.n_stages, 0.0, G, draft_width=4)
    for (a, fa), (b, fb) in zip(ref, got):
        if fa or fb:
            break
        assert a == b
    assert st.N == G - 1
