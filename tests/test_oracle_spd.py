"""Pins for the SPD state machine against the pages' invariants and plain AR decoding.

* lossless at T = 0: the committed stream is the target's own greedy stream;
* n = 1 is autoregressive decoding (alpha = 1, S0 = 1);
* Eq. (9): S0 = N / (K (1/n)) = alpha n, with the pages' printed values;
* K = N + (n-1)(1 + R'), and under forced-Bernoulli(p) acceptance
  alpha -> 1 / (1 + (n-1)(1-p)) (renewal argument: after each reseed, n-1
  refill steps, then Geometric(1-p) verifications that each commit one token);
* Eq. (3): at most n positions carry partial-depth features, at the stage starts;
* KV invariants after every step; the anchor clamp rule.
"""
import json
import os

import numpy as np
import pytest

from conftest import workload
from oracle.sampling import Sampling
from oracle.spd import SPD, ar_decode, spd_run, stage_sizes

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_stage_sizes_reading():
    assert stage_sizes(32, 8) == [4] * 8
    assert stage_sizes(36, 8) == [5, 5, 5, 5, 4, 4, 4, 4]
    assert stage_sizes(7, 3) == [3, 2, 2]
    assert stage_sizes(5, 1) == [5]
    assert stage_sizes(6, 3, (1, 2, 3)) == [1, 2, 3]


@pytest.mark.parametrize("name,ns", [("tiny", (1, 2, 3, 4)),
                                     ("mid_bf16_L7_d256_n3_uneven", (2, 3, 7)),
                                     ("mid_hybrid_bf16_L8_d256_n4", (4, 8))])
def test_lossless_at_temperature_zero(name, ns):
    cfg, W, prompt = workload(name)
    G = min(cfg.gen_len, 24)
    ref = ar_decode(cfg, W, prompt, G=G)
    for n in ns:
        r = spd_run(cfg, W, prompt, G=G, n=n)
        assert r.tokens == ref, n
        assert r.N == G - 1


def test_lossless_with_forced_drafts_and_zero_fill():
    cfg, W, prompt = workload("tiny")
    ref = ar_decode(cfg, W, prompt, G=40 + 8)
    for p in (0.0, 0.5, 0.9, 1.0):
        s = Sampling(forced_p=p, forced_ref=np.array(ref), forced_base=cfg.prompt_len, seed=4)
        r = spd_run(cfg, W, prompt, G=40, sampling=s, n=3, fill="zero")
        assert r.tokens == ref[:40]
        if p == 1.0:
            assert r.rejected == 0
        if p == 0.0:
            assert r.accepted == 0


def test_n1_is_autoregressive():
    cfg, W, prompt = workload("tiny")
    r = spd_run(cfg, W, prompt, G=20, n=1)
    assert r.tokens == ar_decode(cfg, W, prompt, G=20)
    assert r.K == r.N == 19 and r.alpha == 1.0 and r.s0 == 1.0
    assert all(rec.exited for rec in r.records)


def test_eq9_printed_values():
    with open(os.path.join(GOLDEN, "eq9_printed_values.json")) as f:
        g = json.load(f)
    cfg, W, _ = workload("tiny")
    for c in g["cases"]:
        spd = SPD(cfg, W, Sampling(), n=2)
        spd.n = c["n"]
        spd.K = 10000
        spd.N = int(round(c["alpha"] * spd.K))
        assert spd.alpha == pytest.approx(c["alpha"], abs=1e-12)
        assert spd.s0 == pytest.approx(c["S0"], abs=1e-9)


def _refills_identity(r, n, G):
    # R' = rejections that are not the last step
    last_is_reject = bool(r.records) and r.records[-1].exited and not r.records[-1].accepted
    R = r.rejected - (1 if last_is_reject else 0)
    assert r.K == r.N + (n - 1) * (1 + R)
    assert 1 + r.N == G
    assert r.s0 == pytest.approx(r.alpha * n)
    assert 0 < r.alpha <= 1.0


@pytest.mark.parametrize("n", [2, 3, 4])
def test_step_count_identity(n):
    cfg, W, prompt = workload("tiny")
    for s in (Sampling(), Sampling(temperature=1.0, seed=1)):
        r = spd_run(cfg, W, prompt, G=30, sampling=s, n=n)
        _refills_identity(r, n, 30)


def test_forced_bernoulli_closed_form():
    """alpha from a long forced run matches 1 / (1 + (n-1)(1-p))."""
    cfg, W, prompt = workload("tiny")
    G = 700
    n, p = 3, 0.7
    ref = ar_decode(cfg.with_(max_ctx=1024), W, prompt, G=G + n + 1)
    s = Sampling(forced_p=p, forced_ref=np.array(ref), forced_base=cfg.prompt_len, seed=8)
    r = spd_run(cfg.with_(max_ctx=1024), W, prompt, G=G, sampling=s, n=n, record_logits=False)
    assert r.tokens == ref[:G]
    want = 1.0 / (1.0 + (n - 1) * (1 - p))
    # cycles ~ G(1-p) = 210; relative sd of alpha ~ 5%
    assert abs(r.alpha - want) < 0.05
    _refills_identity(r, n, G)
    # each verification accepts independently with probability p
    ver = r.accepted + r.rejected
    assert abs(r.accepted / ver - p) < 4 * np.sqrt(p * (1 - p) / ver)


def test_always_reject_gives_alpha_one_over_n():
    cfg, W, prompt = workload("tiny")
    ref = ar_decode(cfg, W, prompt, G=40)
    n = 4
    s = Sampling(forced_p=0.0, forced_ref=np.array(ref), forced_base=cfg.prompt_len)
    r = spd_run(cfg, W, prompt, G=21, sampling=s, n=n)
    # every verification rejects: n steps per commit, except the refill after the last one
    assert r.K == n * r.N
    assert r.s0 == pytest.approx(1.0)


@pytest.mark.parametrize("name,n", [("tiny", 2), ("mid_bf16_L7_d256_n3_uneven", 3),
                                    ("mid_hybrid_bf16_L8_d256_n4", 4)])
def test_staircase_and_kv_invariants(name, n):
    cfg, W, prompt = workload(name)
    P0 = len(prompt)
    s = Sampling(temperature=1.0, seed=3)
    spd = SPD(cfg, W, s, n=n)
    spd.prefill(prompt)
    L = cfg.n_layers
    starts = spd.starts
    N_before = 0
    for _ in range(24):
        F_start = [tuple(f) for f in spd.F]
        rec = spd.step()
        # Eq. (3): positions with depth < L are the in-flight ones, at most n, at stage starts
        partial = [dep for dep in rec.pdm_row_depths if dep < L]
        assert len(partial) <= n
        assert len(partial) == len(F_start)
        assert partial == [starts[st] for _, st in F_start]
        # every PDM row is either final (depth L) or in flight; the newest has depth 0
        assert rec.pdm_row_depths[-1] == 0
        # KV invariants
        kv = rec.kv_len
        assert all(a >= b for a, b in zip(kv, kv[1:]))
        if rec.exited and not rec.accepted:
            assert kv == [rec.verified_pos] * L
            assert rec.inflight == [(rec.verified_pos, 0)]
        assert rec.pdm_len == P0 + N_before
        N_before = spd.N
        pos = [p for p, _ in rec.inflight]
        assert pos == list(range(pos[0], pos[0] + len(pos)))
        assert [st for _, st in rec.inflight] == list(range(len(pos) - 1, -1, -1))
    if n == 1:
        assert len(set(spd.kv_len)) == 1


def test_anchor_clamp_rule():
    cfg, W, prompt = workload("mid_bf16_L6_d384_n3")
    d, k = cfg.d_model, len(cfg.anchors)
    W2 = dict(W)
    deepest = np.zeros((d, k * d), np.float32)
    deepest[:, (k - 1) * d:] = np.eye(d)
    spd = SPD(cfg.with_(dtype="bf16"), W2, Sampling(), n=3)
    spd.m.W._c["pdm.proj"] = deepest.astype(np.float64)
    spd.prefill(prompt[:60])
    for _ in range(6):
        spd.step()
    L = cfg.n_layers
    full = [x for x in spd.anch if spd.depth.get(x, L) == L]
    assert full
    for x in full:                                  # [0 ... 0 | I] picks anchor b = L exactly
        np.testing.assert_array_equal(spd.feature(x), spd.anch[x][k - 1])
    first = np.zeros((d, k * d))
    first[:, :d] = np.eye(d)
    spd.m.W._c["pdm.proj"] = first
    for x in spd.anch:                              # [I | 0 ... 0] picks g0 at any depth
        np.testing.assert_array_equal(spd.feature(x), spd.anch[x][0])
    # a depth-0 row: every slot is g0 under clamp, zeros under zero fill
    newest = spd.F[-1][0]
    spd.step()
    rng = np.random.default_rng(0)
    Wr = rng.standard_normal((d, k * d))
    spd.m.W._c["pdm.proj"] = Wr
    x0 = spd.F[-1][0]
    spd.anch[x0] = {0: rng.standard_normal(d)}
    spd.depth[x0] = 0
    g0 = spd.anch[x0][0]
    np.testing.assert_allclose(spd.feature(x0), Wr @ np.tile(g0, k), rtol=1e-12)
    spd.fill = "zero"
    np.testing.assert_allclose(spd.feature(x0), Wr[:, :d] @ g0, rtol=1e-12)


# ---- output-state speculation (the ablation of the early start) ----------------------

@pytest.mark.parametrize("name,ns", [("tiny", (1, 2, 3, 4)),
                                     ("mid_hybrid_bf16_L8_d256_n4", (4,))])
def test_output_states_lossless_at_temperature_zero(name, ns):
    cfg, W, prompt = workload(name)
    G = min(cfg.gen_len, 24)
    ref = ar_decode(cfg, W, prompt, G=G)
    for n in ns:
        r = spd_run(cfg, W, prompt, G=G, n=n, speculate_from="output")
        assert r.tokens == ref, n


def test_output_states_forced_drafts_and_counting_identity():
    cfg, W, prompt = workload("tiny")
    ref = ar_decode(cfg, W, prompt, G=48)
    for p in (0.0, 0.6, 1.0):
        s = Sampling(forced_p=p, forced_ref=np.array(ref), forced_base=cfg.prompt_len, seed=4)
        r = spd_run(cfg, W, prompt, G=40, sampling=s, n=3, speculate_from="output")
        assert r.tokens == ref[:40]
        _refills_identity(r, 3, 40)
    r = spd_run(cfg, W, prompt, G=30, sampling=Sampling(temperature=1.0, seed=1), n=4,
                speculate_from="output")
    _refills_identity(r, 4, 30)


@pytest.mark.parametrize("name,n", [("tiny", 2), ("mid_bf16_L7_d256_n3_uneven", 3),
                                    ("mid_hybrid_bf16_L8_d256_n4", 4)])
def test_output_states_read_one_stage_deeper(name, n):
    """Every PDM row sits at the depth its token has after the step: the in-flight rows one
    stage deeper than at the step's start, the exiting row at L (permanent at once)."""
    cfg, W, prompt = workload(name)
    P0 = len(prompt)
    spd = SPD(cfg, W, Sampling(temperature=1.0, seed=3), n=n, speculate_from="output")
    spd.prefill(prompt)
    L, starts, sizes = cfg.n_layers, spd.starts, spd.sizes
    for _ in range(24):
        F_start = [tuple(f) for f in spd.F]
        rec = spd.step()
        want = [starts[st] + sizes[st] for _, st in F_start]          # L for the exiting one
        assert rec.pdm_row_depths[-len(want):] == want
        assert all(dep == L for dep in rec.pdm_row_depths[:-len(want)])
        assert rec.pdm_row_depths[-1] == sizes[0]                     # the newest token
        assert rec.pdm_len == P0 + spd.N                               # exited rows are final
        kv = rec.kv_len
        assert all(a >= b for a, b in zip(kv, kv[1:]))
