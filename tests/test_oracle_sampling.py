"""Pins for the sampling rules and the counter-based RNG.

Rejection sampling must reproduce the target distribution exactly (Leviathan
et al. 2023, the paper's section 3.5 assumption on the pith.science review
page); Gumbel-max must draw from softmax; SplitMix64 must reproduce its
published output sequence.
"""
import numpy as np
import pytest
from scipy import stats

from oracle import sampling as S


def test_splitmix64_published_sequence():
    # Seed 0 output sequence of the SplitMix64 reference generator (Vigna's splitmix64.c,
    # Steele, Lea & Flood 2014).
    want = [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F, 0xF88BB8A8724C81EC]
    assert [int(x) for x in S.splitmix64_sequence(0, 4)] == want


def test_uniform_exact_in_float32_and_open_interval():
    u = S.uniform(123, S.STREAM_DRAFT, 77, np.arange(200000))
    assert u.min() > 0.0 and u.max() < 1.0
    np.testing.assert_array_equal(u.astype(np.float32).astype(np.float64), u)
    assert abs(u.mean() - 0.5) < 3e-3
    # different streams / positions / seeds give different draws
    assert not np.array_equal(u[:100], S.uniform(123, S.STREAM_RES, 77, np.arange(100)))
    assert not np.array_equal(u[:100], S.uniform(123, S.STREAM_DRAFT, 78, np.arange(100)))
    assert not np.array_equal(u[:100], S.uniform(124, S.STREAM_DRAFT, 77, np.arange(100)))
    # a pure function of its counter
    np.testing.assert_array_equal(S.uniform(123, S.STREAM_DRAFT, 77, [5, 9]), u[[5, 9]])


def test_top_p_closed_cases():
    p = np.array([0.1, 0.4, 0.2, 0.3])
    assert S.nucleus(p, 0.5).tolist() == [False, True, False, True]
    assert S.nucleus(p, 0.4).tolist() == [False, True, False, False]    # reaches exactly
    assert S.nucleus(p, 0.95).tolist() == [True, True, True, True]
    assert S.nucleus(p, 1.0).all()
    ties = np.full(4, 0.25)
    assert S.nucleus(ties, 0.5).tolist() == [True, True, False, False]  # ties by lower id
    assert S.nucleus(ties, 0.6).tolist() == [True, True, True, False]
    d = S.distribution(np.log(p), 1.0, 0.5)
    np.testing.assert_allclose(d, [0, 0.4 / 0.7, 0, 0.3 / 0.7])


def _rand_dist(rng, V, zeros=0):
    w = rng.gamma(0.5, size=V)
    if zeros:
        w[rng.choice(V, zeros, replace=False)] = 0.0
    return w / w.sum()


@pytest.mark.parametrize("V", [2, 3, 5, 8])
def test_rejection_sampling_exact_enumeration(V):
    """sum_d q(d) a(d) [d = x] + (1 - sum_d q(d) a(d)) r(x) == p(x) for every x."""
    rng = np.random.default_rng(V)
    cases = []
    for _ in range(30):
        cases.append((_rand_dist(rng, V), _rand_dist(rng, V)))
    cases.append((_rand_dist(rng, V, zeros=V // 2), _rand_dist(rng, V)))
    cases.append((_rand_dist(rng, V), _rand_dist(rng, V, zeros=V // 2)))
    same = _rand_dist(rng, V)
    cases.append((same, same.copy()))
    for p, q in cases:
        a = S.accept_probability(p, q)
        acc = q * a
        out = acc + (1.0 - acc.sum()) * S.residual_distribution(p, q)
        np.testing.assert_allclose(out, p, rtol=0, atol=1e-12)


def test_gumbel_max_draws_from_its_weights():
    w = np.array([0.05, 0.4, 0.0, 0.25, 0.3])
    n = 40000
    draws = np.array([S.gumbel_max(w, 9, S.STREAM_DRAFT, pos)[0] for pos in range(n)])
    assert not np.any(draws == 2)
    counts = np.bincount(draws, minlength=5)
    keep = w > 0
    chi = stats.chisquare(counts[keep], n * w[keep])
    assert chi.pvalue > 1e-3


def test_rejection_sampling_monte_carlo_through_verify():
    """Draft with select_draft, verify with verify(): committed tokens are distributed as p."""
    rng = np.random.default_rng(11)
    V = 6
    z_t = rng.standard_normal(V) * 1.5
    z_q = rng.standard_normal(V) * 1.5
    s = S.Sampling(temperature=1.0, seed=5)
    p = S.distribution(z_t, 1.0, 1.0)
    n = 30000
    out = np.empty(n, dtype=np.int64)
    acc = 0
    for pos in range(n):
        d, q, _ = S.select_draft(z_q, s, pos)
        y, a, _ = S.verify(z_t, d, q, s, pos)
        out[pos] = y
        acc += a
    chi = stats.chisquare(np.bincount(out, minlength=V), n * p)
    assert chi.pvalue > 1e-3
    q = S.distribution(z_q, 1.0, 1.0)
    # acceptance rate is sum_x min(p, q)
    assert abs(acc / n - np.minimum(p, q).sum()) < 4 * np.sqrt(0.25 / n)


def test_rejection_sampling_monte_carlo_with_top_p():
    rng = np.random.default_rng(12)
    V = 7
    z_t = rng.standard_normal(V) * 2
    z_q = rng.standard_normal(V) * 2
    s = S.Sampling(temperature=0.8, top_p=0.7, seed=6)
    p = S.distribution(z_t, 0.8, 0.7)
    n = 30000
    out = np.array([S.verify(z_t, *S.select_draft(z_q, s, pos)[:2], s, pos)[0] for pos in range(n)])
    counts = np.bincount(out, minlength=V)
    assert counts[p == 0].sum() == 0
    chi = stats.chisquare(counts[p > 0], n * p[p > 0])
    assert chi.pvalue > 1e-3


def test_greedy_verify_and_ties():
    z = np.array([0.5, 2.0, 2.0, -1.0])
    y, acc, flag = S.verify(z, 2, None, S.Sampling(), 10)
    assert y == 1 and not acc and flag        # tie -> lowest id, flagged as near-tie
    y, acc, flag = S.verify(np.array([0.0, 3.0, 1.0]), 1, None, S.Sampling(), 10)
    assert y == 1 and acc and not flag


def test_forced_mode_replaces_the_draft():
    ref = np.array([7, 3, 9, 1] * 50)
    s = S.Sampling(seed=2, forced_p=0.6, forced_ref=ref, forced_base=100)
    z = np.zeros(16)
    hits = 0
    for x in range(100, 300):
        d, _, _ = S.select_draft(z, s, x)
        r = ref[x - 100]
        assert d in (r, (r + 1) % 16)
        hits += d == r
    assert 0.45 < hits / 200 < 0.75


def test_top_p_envelope_closed_case():
    # p = [0.4, 0.3, 0.2, 0.1]: masses ahead 0, 0.4, 0.7, 0.9; at top_p = 0.7 the third
    # token sits exactly on the edge, so with no logit slack it alone is undecided
    z = np.log(np.array([0.4, 0.3, 0.2, 0.1]))
    certain, band = S.nucleus_bounds(z, 1.0, 0.7, 0.0)
    assert certain.tolist() == [True, True, False, False]
    assert band.tolist() == [False, False, True, False]
    certain, band = S.nucleus_bounds(z, 1.0, 0.6, 0.0)
    assert certain.tolist() == [True, True, False, False] and not band.any()
    certain, band = S.nucleus_bounds(z, 1.0, 1.0, 0.3)
    assert certain.all() and not band.any()


def _perturbed(rng, z, slack):
    # mostly the envelope's corners, where a wrong bound shows first
    if rng.random() < 0.7:
        return z + slack * rng.choice([-1.0, 1.0], z.size)
    return z + rng.uniform(-slack, slack, z.size)


@pytest.mark.parametrize("top_p", [0.3, 0.8, 0.95])
def test_top_p_envelope_holds_under_logit_perturbation(top_p):
    """Brute force: for logits moved by at most the slack, the exact top-p set and the
    renormalised probabilities stay inside nucleus_bounds / prob_range."""
    rng = np.random.default_rng(21)
    T, slack = 0.7, 2e-3
    for trial in range(200):
        V = int(rng.integers(2, 60))
        z = rng.standard_normal(V) * rng.choice([0.05, 0.5, 2.0])
        if trial % 7 == 0:
            z[: V // 2] = z[0]                      # ties
        certain, band = S.nucleus_bounds(z, T, top_p, slack)
        lo, hi = S.prob_range(z, T, top_p, slack)
        for _ in range(5):
            z2 = _perturbed(rng, z, slack)
            keep = S.nucleus(S.softmax_t(z2, T), top_p)
            assert np.all(keep[certain]) and not np.any(keep & ~(certain | band))
            q = S.distribution(z2, T, top_p)
            assert np.all(q >= lo * (1 - 1e-12)) and np.all(q <= hi * (1 + 1e-12))


def test_top_p_unflagged_decisions_survive_logit_perturbation():
    """Brute force: a sampled draw, an accept test or a residual draw that the oracle does
    not flag comes out the same from every logit vector within the slack."""
    rng = np.random.default_rng(5)
    T, slack = 1.0, 2e-2
    seen = {"flag": 0, "clean": 0, "reject": 0}
    for pos in range(1500):
        V = int(rng.integers(3, 12))
        s = S.Sampling(temperature=T, top_p=float(rng.choice([0.5, 0.9])), seed=9,
                       logit_slack=slack)
        z_t = rng.standard_normal(V) * 0.8
        z_q = z_t + rng.standard_normal(V) * 0.5
        d, q, dflag = S.select_draft(z_q, s, pos)
        y, acc, vflag = S.verify(z_t, d, q, s, pos, z_q)
        seen["flag"] += int(dflag or vflag)
        if dflag or vflag:
            continue
        seen["clean"] += 1
        seen["reject"] += int(not acc)
        for _ in range(8):
            zt2, zq2 = _perturbed(rng, z_t, slack), _perturbed(rng, z_q, slack)
            d2, q2, _ = S.select_draft(zq2, s, pos)
            assert d2 == d
            y2, acc2, _ = S.verify(zt2, d2, q2, s, pos, zq2)
            assert (y2, acc2) == (y, acc)
    assert seen["clean"] > 500 and seen["reject"] > 100 and seen["flag"] > 0


def test_rejection_with_an_empty_residual_commits_the_target_argmax():
    """Degenerate rejection: q >= p everywhere (here q = 1.5 p, so the accept test
    u q(d) < p(d) fails for u >= 2/3 and max(0, p - q) is all zero). No residual token
    exists, so the commit falls back to the target's argmax, flagged as a near-tie."""
    z = np.array([0.3, 1.7, -0.4, 1.1, 0.2])
    s = S.Sampling(temperature=1.0, seed=5)
    p = S.distribution(z, 1.0, 1.0)
    q = 1.5 * p
    seen = 0
    for v in range(200):
        y, acc, flag = S.verify(z, 3, q, s, v)
        u = S.uniform(5, S.STREAM_ACC, v, 0)[()]
        assert acc == (u * q[3] < p[3])
        if not acc:
            assert (y, flag) == (1, True)
            seen += 1
    assert seen > 0
