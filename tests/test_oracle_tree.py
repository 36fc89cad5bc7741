"""Pins for the oracle's draft tree of width W (W candidates per draft position).

* lossless at T = 0 for W = 2, 3, 4: the committed stream is the target's greedy stream,
  on workloads where siblings do get accepted (and adopted);
* verification preserves the target distribution: exact enumeration on tiny vocabularies
  of every ordered candidate tuple drawn without replacement (the Plackett-Luce
  probabilities of sampling without replacement) through the oracle's own rounds
  (sampling.tree_rounds) gives P(y = x) = p(x) to 1e-12; a Monte-Carlo run through the
  real select_drafts and verify_tree passes a chi-square test, and the candidates'
  ordered tuples follow the Plackett-Luce law;
* a sibling's hidden states equal those of a causal forward of the sequence in which it
  is the token at its position (it attends over its ancestors and itself, nothing else);
* the PDM pin of tests/test_oracle_pdm.py holds with W > 1 (adoptions change tokens and
  KV rows, and the drafts must still equal the independent route's);
* the step count: K = N + (n - 1)(1 + R''), R'' the verifications before the last step that
  restart the pipeline (a rejection, or a verification of the step's own drafts).
"""
import itertools

import numpy as np
import pytest
from scipy import stats

import reference_torch as ref
from conftest import workload
from oracle import sampling as S
from oracle.spd import SPD, ar_decode, spd_run
from test_oracle_pdm import check_pdm


@pytest.mark.parametrize("name,Ws", [("tiny", (2, 3, 4)), ("mid_bf16_L7_d256_n3_uneven", (2, 4)),
                                     ("mid_bf16_L6_d384_n3", (3,))])
def test_tree_lossless_at_temperature_zero(name, Ws):
    cfg, W, prompt = workload(name)
    G = min(cfg.gen_len, 40)
    want = ar_decode(cfg, W, prompt, G=G)
    siblings = 0
    for w in Ws:
        r = spd_run(cfg, W, prompt, G=G, W=w)
        assert r.tokens == want, w
        siblings += sum(1 for rec in r.records if rec.exited and rec.accepted_index > 0)
    if name == "tiny":
        assert siblings > 0      # the adoption path ran


def _plackett_luce(q, c):
    """Probability of drawing the ordered tuple c from q without replacement."""
    pr, left = 1.0, 1.0
    for x in c:
        pr *= q[x] / left
        left -= q[x]
    return pr


@pytest.mark.parametrize("V,Wd", [(3, 2), (5, 2), (5, 3), (8, 3), (8, 4)])
def test_tree_verification_exact_enumeration(V, Wd):
    rng = np.random.default_rng(V * 10 + Wd)
    for trial in range(6):
        p = rng.dirichlet(np.ones(V) * (0.3 if trial % 2 else 2.0))
        q = rng.dirichlet(np.ones(V) * (0.3 if trial % 3 else 2.0))
        if trial == 5:
            q = p.copy()                                   # identical distributions
        dist = np.zeros(V)
        for c in itertools.permutations(range(V), Wd):
            w = _plackett_luce(q, c)
            if w == 0.0:
                continue
            rounds, res = S.tree_rounds(p, q, list(c))
            reach = 1.0
            for i, (qc, rc) in enumerate(rounds):
                a = min(1.0, rc / qc)
                dist[c[i]] += w * reach * a
                reach *= 1.0 - a
            if reach > 0:
                assert res is not None
                dist += w * reach * res / res.sum()
        np.testing.assert_allclose(dist, p, rtol=0, atol=1e-12)


def test_tree_verification_monte_carlo_through_the_real_functions():
    V, Wd, Npos = 6, 3, 60000
    rng = np.random.default_rng(11)
    z_t, z_q = rng.normal(size=V), rng.normal(size=V)
    s = S.Sampling(temperature=1.0, seed=21)
    p = S.softmax_t(z_t, 1.0)
    counts = np.zeros(V)
    tuples = {}
    for v in range(Npos):
        cands, q, _ = S.select_drafts(z_q, s, v, Wd)
        tuples[tuple(cands)] = tuples.get(tuple(cands), 0) + 1
        y, _, _ = S.verify_tree(z_t, cands, q, s, v)
        counts[y] += 1
    assert stats.chisquare(counts, Npos * p).pvalue > 1e-3
    q = S.softmax_t(z_q, 1.0)
    keys = list(itertools.permutations(range(V), Wd))
    obs = np.array([tuples.get(k, 0) for k in keys], dtype=float)
    exp = np.array([_plackett_luce(q, k) for k in keys]) * Npos
    assert stats.chisquare(obs, exp).pvalue > 1e-3


def test_greedy_tree_candidates_are_the_top_logits():
    z = np.array([0.1, 2.0, 2.0, -1.0, 1.5, 0.7])
    cands, q, flag = S.select_drafts(z, S.Sampling(), 0, 3)
    assert cands == [1, 2, 4] and q is None and flag          # the tie 2.0 / 2.0 is flagged
    z = np.array([0.1, 3.0, 2.0, -1.0, 1.0, 0.0])
    assert S.select_drafts(z, S.Sampling(), 0, 3)[0] == [1, 2, 4]
    assert not S.select_drafts(z, S.Sampling(), 0, 3)[2]
    y, idx, _ = S.verify_tree(z, [4, 1, 2], None, S.Sampling(), 0)
    assert (y, idx) == (1, 1)
    y, idx, _ = S.verify_tree(z, [4, 2, 0], None, S.Sampling(), 0)
    assert (y, idx) == (1, -1)


@pytest.mark.parametrize("name,w,T", [("tiny", 4, 0.0), ("tiny", 3, 1.0),
                                      ("mid_bf16_L7_d256_n3_uneven", 2, 1.0)])
def test_sibling_states_equal_a_forward_with_the_sibling_token(name, w, T):
    """After each step, every sibling still in flight (n = 3: the siblings of the newest
    position survive the step's verification) is compared with the reference."""
    cfg, Wt, prompt = workload(name)
    spd = SPD(cfg, Wt, S.Sampling(temperature=T, seed=3), W=w, n=3)
    spd.prefill(prompt)
    checked = 0
    for _ in range(10):
        spd.step()
        for (x, b), hs in spd.sib_h.items():
            toks = [spd.tok[i] for i in range(x)] + [spd.sib[x][b - 1]]
            depth = spd.depth[x]
            Hs = ref.target_depths(cfg, Wt, toks)
            np.testing.assert_allclose(hs, Hs[depth][x].numpy(), rtol=0,
                                       atol=1e-9 * max(1.0, float(np.abs(hs).max())))
            checked += 1
    assert checked > 0


@pytest.mark.parametrize("name,w,seed", [("tiny", 4, 4), ("mid_bf16_L7_d256_n3_uneven", 2, 3)])
def test_pdm_pin_holds_with_draft_trees(name, w, seed):
    class Tree(SPD):
        def __init__(self, *a, **kw):
            super().__init__(*a, W=w, **kw)
    plen = 32 if name == "tiny" else 45
    check_pdm(Tree, name, plen, 14, seed=seed)


@pytest.mark.parametrize("name,w,T", [("tiny", 4, 0.0), ("tiny", 3, 1.0),
                                      ("mid_bf16_L7_d256_n3_uneven", 2, 1.0)])
def test_tree_step_count_identity(name, w, T):
    cfg, Wt, prompt = workload(name)
    G = 30
    r = spd_run(cfg, Wt, prompt, G=G, sampling=S.Sampling(temperature=T, seed=5), W=w)
    n = cfg.n_stages
    ex = [rec for rec in r.records[:-1] if rec.exited]
    restarts = sum(1 for rec in ex if rec.single or not rec.accepted)
    assert r.K == r.N + (n - 1) * (1 + restarts)
    assert 1 + r.N == G
    for rec in r.records:
        kv = rec.kv_len
        assert all(a >= b for a, b in zip(kv, kv[1:]))


def test_tree_residuals_off_the_candidates_are_one_clamp():
    """The rounds' residuals, off the candidates, are one clamp of a linear combination:
    R_i(x) = max(0, A_i p(x) - B_i q(x)) with A_{i+1} = A_i / Z_i, B_{i+1} = B_i / Z_i + s_i
    (A_0 = 1, B_0 = 0, Z_0 = 1, s_0 = 1, s_i = 1 / (1 - E_i), E_i the q-mass of c_0..c_{i-1}),
    because max(0, max(0, a) / Z - b) = max(0, a / Z - b) for b >= 0 and Z > 0. Checked
    against the oracle's own rounds (sampling.tree_rounds) to rounding, so a pass over the
    vocabulary needs two exponentials and a clamp per token."""
    rng = np.random.default_rng(5)
    for trial in range(40):
        V, W = int(rng.integers(6, 40)), int(rng.integers(2, 5))
        p = rng.dirichlet(np.ones(V) * rng.choice([0.2, 1.0, 3.0]))
        q = rng.dirichlet(np.ones(V) * rng.choice([0.2, 1.0, 3.0]))
        cands = [int(c) for c in rng.choice(V, size=W, replace=False)]
        # the oracle's unnormalised residuals R_1 .. R_W, round by round
        r, left, Rs, Zs = p, q.copy(), [], [1.0]
        for i, c in enumerate(cands):
            qi = q if i == 0 else left / left.sum()
            res = np.maximum(r - qi, 0.0)
            Rs.append(res)
            if not (res > 0).any():
                break
            Zs.append(res.sum())
            r = res / res.sum()
            left[c] = 0.0
        off = np.setdiff1d(np.arange(V), cands)
        A, B, E = 1.0, 0.0, 0.0
        for i, R in enumerate(Rs):
            s = 1.0 if i == 0 else 1.0 / (1.0 - E)
            A, B = A / Zs[i], B / Zs[i] + s
            np.testing.assert_allclose(np.maximum(0.0, A * p[off] - B * q[off]), R[off],
                                       rtol=1e-12, atol=1e-15)
            E += q[cands[i]]
