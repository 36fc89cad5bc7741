"""Draft selection, verification and the counter-based RNG.

Verification follows the pages: greedy match at temperature 0 (lossless),
and at T > 0 rejection sampling as in Leviathan et al. 2023, which the paper
inherits to keep the target distribution (pith.science review, "Assumptions",
section 3.5 entry). For a draft d ~ q and target distribution p:
    accept d iff u * q(d) < p(d),  u ~ U(0,1)          (so P(accept) = min(1, p/q))
    else  y ~ r,  r(x) = max(0, p(x) - q(x)) / sum_x max(0, p(x) - q(x)).
Sampling from a distribution is done by the Gumbel-max rule:
    argmax_i (log w_i + G_i),  G_i = -log(-log u_i),
which draws i with probability w_i / sum(w) (Gumbel 1954; Maddison et al. 2014).

Readings (the pages are silent):
  * argmax ties go to the lowest token id;
  * top-p: sort by probability (ties: lower id first), keep the shortest prefix
    whose sum reaches top_p, including the token that crosses; top_p >= 1 keeps all;
  * the RNG is counter based, so every draw is a pure function of
    (seed, stream, position, index): u = ((x >> 41) + 0.5) * 2^-23 with
    x = mix(mix(mix(seed) ^ (stream << 32 | pos)) + index * 0x9E3779B97F4A7C15),
    where mix is the SplitMix64 output function (Steele, Lea & Flood 2014);
  * forced mode (acceptance sweep): the draft at position x becomes the
    reference greedy token r[x] when u_FORCE(x) < p_force, else (r[x] + 1) mod V.

Draft trees of width W (the review's "Assumptions & free parameters" lists W = 1 and 4; a
reading, since the pages describe no mechanism): the PDM proposes W distinct candidates
for a position, best first. At T = 0 they are the W largest logits (ties: lower id first);
at T > 0 the W largest Gumbel-perturbed scores log q_i + G_i, which draws W tokens from q
without replacement (Gumbel-top-k: Kool, van Hoof & Welling 2019); W = 1 is the plain
draft. Verification tests them in rank order (recursive rejection sampling, Jeon et al.
2024): round i proposes c_i from q_i, q renormalised without c_0 .. c_{i-1}, against the
target r_i (r_0 = p); accept iff u_i q_i(c_i) < r_i(c_i), else
r_{i+1} = max(0, r_i - q_i) / sum(max(0, r_i - q_i)). Each round is one speculative
sampling step whose proposal is, given the earlier rounds, distributed as q_i and
independent of u_i, so by induction the committed token is distributed as p. If every
candidate is rejected, y ~ r_W. At T = 0 the committed token is argmax p, accepted when it
is a candidate.

Near-ties at top_p < 1. Another implementation computes the same decisions from
logits that differ from these by at most Sampling.logit_slack (delta) each, and
sums masses with a relative rounding of at most TOP_P_EPS. Every probability it
sees is then within a factor exp(+-2 delta / T) of ours, so a token's mass ahead
(the sum over the tokens before it in the nucleus order) lies in a known interval,
and so does the renormalised probability of every token (prob_range). A decision
is flagged whenever some logits inside that envelope would change it: a sampled
token whose win is not certain over every token that may be in the set, a verified
draft whose accept test can go either way, a residual winner that may be overtaken.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Tuple

import numpy as np

GOLDEN = 0x9E3779B97F4A7C15
MASK64 = 0xFFFFFFFFFFFFFFFF

STREAM_DRAFT = 1
STREAM_ACC = 2
STREAM_RES = 3
STREAM_FORCE = 4
STREAM_FIRST = 5

NEAR_TIE = 1e-3
TOP_P_EPS = 1e-6


def mix64(z) -> np.ndarray:
    """SplitMix64 output function on uint64 values (wrapping arithmetic)."""
    z = np.asarray(z, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
        return z ^ (z >> np.uint64(31))


def splitmix64_sequence(seed: int, count: int) -> np.ndarray:
    """The SplitMix64 generator itself: state += golden; output mix(state)."""
    with np.errstate(over="ignore"):
        states = (np.uint64(seed) + np.uint64(GOLDEN) * np.arange(1, count + 1, dtype=np.uint64))
    return mix64(states)


def uniform(seed: int, stream: int, pos: int, idx) -> np.ndarray:
    """u(seed, stream, pos, idx) in (0, 1); exact in float32 and float64."""
    idx = np.asarray(idx, dtype=np.uint64)
    k0 = mix64(np.uint64(seed & MASK64))
    key = np.uint64(((stream & 0xFFFFFFFF) << 32) | (pos & 0xFFFFFFFF))
    k1 = mix64(k0 ^ key)
    with np.errstate(over="ignore"):
        x = mix64(k1 + idx * np.uint64(GOLDEN))
    return ((x >> np.uint64(41)).astype(np.float64) + 0.5) * 2.0 ** -23


def gumbel(u: np.ndarray) -> np.ndarray:
    return -np.log(-np.log(u))


def top2_gap(scores: np.ndarray) -> float:
    finite = scores[np.isfinite(scores)]
    if finite.size < 2:
        return np.inf
    top = np.partition(finite, -2)[-2:]
    return float(top[1] - top[0])


def argmax_lowest(scores: np.ndarray) -> int:
    return int(np.argmax(scores))          # numpy returns the first (lowest) index


def nucleus(p: np.ndarray, top_p: float) -> np.ndarray:
    """Boolean mask of the top-p nucleus of distribution p."""
    if top_p >= 1.0:
        return np.ones(p.shape, dtype=bool)
    ids = np.arange(p.size)
    order = np.lexsort((ids, -p))
    cum = np.cumsum(p[order])
    r = int(np.searchsorted(cum, top_p, side="left"))
    r = min(r, p.size - 1)
    keep = np.zeros(p.shape, dtype=bool)
    keep[order[: r + 1]] = True
    return keep


def softmax_t(z: np.ndarray, T: float) -> np.ndarray:
    """softmax(z / T) over the whole vocabulary."""
    p = np.exp(z / T - np.max(z / T))
    return p / p.sum()


def nucleus_bounds(z: np.ndarray, T: float, top_p: float, slack: float):
    """(certain, band): tokens inside the top-p set for every logit vector within `slack`
    of z, and tokens that are inside for some and outside for others."""
    V = z.size
    if top_p >= 1.0:
        return np.ones(V, dtype=bool), np.zeros(V, dtype=bool)
    p0 = softmax_t(z, T)
    f = np.exp(2.0 * slack / T)
    order = np.argsort(-z, kind="stable")
    cum = np.concatenate([[0.0], np.cumsum(p0[order])])
    neg = -z[order]                                    # ascending
    n_above = np.searchsorted(neg, -(z + 2.0 * slack), side="left")   # z_j > z_i + 2 slack
    n_atleast = np.searchsorted(neg, -(z - 2.0 * slack), side="right")  # z_j >= z_i - 2 slack
    ahead_lo = cum[n_above] / f
    ahead_hi = (cum[n_atleast] - p0) * f
    certain = ahead_hi < top_p * (1.0 - TOP_P_EPS)
    out = ahead_lo >= top_p * (1.0 + TOP_P_EPS)
    return certain, ~certain & ~out


def prob_range(z: np.ndarray, T: float, top_p: float, slack: float):
    """Per-token [lo, hi] of the renormalised top-p probability over the same envelope."""
    p0 = softmax_t(z, T)
    certain, band = nucleus_bounds(z, T, top_p, slack)
    f = np.exp(2.0 * slack / T)
    m_lo = p0[certain].sum() / f
    m_hi = p0[certain | band].sum() * f
    lo = np.where(certain, p0 / (f * m_hi), 0.0)
    with np.errstate(divide="ignore"):
        hi = np.where(certain | band, p0 * f / m_lo, 0.0)   # inf when no token is certain
    return lo, hi


def _uncertain_winner(lo_score: np.ndarray, hi_score: np.ndarray, y: int) -> bool:
    """y wins for sure iff its lowest score beats every other token's highest by NEAR_TIE."""
    if lo_score[y] == -np.inf:
        return True
    others = np.delete(hi_score, y)
    best = others.max() if others.size else -np.inf
    return not (lo_score[y] - best >= NEAR_TIE)


def top_p_gumbel_flag(z: np.ndarray, s: "Sampling", stream: int, pos: int, y: int) -> bool:
    """Near-tie flag of a Gumbel-max draw over the top-p set (top_p < 1)."""
    certain, band = nucleus_bounds(z, s.temperature, s.top_p, s.slack())
    sc = z / s.temperature + gumbel(uniform(s.seed, stream, pos, np.arange(z.size)))
    e = s.slack() / s.temperature
    lo = np.where(certain, sc - e, -np.inf)
    hi = np.where(certain | band, sc + e, -np.inf)
    return _uncertain_winner(lo, hi, y)


def distribution(z: np.ndarray, T: float, top_p: float) -> np.ndarray:
    """softmax(z / T) restricted to its top-p nucleus and renormalised."""
    p = np.exp(z / T - np.max(z / T))
    p = p / p.sum()
    keep = nucleus(p, top_p)
    p = np.where(keep, p, 0.0)
    return p / p.sum()


def gumbel_max(w: np.ndarray, seed: int, stream: int, pos: int) -> Tuple[int, bool]:
    """Sample i ~ w / sum(w) by Gumbel-max; returns (i, near-tie flag)."""
    G = gumbel(uniform(seed, stream, pos, np.arange(w.size)))
    with np.errstate(divide="ignore"):
        s = np.where(w > 0, np.log(w) + G, -np.inf)
    return argmax_lowest(s), top2_gap(s) < NEAR_TIE


@dataclass
class Sampling:
    temperature: float = 0.0
    top_p: float = 1.0
    seed: int = 0
    forced_p: Optional[float] = None       # forced mode when not None (T = 0 only)
    forced_ref: Optional[np.ndarray] = None  # reference tokens for positions P0, P0+1, ...
    forced_base: int = 0                   # position of forced_ref[0]
    logit_slack: Optional[float] = None    # top_p < 1 near-ties: logit error allowed to
                                           # the compared implementation (None: 1e-4)

    def slack(self) -> float:
        return 1e-4 if self.logit_slack is None else float(self.logit_slack)


def first_token(z: np.ndarray, s: Sampling, pos: int) -> Tuple[int, bool]:
    if s.temperature == 0.0:
        return argmax_lowest(z), top2_gap(z) < NEAR_TIE
    y, flag = gumbel_max(distribution(z, s.temperature, s.top_p), s.seed, STREAM_FIRST, pos)
    if s.top_p < 1.0:
        flag = flag or top_p_gumbel_flag(z, s, STREAM_FIRST, pos, y)
    return y, flag


def select_draft(z_q: np.ndarray, s: Sampling, pos: int):
    """The PDM's draft for position pos: (d, q or None, near-tie flag)."""
    V = z_q.size
    if s.temperature == 0.0:
        d, flag, q = argmax_lowest(z_q), top2_gap(z_q) < NEAR_TIE, None
    else:
        q = distribution(z_q, s.temperature, s.top_p)
        d, flag = gumbel_max(q, s.seed, STREAM_DRAFT, pos)
        if s.top_p < 1.0:
            flag = flag or top_p_gumbel_flag(z_q, s, STREAM_DRAFT, pos, d)
    if s.forced_p is not None and s.forced_ref is not None:
        j = pos - s.forced_base
        if 0 <= j < len(s.forced_ref):
            ref = int(s.forced_ref[j])
            # p_force crosses the C boundary as a float32; u is exact in both types.
            hit = uniform(s.seed, STREAM_FORCE, pos, 0)[()] < float(np.float32(s.forced_p))
            d, flag = (ref if hit else (ref + 1) % V), False
    return int(d), q, bool(flag)


def verify(z_t: np.ndarray, d: int, q: Optional[np.ndarray], s: Sampling, v: int,
           z_q: Optional[np.ndarray] = None):
    """Verify draft d at position v against target logits z_t.

    z_q: the draft logits q was computed from (for the top_p < 1 near-tie flags).
    Returns (y, accepted, near-tie flag): y is the committed token.
    """
    if s.temperature == 0.0:
        y = argmax_lowest(z_t)
        return y, y == d, top2_gap(z_t) < NEAR_TIE
    p = distribution(z_t, s.temperature, s.top_p)
    u = uniform(s.seed, STREAM_ACC, v, 0)[()]
    lhs, rhs = u * q[d], p[d]
    flag = abs(lhs - rhs) < NEAR_TIE * q[d]
    top_p_ranges = s.top_p < 1.0 and z_q is not None
    if top_p_ranges:
        pl, ph = prob_range(z_t, s.temperature, s.top_p, s.slack())
        ql, qh = prob_range(z_q, s.temperature, s.top_p, s.slack())
        sure_accept = u * qh[d] < pl[d]
        sure_reject = u * ql[d] >= ph[d]
        flag = flag or not (sure_accept or sure_reject)
    if lhs < rhs:
        return int(d), True, bool(flag)
    r = np.maximum(p - q, 0.0)
    if not (r > 0).any():
        # p <= q everywhere in floating point (the two agree to rounding), so the residual
        # has no mass to sample from: commit the target's argmax, flagged as a near-tie
        return argmax_lowest(z_t), False, True
    y, rflag = gumbel_max(r, s.seed, STREAM_RES, v)
    if top_p_ranges and not rflag:
        G = gumbel(uniform(s.seed, STREAM_RES, v, np.arange(p.size)))
        with np.errstate(divide="ignore"):
            lo = np.log(np.maximum(pl - qh, 0.0)) + G
            hi = np.log(np.maximum(ph - ql, 0.0)) + G
        rflag = _uncertain_winner(lo, hi, y)
    return int(y), False, bool(flag or rflag)


def accept_probability(p: np.ndarray, q: np.ndarray) -> np.ndarray:
    """P(accept | draft x) = min(1, p(x)/q(x)) for x with q(x) > 0."""
    with np.errstate(divide="ignore", invalid="ignore"):
        return np.where(q > 0, np.minimum(1.0, p / np.where(q > 0, q, 1.0)), 0.0)


def residual_distribution(p: np.ndarray, q: np.ndarray) -> np.ndarray:
    r = np.maximum(p - q, 0.0)
    tot = r.sum()
    return r / tot if tot > 0 else r


def select_drafts(z_q: np.ndarray, s: Sampling, pos: int, W: int):
    """The PDM's W candidates for position pos, best first: (candidates, q or None, flag).
    W = 1 is select_draft. Otherwise (top_p >= 1, no forced mode): the W largest logits at
    T = 0, the W largest log q_i + G_i at T > 0 (lower id first on ties); flag marks a gap
    below NEAR_TIE between two of the W + 1 largest scores, whose order decides the
    candidates and their ranks."""
    if W == 1:
        d, q, flag = select_draft(z_q, s, pos)
        return [d], q, flag
    assert s.forced_p is None and s.top_p >= 1.0
    V = z_q.size
    if s.temperature == 0.0:
        q, sc = None, z_q
    else:
        q = distribution(z_q, s.temperature, s.top_p)
        G = gumbel(uniform(s.seed, STREAM_DRAFT, pos, np.arange(V)))
        with np.errstate(divide="ignore"):
            sc = np.where(q > 0, np.log(q) + G, -np.inf)
    order = np.lexsort((np.arange(V), -sc))        # descending score, lower id first
    top = order[: W + 1]
    vals = sc[top]
    flag = any(vals[j] - vals[j + 1] < NEAR_TIE for j in range(len(top) - 1))
    return [int(t) for t in top[:W]], q, bool(flag)


def tree_rounds(p: np.ndarray, q: np.ndarray, cands):
    """The rounds of recursive rejection sampling of candidates cands (best first) against
    target p with draft distribution q, without any randomness: per round i the pair
    (q_i(c_i), r_i(c_i)), so that c_i is accepted iff u_i q_i(c_i) < r_i(c_i), and the
    unnormalised residual max(0, r_{W-1} - q_{W-1}) that y is drawn from when every round
    rejects. Stops early (residual None) if a residual has no mass in floating point."""
    r, left, rounds = p, q.copy(), []
    res = None
    for i, c in enumerate(cands):
        qi = q if i == 0 else left / left.sum()
        rounds.append((qi[c], r[c]))
        res = np.maximum(r - qi, 0.0)
        if not (res > 0).any():
            return rounds, None
        r = res / res.sum()
        left[c] = 0.0
    return rounds, res


def verify_tree(z_t: np.ndarray, cands, q: Optional[np.ndarray], s: Sampling, v: int):
    """Verify the candidates for position v (best first) against target logits z_t.
    Returns (y, index of the accepted candidate or -1, near-tie flag)."""
    if len(cands) == 1:
        y, acc, flag = verify(z_t, cands[0], q, s, v)
        return y, (0 if acc else -1), flag
    assert s.top_p >= 1.0
    if s.temperature == 0.0:
        y = argmax_lowest(z_t)
        return y, (cands.index(y) if y in cands else -1), top2_gap(z_t) < NEAR_TIE
    p = distribution(z_t, s.temperature, s.top_p)
    rounds, res = tree_rounds(p, q, cands)
    flag = False
    for i, (qc, rc) in enumerate(rounds):
        u = uniform(s.seed, STREAM_ACC, v, i)[()]
        flag = flag or abs(u * qc - rc) < NEAR_TIE * qc
        if u * qc < rc:
            return int(cands[i]), i, bool(flag)
    if res is None:
        # a residual without mass (see verify): the target's argmax, flagged
        return argmax_lowest(z_t), -1, True
    y, rflag = gumbel_max(res, s.seed, STREAM_RES, v)
    return int(y), -1, bool(flag or rflag)
