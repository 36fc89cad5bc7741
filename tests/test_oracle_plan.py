"""Pins for the stage planner (non-uniform stage partitioning, the pith.science review's
remarks on Appendix C.1): exhaustive search over every split on small layer counts, and
the closed case of equal costs."""
import itertools

import numpy as np
import pytest

from oracle.plan import _costs, balance_stages, stage_cost


def brute_force(costs, n):
    """Every split of L layers into n contiguous non-empty stages; keep the one with the
    smallest largest cost, then the largest smallest cost, then the largest sizes in order."""
    c = _costs(costs)
    L = len(c)
    best = None
    for cuts in itertools.combinations(range(1, L), n - 1):
        bounds = (0,) + cuts + (L,)
        sizes = [bounds[k + 1] - bounds[k] for k in range(n)]
        sc = [stage_cost(c, bounds[k], bounds[k + 1]) for k in range(n)]
        key = (max(sc), -min(sc), [-x for x in sizes])
        if best is None or key < best[0]:
            best = (key, sizes)
    return best[1]


def test_equal_costs_give_the_default_split():
    for L, n in [(36, 8), (32, 16), (7, 3), (5, 5), (9, 1)]:
        want = [len(a) for a in np.array_split(np.arange(L), n)]
        assert balance_stages([1.0] * L, n) == want


def test_closed_case():
    # costs 3 1 1 1 | 2 2 1 1, n = 4: no plan keeps every stage <= 3, the best keeps them
    # within [2, 4], and the first stage can take 2 layers ([3, 1]) without breaking that
    assert balance_stages([3, 1, 1, 1, 2, 2, 1, 1], 4) == [2, 3, 1, 2]
    assert brute_force([3, 1, 1, 1, 2, 2, 1, 1], 4) == [2, 3, 1, 2]


@pytest.mark.parametrize("seed", range(6))
def test_matches_exhaustive_search(seed):
    rng = np.random.default_rng(seed)
    for _ in range(40):
        L = int(rng.integers(1, 10))
        n = int(rng.integers(1, L + 1))
        kind = rng.integers(0, 3)
        if kind == 0:
            costs = rng.integers(0, 4, L).astype(float)          # small integers: many ties
        elif kind == 1:
            costs = rng.uniform(0.5, 1.5, L)
        else:
            costs = rng.choice([1.0, 1.1], L)                     # two layer kinds
        assert balance_stages(costs, n) == brute_force(costs, n), (costs, n)


def test_rejects_bad_stage_counts():
    with pytest.raises(ValueError):
        balance_stages([1.0, 2.0], 3)
    with pytest.raises(ValueError):
        balance_stages([1.0, 2.0], 0)
