"""Stage planning (test infrastructure: the oracle; only tests, smoke() and bench.py's CPU
baseline use this package).

Non-uniform stage partitioning, which the pith.science review of the paper names among
the deployment ideas of its Appendix C.1 (not evaluated there), with the compute
imbalance of mixed attention layers that its Section 6 admits. Reading taken: a plan is
a split of the layers, in order, into n contiguous stages of at least one layer; a
stage's cost is the sum of its layers' costs (float32 values, added in float64 from the
stage's first layer upward); the plan minimises the largest stage cost, then maximises
the smallest, and then lets each stage in turn take as many layers as it can (equal
costs give numpy.array_split's sizes).
"""
from __future__ import annotations

from bisect import bisect_left
from functools import lru_cache
from typing import List, Sequence

import numpy as np


def _costs(layer_cost: Sequence[float]) -> List[float]:
    return [float(x) for x in np.asarray(layer_cost, dtype=np.float32)]


def stage_cost(c: Sequence[float], i: int, j: int) -> float:
    """Cost of layers i .. j-1, added from layer i upward."""
    s = 0.0
    for l in range(i, j):
        s += c[l]
    return s


def balance_stages(layer_cost: Sequence[float], n: int) -> List[int]:
    c = _costs(layer_cost)
    L = len(c)
    if not 1 <= n <= L:
        raise ValueError("need 1 <= n <= number of layers")

    def splittable(A: float, B: float):
        @lru_cache(maxsize=None)
        def ok(i: int, k: int) -> bool:
            """Layers i.. split into exactly k stages, each costing within [A, B]."""
            if k == 0:
                return i == L
            return any(A <= stage_cost(c, i, j) <= B and ok(j, k - 1)
                       for j in range(i + 1, L - k + 2))
        return ok

    # both bounds of an optimal plan are the cost of some run of layers
    cands = sorted({stage_cost(c, i, j) for i in range(L) for j in range(i + 1, L + 1)})
    # smallest feasible largest cost (feasibility grows with B)
    b = bisect_left(range(len(cands)), True, key=lambda t: splittable(0.0, cands[t])(0, n))
    B = cands[b]
    # largest feasible smallest cost, given B (feasibility shrinks as A grows)
    a = bisect_left(range(len(cands)), True, key=lambda t: not splittable(cands[t], B)(0, n)) - 1
    A = cands[a]
    ok = splittable(A, B)
    sizes, i = [], 0
    for st in range(n):
        rest = n - st - 1
        j = max(j for j in range(i + 1, L - rest + 1)
                if A <= stage_cost(c, i, j) <= B and ok(j, rest))
        sizes.append(j - i)
        i = j
    return sizes
