"""Pins of the brute-force planner oracle (CPU).

The oracle is the planner's definition written out (least total reads over every feasible
kind assignment; "LoopKV: Loop-Aware KV Cache Compression for Serving Looped Transformers",
arXiv:2611.04137, Abstract, sentences on additive damage and on the planner). It is pinned
here by a hand-solved table, closed forms and invariants that a plausible mistake (a dropped
budget, reuse allowed in the final loop, max instead of min) would break.
"""
import math

import numpy as np
import pytest

from oracle import planner_oracle as P

INF = math.inf


def _hand_table():
    # 2 loops x 1 layer. cell 0 (loop 0): 4-bit, 2-bit, reuse; cell 1 (final loop): its reuse
    # entry is very attractive and must never be taken.
    damage = [[0, 3, 2], [0, 4, 0]]
    reads = [[10, 6, 10], [10, 6, 0]]
    storage = [[5, 3, 0], [5, 3, 0]]
    return damage, reads, storage


@pytest.mark.parametrize("D,S,want", [
    # the six plans, solved by hand:
    # (4,4) d0 r20 s10 | (4,2) d4 r16 s8 | (2,4) d3 r16 s8 | (2,2) d7 r12 s6 | (R,4) d2 r20 s5 | (R,2) d6 r16 s3
    (INF, 10 ** 9, ((1, 1), 7, 12, 6)),
    (6, 10 ** 9, ((1, 0), 3, 16, 8)),      # three plans at 16 reads: least damage wins the tie
    (6, 5, ((2, 1), 6, 16, 3)),
    (1, 10 ** 9, ((0, 0), 0, 20, 10)),
    (2, 9, ((2, 0), 2, 20, 5)),
    (0, 9, None),
])
def test_hand_solved_table(D, S, want):
    damage, reads, storage = _hand_table()
    got = P.plan_search_brute(2, 1, damage, reads, storage, D, S)
    assert got == want


def _random_table(rng, n, dyadic=True):
    # dyadic rationals (k / 1024): every sum is exact in float64
    d = rng.integers(0, 4096, size=(n, 3)) / 1024.0
    r = rng.integers(64, 8192, size=(n, 3)) / 1024.0
    s = rng.integers(0, 6, size=(n, 3)).astype(np.int64)
    return d, r, s


@pytest.mark.parametrize("shape", [(1, 3), (2, 3), (3, 2), (4, 2), (2, 5)])
def test_invariants(shape):
    rng = np.random.default_rng(sum(shape))
    L, NL = shape
    n = L * NL
    allowed = P.allowed_kinds(L, NL)
    for trial in range(6):
        d, r, s = _random_table(rng, n)
        # unbounded budgets: each cell at its least-reads allowed kind
        free = P.plan_search_brute(L, NL, d, r, s, INF, 10 ** 9)
        want = sum(min(r[c][k] for k in allowed[c]) for c in range(n))
        assert free[2] == want
        # damage budget below the least reachable damage: no plan
        dmin = sum(min(d[c][k] for k in allowed[c]) for c in range(n))
        if dmin > 0:
            assert P.plan_search_brute(L, NL, d, r, s, dmin - 1 / 1024, 10 ** 9) is None
        # the result is feasible, keeps the final loop off reuse, and loosening budgets
        # never raises the optimum
        prev = None
        for frac in (0.2, 0.4, 0.6, 0.8, 1.0):
            D = frac * float(np.sum(d.max(axis=1)))
            S = int(frac * float(np.sum(s.max(axis=1))))
            got = P.plan_search_brute(L, NL, d, r, s, D, S)
            if got is None:
                assert prev is None
                continue
            kinds, dd, rr, ss = got
            assert dd <= D and ss <= S
            assert all(k in allowed[c] for c, k in enumerate(kinds))
            assert (dd, rr, ss) == P.plan_cost(kinds, d, r, s)
            if prev is not None:
                assert rr <= prev
            prev = rr


def test_final_loop_never_reuses():
    # reuse is free and harmless everywhere; only loops before the last may take it
    L, NL = 3, 2
    n = L * NL
    d = np.zeros((n, 3))
    r = np.tile([3.0, 2.0, 1.0], (n, 1))
    s = np.tile([5, 3, 0], (n, 1)).astype(np.int64)
    kinds, _, rr, ss = P.plan_search_brute(L, NL, d, r, s, INF, 10 ** 9)
    assert kinds == (2, 2, 2, 2, 1, 1) and rr == 4 * 1.0 + 2 * 2.0 and ss == 6
