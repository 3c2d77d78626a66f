"""The library's planner (loopkv_plan_search, host code) against the brute-force oracle (CPU).

"LoopKV: Loop-Aware KV Cache Compression for Serving Looped Transformers" (arXiv:2611.04137),
Abstract (sentence on the planner): per (loop, layer) cell the planner picks 4-bit, 2-bit or
final-loop reuse so that reads are least while predicted (additive) damage and storage stay
within budget.

Costs are dyadic rationals (multiples of 2^-10), so every sum is exact in float64 and both
sides decide feasibility identically. Several plans can share the least reads: the total
reads are compared exactly, and the library's plan is checked to be feasible, to keep the
final loop off reuse and to have the sums it reports.
"""
import math

import numpy as np
import pytest

import quantized_kv_cache_loopkv_amd as lkv
from oracle import planner_oracle as P

INF = math.inf


def _table(rng, n, dmax=4096, rmax=8192, smax=6):
    d = rng.integers(0, dmax, size=(n, 3)) / 1024.0
    r = rng.integers(64, rmax, size=(n, 3)) / 1024.0
    s = rng.integers(0, smax, size=(n, 3)).astype(np.int64)
    return d, r, s


def _check_plan(L, NL, d, r, s, D, S, got):
    kinds, dd, rr, ss = got
    allowed = P.allowed_kinds(L, NL)
    assert all(k in allowed[c] for c, k in enumerate(kinds)), kinds
    assert (dd, rr, ss) == P.plan_cost(kinds, d, r, s)
    assert dd <= D and ss <= S


@pytest.mark.parametrize("shape", [(1, 1), (1, 5), (2, 3), (3, 2), (2, 6), (3, 4), (4, 3)])
def test_planner_matches_brute_force(shape):
    L, NL = shape
    n = L * NL
    rng = np.random.default_rng(100 + 7 * L + NL)
    checked = infeasible = 0
    for trial in range(8):
        d, r, s = _table(rng, n)
        dsum, ssum = float(d.max(axis=1).sum()), int(s.max(axis=1).sum())
        for fd, fs in ((INF, 10 ** 9), (0.5, 10 ** 9), (INF, 0.5), (0.3, 0.6), (0.15, 0.4), (0.05, 0.2), (0.0, 0.0)):
            D = fd if fd == INF else fd * dsum
            S = fs if fs == 10 ** 9 else int(fs * ssum)
            want = P.plan_search_brute(L, NL, d, r, s, D, S)
            if want is None:
                with pytest.raises(lkv.LoopKVError) as e:
                    lkv.plan_search(L, NL, d, r, s, D, S)
                assert e.value.status == lkv.loopkv.ERR_PLAN
                infeasible += 1
                continue
            got = lkv.plan_search(L, NL, d, r, s, D, S)
            _check_plan(L, NL, d, r, s, D, S, got)
            assert got[2] == want[2], (shape, trial, fd, fs, got, want)
            checked += 1
    assert checked >= 15 and infeasible >= 1


def test_planner_at_plan_scale_identical_cells():
    """4 x 24 cells with one cost table for every cell: the optimum depends only on how many
    cells take each kind, so it is found exactly by enumerating the counts."""
    L, NL = 4, 24
    n = L * NL
    rng = np.random.default_rng(7)
    for trial in range(6):
        dk = rng.integers(0, 64, size=3) / 1024.0
        rk = rng.integers(64, 512, size=3) / 1024.0
        sk = rng.integers(0, 6, size=3).astype(np.int64)
        d, r, s = np.tile(dk, (n, 1)), np.tile(rk, (n, 1)), np.tile(sk, (n, 1))
        for fd, fs in ((0.5, 0.5), (0.3, 0.8), (0.8, 0.3), (INF, 0.5)):
            D = INF if fd == INF else fd * float(dk.max()) * n
            S = int(fs * int(sk.max()) * n)
            best = None
            n_o, n_f = n - NL, NL   # cells that may reuse / final-loop cells
            for a4f in range(n_f + 1):
                a2f = n_f - a4f
                for a4 in range(n_o + 1):
                    for a2 in range(n_o - a4 + 1):
                        aS = n_o - a4 - a2
                        cnt = (a4 + a4f, a2 + a2f, aS)
                        dd = sum(c * x for c, x in zip(cnt, dk))
                        ss = sum(c * int(x) for c, x in zip(cnt, sk))
                        if dd <= D and ss <= S:
                            rr = sum(c * x for c, x in zip(cnt, rk))
                            best = rr if best is None else min(best, rr)
            if best is None:
                with pytest.raises(lkv.LoopKVError):
                    lkv.plan_search(L, NL, d, r, s, D, S)
                continue
            got = lkv.plan_search(L, NL, d, r, s, D, S)
            _check_plan(L, NL, d, r, s, D, S, got)
            assert got[2] == best


def test_planner_random_plan_scale_properties():
    """4 x 24 random tables: the plan is feasible, no single-cell change lowers its reads
    within the budgets, and renumbering the cells of each loop leaves the optimum unchanged."""
    L, NL = 4, 24
    n = L * NL
    rng = np.random.default_rng(11)
    allowed = P.allowed_kinds(L, NL)
    for trial in range(3):
        d, r, s = _table(rng, n, dmax=256, rmax=4096, smax=6)
        D = 0.4 * float(d.max(axis=1).sum())
        S = int(0.5 * int(s.max(axis=1).sum()))
        kinds, dd, rr, ss = lkv.plan_search(L, NL, d, r, s, D, S)
        _check_plan(L, NL, d, r, s, D, S, (kinds, dd, rr, ss))
        for c in range(n):
            for k in allowed[c]:
                if k == kinds[c]:
                    continue
                d2, r2, s2 = dd - d[c, kinds[c]] + d[c, k], rr - r[c, kinds[c]] + r[c, k], ss - s[c, kinds[c]] + s[c, k]
                assert not (d2 <= D and s2 <= S and r2 < rr), (c, k)
        perm = np.concatenate([rng.permutation(NL) + i * NL for i in range(L)])
        k2, _, rr2, _ = lkv.plan_search(L, NL, d[perm], r[perm], s[perm], D, S)
        assert rr2 == rr


def test_planner_reads_model_plan():
    """A table in the decode's own units (bytes per token-head at head dim 128): 4-bit reads
    96 + 64 f (f: selected fraction), 2-bit 96, reuse the final-loop cell's 4-bit bytes (a table
    entry, as a profile would give it); storage 160 / 96
    / 0 bytes in 32-byte units; damages rise toward earlier loops for reuse. With the storage
    budget of the 50/30/20 reference plan the planner meets both budgets."""
    L, NL = 4, 24
    n = L * NL
    rng = np.random.default_rng(3)
    f = rng.integers(0, 64, size=n) / 4096.0
    reads = np.stack([96 + 64 * f, np.full(n, 96.0), 96 + 64 * f[(L - 1) * NL + np.arange(n) % NL]], axis=1)
    storage = np.tile(np.array([5, 3, 0], np.int64), (n, 1))
    loop = np.arange(n) // NL
    damage = np.stack([rng.integers(0, 8, size=n), rng.integers(16, 64, size=n),
                       rng.integers(8, 32, size=n) * (L - loop)], axis=1) / 1024.0
    S = 48 * 5 + 29 * 3
    D = float(damage[:, 1].sum()) * 0.6
    kinds, dd, rr, ss = lkv.plan_search(L, NL, damage, reads, storage, D, S)
    _check_plan(L, NL, damage, reads, storage, D, S, (kinds, dd, rr, ss))
    ctx = lkv.Context(L, NL, 16, 128, 64, 2)
    ctx.plan(kinds)   # a valid plan for the library
    print(f"kinds: {np.bincount(kinds, minlength=3)}, damage {dd:.3f} / {D:.3f}, storage {ss} / {S}")


@pytest.mark.parametrize("bad", ["nan_damage", "neg_reads", "inf_reads", "neg_storage", "nan_budget", "neg_budget",
                                 "zero_cells"])
def test_planner_rejects(bad):
    d = np.zeros((2, 3))
    r = np.ones((2, 3))
    s = np.ones((2, 3), np.int64)
    L, NL, D, S = 2, 1, 1.0, 10
    if bad == "nan_damage":
        d[0, 1] = np.nan
    elif bad == "neg_reads":
        r[1, 0] = -1
    elif bad == "inf_reads":
        r[0, 2] = np.inf
    elif bad == "neg_storage":
        s[0, 0] = -1
    elif bad == "nan_budget":
        D = np.nan
    elif bad == "neg_budget":
        S = -1
    elif bad == "zero_cells":
        L = 0
    with pytest.raises(lkv.LoopKVError) as e:
        lkv.plan_search(L, NL, d, r, s, D, S)
    assert e.value.status == lkv.loopkv.ERR_INVALID_ARG
