"""Brute-force oracle of the LoopKV planner.

TEST INFRASTRUCTURE ONLY. Nothing in the library imports this module; only the tests
may use it. It shares no code with the library's planner.

Source: "LoopKV: Loop-Aware KV Cache Compression for Serving Looped Transformers"
(arXiv:2611.04137), Abstract: every (loop, layer) cell is stored at 4 bits, at 2 bits,
or reuses the final loop's KV of its layer (sentence on the one-time offline profile);
damages measured one cell at a time roughly add up to the whole model's (sentence on
the measurements on Ouro); the chosen plan reads as little as possible while its
predicted damage and its storage stay within their budgets (sentence on the planner).

Readings taken where the abstract is silent:

* the predicted damage of a plan is the sum of its cells' damages for their chosen
  kinds (the additive model); reads and storage add up over cells in the same way;
* each cell's damage, reads and storage for each kind are given numbers (the offline
  profile produces them; it is outside this path);
* a plan is feasible when its damage sum is at most the damage budget and its storage
  sum at most the storage budget; cells of the final loop cannot reuse;
* the planner returns a feasible plan of least total reads (None if there is none).

This is that definition written out: every kind assignment (3 kinds per cell, 2 in the
final loop) is enumerated, its sums taken, the infeasible ones dropped and the least-reads
one kept.
Ties in reads are broken by least damage, then least storage, then the smallest
assignment in lexicographic order over cells (kind codes 0 = 4-bit, 1 = 2-bit,
2 = reuse); callers compare the objective, not the tie-break.
"""
from __future__ import annotations

import itertools

import numpy as np

KIND_Q4, KIND_Q2, KIND_SHARE = 0, 1, 2


def allowed_kinds(n_loops: int, n_layers: int):
    """Kinds each cell may take: all three, except reuse in the final loop."""
    out = []
    for c in range(n_loops * n_layers):
        final = c // n_layers == n_loops - 1
        out.append((KIND_Q4, KIND_Q2) if final else (KIND_Q4, KIND_Q2, KIND_SHARE))
    return out


def plan_cost(kinds, damage, reads, storage):
    """Sums of damage, reads and storage of one assignment (arrays [cells][3])."""
    idx = np.arange(len(kinds))
    k = np.asarray(kinds)
    return (float(np.sum(np.asarray(damage, np.float64)[idx, k])),
            float(np.sum(np.asarray(reads, np.float64)[idx, k])),
            int(np.sum(np.asarray(storage, np.int64)[idx, k])))


def plan_search_brute(n_loops: int, n_layers: int, damage, reads, storage, damage_budget: float,
                      storage_budget: int):
    """Least-reads feasible assignment by exhaustive enumeration (small k only).

    Returns (kinds tuple, damage sum, reads sum, storage sum) or None if no plan is feasible."""
    n = n_loops * n_layers
    if n > 13:
        raise ValueError("brute force is for at most 13 cells")
    damage = np.asarray(damage, np.float64)
    reads = np.asarray(reads, np.float64)
    storage = np.asarray(storage, np.int64)
    # every assignment, one per row
    plans = np.array(list(itertools.product(*allowed_kinds(n_loops, n_layers))), dtype=np.int64)
    cells = np.arange(n)
    d = damage[cells, plans].sum(axis=1)
    r = reads[cells, plans].sum(axis=1)
    s = storage[cells, plans].sum(axis=1)
    ok = (d <= damage_budget) & (s <= storage_budget)
    if not ok.any():
        return None
    plans, d, r, s = plans[ok], d[ok], r[ok], s[ok]
    # least reads, then least damage, then least storage, then the lexicographically first plan
    order = np.lexsort(tuple(plans[:, c] for c in range(n - 1, -1, -1)) + (s, d, r))
    i = order[0]
    return tuple(int(k) for k in plans[i]), float(d[i]), float(r[i]), int(s[i])
