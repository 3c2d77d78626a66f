"""bench.py's algorithmic byte counts against the per-token-head figures of the record layout.

At D = 128 with groups of 32 a 4-bit or 2-bit target reads 96 bytes per quantized token-head
(K_hi 32 + K_meta 16 + V_hi 32 + V_meta 16), a selected token adds 64 (K_lo + V_lo), KIVI-4
reads 160; groups of 64 halve the meta (80, 64, 144). A tail token costs 4 D bytes (bf16 K
and V); each row adds q and output (2 D bytes each in bf16), 4 bytes per 16-token block of
the block table and 4 for its length.
"""
import numpy as np
import pytest

import bench


def _row_extra(N, D, G):
    n_q = G * (N // G)
    return (N - n_q) * 4 * D + 2 * D + 2 * D + 4 * ((N + 15) // 16) + 4, n_q


@pytest.mark.parametrize("D,G,base,kivi", [(128, 32, 96, 160), (128, 64, 80, 144), (64, 32, 48, 80),
                                          (64, 64, 40, 72), (256, 64, 160, 288)])
def test_decode_bytes_per_token_head(D, G, base, kivi):
    N = 1000
    extra, n_q = _row_extra(N, D, G)
    plan = [0, 1]   # one 4-bit and one 2-bit cell, one sequence, one head
    sel = np.zeros((2, 1, 1), dtype=np.int64)
    sel[0, 0, 0] = 7
    got = bench.algorithmic_bytes(plan, [N], 1, D, sel, group=G)
    assert got == 2 * (n_q * base + extra) + 7 * (D // 2)
    assert bench.algorithmic_bytes(plan, [N], 1, D, layout_kivi=True, group=G) == 2 * (n_q * kivi + extra)


@pytest.mark.parametrize("G", [32, 64])
def test_skip_bytes(G):
    D, N = 128, 700
    extra, n_q = _row_extra(N, D, G)
    sel = np.zeros((2, 1, 1), dtype=np.int64)
    sel[0, 0, 0] = 5
    got = bench.algorithmic_bytes_skip(np.array([0, 1]), [N], 1, D, sel, group=G)
    k_part = 32 + 4 * D // G          # K_hi + K_meta
    rest = 32 + 32 + 32 + 4 * D // G  # K_lo + V_hi + V_lo + V_meta of a selected token
    assert got == (n_q * k_part + extra) + (n_q * (64 + 8 * D // G) + extra) + 5 * rest


@pytest.mark.parametrize("G", [32, 64])
def test_append_bytes(G):
    D, H, B = 128, 2, 3
    before = [G - 1, 5, 2 * G - 1]   # two sequences complete a group
    tok = 2 * H * D * 2
    got = bench.append_bytes(4, B, H, D, before, group=G)
    flush = H * ((G - 1) * 4 * D + (G // 16) * (16 * D + 2 * (64 * D // G)))
    assert got == 4 * B * 2 * tok + 4 * 2 * flush
