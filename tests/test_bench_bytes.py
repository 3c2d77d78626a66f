"""bench.py's algorithmic byte counts against the per-token-head figures of the record layout.

At D = 128 with groups of 32 a 4-bit or 2-bit target reads 96 bytes per quantized token-head
(K_hi 32 + K_meta 16 + V_hi 32 + V_meta 16), a selected token adds 64 (K_lo + V_lo), KIVI-4
reads 160; groups of 64 halve the meta (80, 64, 144). A tail token costs 4 D bytes (bf16 K
and V); each row adds q and output (2 D bytes each in bf16); each (cell, sequence) adds 4 bytes
per 16-token block of the block table, which its heads share.
"""
import numpy as np
import pytest

import bench


def _row_extra(N, D, G):
    """Per-row bytes besides the quantized prefix (tail, q, output), and n_q."""
    n_q = G * (N // G)
    return (N - n_q) * 4 * D + 2 * D + 2 * D, n_q


def _table(N):
    """Block-table bytes of one (cell, sequence): read once for all of its heads."""
    return 4 * ((N + 15) // 16)


@pytest.mark.parametrize("H", [1, 16])
@pytest.mark.parametrize("D,G,base,kivi", [(128, 32, 96, 160), (128, 64, 80, 144), (64, 32, 48, 80),
                                          (64, 64, 40, 72), (256, 64, 160, 288)])
def test_decode_bytes_per_token_head(D, G, base, kivi, H):
    lengths = [1000, 77]
    plan = [0, 1]   # one 4-bit and one 2-bit cell
    sel = np.zeros((2, 2, H), dtype=np.int64)
    sel[0, 0, 0] = 7
    sel[0, 1, H - 1] = 2
    want = sel_bytes = 9 * (D // 2)
    want_kivi = 0
    for N in lengths:
        extra, n_q = _row_extra(N, D, G)
        want += 2 * (H * (n_q * base + extra) + _table(N))
        want_kivi += 2 * (H * (n_q * kivi + extra) + _table(N))
    assert bench.algorithmic_bytes(plan, lengths, H, D, sel, group=G) == want
    assert bench.algorithmic_bytes(plan, lengths, H, D, layout_kivi=True, group=G) == want_kivi
    assert sel_bytes == 9 * (D // 2)


def test_headline_bytes_match_the_formula():
    """The 16K, batch-32, 16-head plan: 96 cells x 32 sequences x (16 heads x (n_q x 96 + 512)
    + 4096 table bytes), plus 64 bytes per selected token of a 4-bit target."""
    from synth import recipes as R
    plan = R.make_config("C4").plan.reshape(-1)
    sel = np.zeros((96, 32, 16), dtype=np.int64)
    sel[0, 0, 0] = 100
    got = bench.algorithmic_bytes(plan, [16384] * 32, 16, 128, sel)
    assert got == 96 * 32 * (16 * (16384 * 96 + 512) + 4096) + 100 * 64
    assert abs(got / 1e9 - 77.347) < 0.001


@pytest.mark.parametrize("G", [32, 64])
def test_skip_bytes(G):
    D, N, H = 128, 700, 3
    extra, n_q = _row_extra(N, D, G)
    sel = np.zeros((2, 1, H), dtype=np.int64)
    sel[0, 0, 1] = 5
    got = bench.algorithmic_bytes_skip(np.array([0, 1]), [N], H, D, sel, group=G)
    k_part = 32 + 4 * D // G          # K_hi + K_meta
    rest = 32 + 32 + 32 + 4 * D // G  # K_lo + V_hi + V_lo + V_meta of a selected token
    assert got == (H * (n_q * k_part + extra) + _table(N)) + (H * (n_q * (64 + 8 * D // G) + extra) + _table(N)) \
        + 5 * rest


@pytest.mark.parametrize("G", [32, 64])
def test_append_bytes(G):
    D, H, B = 128, 2, 3
    before = [G - 1, 5, 2 * G - 1]   # two sequences complete a group
    tok = 2 * H * D * 2
    got = bench.append_bytes(4, B, H, D, before, group=G)
    flush = H * ((G - 1) * 4 * D + (G // 16) * (16 * D + 2 * (64 * D // G)))
    assert got == 4 * B * 2 * tok + 4 * 2 * flush
    # one of the four storing cells at 2 bits: its records hold one K and one V plane (8 D per block)
    flush2 = H * ((G - 1) * 4 * D + (G // 16) * (8 * D + 2 * (64 * D // G)))
    assert bench.append_bytes(4, B, H, D, before, group=G, n_q2=1) == 4 * B * 2 * tok + 3 * 2 * flush + 2 * flush2


def test_append_figures_split_step_kinds():
    """Token-only steps and group-completing steps are reported apart, each with its own bytes."""
    D, H, B, G = 128, 2, 2, 32
    lens = [[5, 7], [G - 1, 2 * G - 1], [6, 8]]
    fig = bench.append_figures([0.01, 0.5, 0.03], lens, 3, B, H, D, G, n_q2=1)
    assert fig["token_only"]["steps"] == 2 and fig["group_completing"]["steps"] == 1
    assert abs(fig["token_only"]["ms"] - 0.02) < 1e-9 and fig["group_completing"]["ms"] == 0.5
    by = bench.append_bytes(3, B, H, D, lens[1], G, 1)
    assert abs(fig["group_completing"]["algorithmic_GB"] - round(by / 1e9, 4)) < 1e-12


def test_gathered_bytes_counts_units_and_blocks():
    """The corrections load, per unit holding a selected token, its K low plane (2 records x 4D)
    and its group's K meta (4D); per block holding one, its V planes (2 x 4D) and V meta."""
    import torch
    D = 128
    sm = torch.zeros((2, 1, 1, 4), dtype=torch.int32)
    sm[0, 0, 0, 0] = 1                    # unit 0: block 0
    sm[0, 0, 0, 2] = (1 << 16) | 1        # unit 2: blocks 4 and 5
    sm[1, 0, 0, 1] = 5                    # a 2-bit target's row: nothing is gathered
    assert bench.gathered_bytes(sm, np.array([0, 1]), D, 32) == 2 * (8 * D + 4 * D) + 3 * (8 * D + 2 * D)
    assert bench.gathered_bytes(sm, np.array([0, 1]), D, 64) == 2 * (8 * D + 4 * D) + 3 * (8 * D + D)


def test_cpu_rows_task(tmp_path):
    """The oracle leg's worker: reads a chunk, decodes each row as the oracle does."""
    import math
    from oracle import loopkv_oracle as O
    from synth.philox import bf16_bits_to_f32, f32_to_bf16_bits
    rng = np.random.default_rng(0)
    N, H, D = 200, 2, 64
    kb = f32_to_bf16_bits(rng.standard_normal((N, H, D)).astype(np.float32))
    vb = f32_to_bf16_bits(rng.standard_normal((N, H, D)).astype(np.float32))
    kp, vp = str(tmp_path / "k.npy"), str(tmp_path / "v.npy")
    np.save(kp, kb)
    np.save(vp, vb)
    q = rng.standard_normal((H, D))
    sig = 1.0 / math.sqrt(D)
    res = bench.cpu_rows_task(kp, vp, [(1, q[1], 0), (0, q[0], 0)], 0.01, sig, 32, 4, 2)
    assert [r[0] for r in res] == [0, 1] and all(len(r[1]) == 2 for r in res)
    for h, _, n_sel in res:
        K = bf16_bits_to_f32(np.ascontiguousarray(kb[:, h])).astype(np.float64)
        V = bf16_bits_to_f32(np.ascontiguousarray(vb[:, h])).astype(np.float64)
        _, sel, _ = O.decode_row(q[h], K, V, 0, 0.01, sig)
        assert n_sel == int(sel.sum())


@pytest.mark.parametrize("G", [32, 64])
def test_prefill_bytes(G):
    """Bulk appends: K and V in, the complete groups' records out, the rest into the tail; reuse
    cells store nothing."""
    D, H = 128, 2
    lengths = [3 * G + 5, G]
    got = bench.prefill_bytes(np.array([0, 1, 2]), lengths, H, D, group=G)
    rec4, rec2 = (G // 16) * record_size(0, D, G), (G // 16) * record_size(1, D, G)
    want = 0
    for rec in (rec4, rec2):
        for N in lengths:
            want += H * (N * 4 * D + (N // G) * rec + (N % G) * 4 * D)
    assert got == want
    assert record_size(0, D, 32) == 20 * D and record_size(1, D, 32) == 12 * D   # the layout's 20D / 12D
    assert record_size(0, D, 64) == 18 * D and record_size(1, D, 64) == 10 * D


def record_size(kind, D, G):
    """Bytes of one 16-token record, from the record layout: the K and V high planes (4 D each),
    the K meta and the V meta (64 D / G each: 2 D at G = 32), and at 4 bits the K and V low
    planes (4 D each)."""
    meta = 2 * (64 * D // G)
    planes = 2 * 4 * D + (2 * 4 * D if kind == 0 else 0)
    return planes + meta
