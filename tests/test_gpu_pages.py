"""32-token pages of the block table on the GPU.

A page of 32 tokens is two consecutive 16-token record slots (the record layout does not
change), so a cache paged at 32 tokens must hold, record for record, the bytes of the same
cache paged at 16, and every decode over it must give bit-identical outputs and selections.
Checked on a mixed plan (4-bit, 2-bit and reuse cells) with grouped queries, shuffled page
tables and ragged lengths: records and tails after the bulk fill, the one-workgroup, split and
token-skipping decodes, and one-token appends at decode time that complete groups; plus rows
against the fp64 oracle. Paging of the KV cache: "LoopKV: Loop-Aware KV Cache Compression for
Serving Looped Transformers" (arXiv:2611.04137), Abstract (serving sentence).
"""
import numpy as np
import pytest
import torch

from synth import recipes as R
from tests.harness import Workload
from tests.test_gpu_parity import check_row

pytestmark = pytest.mark.gpu

STEPS = 3
LENGTHS = [95, 517, 1000]   # the first sequence completes a group during the steps


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _pair(D=128, H=4, Hkv=2):
    plan = np.array([[0, 2], [1, 0]], dtype=np.uint8)
    out = []
    for bt in (16, 32):
        cfg = R.small_config("pages", 2, 2, H, D, LENGTHS, [0.01], plan=plan, cell_scales=True, shuffled=True,
                             n_kv_heads=Hkv, append_steps=STEPS, outlier_count=2, outlier_mult=8.0, block_tokens=bt)
        wl = Workload(cfg, gpu_synth=False)
        wl.fill()
        out.append(wl)
    torch.cuda.synchronize()
    return out


def _same_storage(w16, w32, lengths):
    cfg = w16.cfg
    for c in w16.storing_cells():
        for b, N in enumerate(lengths):
            for h in range(cfg.kv_heads):
                for j in range(32 * (N // 32) // 16):
                    assert np.array_equal(w16.record(c, b, h, j), w32.record(c, b, h, j)), (c, b, h, j)
                r = N % 32   # tail rows past the length are not written
                assert np.array_equal(w16.tail(c, b, h)[:, :r], w32.tail(c, b, h)[:, :r]), (c, b, h)


@pytest.mark.parametrize("D", [64, 128, 256])
def test_gpu_pages_of_32_equal_pages_of_16(D):
    _need_gpu()
    w16, w32 = _pair(D=D)
    assert w32.bt.shape[1] * 2 >= w16.bt.shape[1]
    _same_storage(w16, w32, LENGTHS)
    q = w16.q_all() * 2
    q = q.to(torch.bfloat16).float().to(q.dtype)
    print(f"D={D}: storage equal", flush=True)
    for tau in (0.0, 0.01, 1.1):
        for n_split, skip in ((0, False), (3, False), (0, True)):
            if skip and tau == 0.0:
                continue
            o16, s16 = w16.ctx.decode(q, w16.bt, w16.seq_lens, w16.max_len(), tau, sel_mask=True, n_split=n_split,
                                      skip=skip)
            o32, s32 = w32.ctx.decode(q, w32.bt, w32.seq_lens, w32.max_len(), tau, sel_mask=True, n_split=n_split,
                                      skip=skip)
            torch.cuda.synchronize()
            assert torch.equal(o16, o32) and torch.equal(s16, s32), f"D={D} tau={tau} split={n_split} skip={skip}"
    out, sm = w32.ctx.decode(q, w32.bt, w32.seq_lens, w32.max_len(), 0.01, sel_mask=True)
    torch.cuda.synchronize()
    for c in range(4):
        for b, N in enumerate(LENGTHS):
            for h in range(4):
                check_row(w32, out, sm, q, c, b, h, 0.01, N, f"pages of 32, D={D} cell={c} b={b} h={h}")


def test_gpu_pages_of_32_serving_appends():
    """One-token appends at decode time (per-(loop, layer) order) write the same records."""
    _need_gpu()
    w16, w32 = _pair()
    cfg = w16.cfg
    C, B, H, D = cfg.n_cells, cfg.batch, cfg.n_heads, cfg.head_dim
    max_len = max(LENGTHS) + STEPS
    words = (max_len + 31) // 32
    lens = [(torch.tensor(LENGTHS, dtype=torch.int32, device="cuda"),
             torch.tensor(LENGTHS, dtype=torch.int32, device="cuda") + 1) for _ in range(2)]
    for s in range(STEPS):
        K, V, _, _ = w16.append_inputs(s)
        q = w16.q_all(s)
        res = []
        for wl, (lb, la) in zip((w16, w32), lens):
            out = torch.zeros((C, B, H, D), dtype=torch.float32, device="cuda")
            sm = torch.zeros((C, B, H, words), dtype=torch.int32, device="cuda")
            wl.serving_step(K, V, q, lb, la, max_len, 0.01, out, sm)
            res.append((out, sm))
        torch.cuda.synchronize()
        assert torch.equal(res[0][0], res[1][0]) and torch.equal(res[0][1], res[1][1]), f"step {s}"
    _same_storage(w16, w32, [n + STEPS for n in LENGTHS])


def test_gpu_out_of_range_pages():
    """Page ids outside the pool: a row whose quantized prefix maps one gets NaN output and an
    empty selection (no record read), rows whose prefix is mapped are untouched, and an append
    skips the records of unmapped pages while writing the rest."""
    _need_gpu()
    import math
    from oracle import loopkv_oracle as O
    from tests.harness import oracle_row_inputs
    lengths = [300, 500, 40]
    cfg = R.small_config("badpages", 1, 1, 2, 128, lengths, [0.01], outlier_count=2, outlier_mult=8.0, shuffled=True)
    wl = Workload(cfg, gpu_synth=False)
    wl.fill()
    q = wl.q_all()
    bad = wl.bt.clone()
    bad[0, 3] = -1          # inside sequence 0's quantized prefix (pages 0..17)
    bad[1, 5] = wl.nb       # one past the pool, inside sequence 1's prefix
    bad[2, 5] = -1          # past sequence 2's prefix (pages 0..1): never read
    for n_split, skip in ((0, False), (3, False), (0, True)):
        good = wl.ctx.decode(q, wl.bt, wl.seq_lens, wl.max_len(), 0.01, sel_mask=True, n_split=n_split, skip=skip)
        got = wl.ctx.decode(q, bad, wl.seq_lens, wl.max_len(), 0.01, sel_mask=True, n_split=n_split, skip=skip)
        torch.cuda.synchronize()
        label = f"split={n_split} skip={skip}"
        assert torch.isnan(got[0][0, :2]).all(), label
        assert not got[1][0, :2].any(), label
        assert torch.equal(got[0][0, 2], good[0][0, 2]) and torch.equal(got[1][0, 2], good[1][0, 2]), label
        assert not torch.isnan(good[0]).any(), label

    # append through a table whose page for tokens 32..47 of sequence 1 is unmapped
    ctx = wl.ctx.__class__(1, 1, 2, 128, wl.nb, 3)
    ctx.plan([0])
    ws = torch.zeros(ctx.workspace_bytes(), dtype=torch.uint8, device="cuda")
    ctx.bind(ws)
    holes = wl.bt.clone()
    holes[1, 2] = -1
    holes[1, 3] = 1 << 30
    K, V = wl.kv_chunk(0, 0, 64, seqs=[1])
    lens = torch.zeros(1, dtype=torch.int32, device="cuda")
    slots = torch.tensor([1], dtype=torch.int32, device="cuda")
    ctx.append(K[:, :64].contiguous(), V[:, :64].contiguous(), holes[1:2].contiguous(), lens, cell=(0, 0),
               seq_slots=slots)
    torch.cuda.synchronize()
    st = ctx.cell_storage(0, 0)
    _, _, Kd, Vd = oracle_row_inputs(cfg, 0, 1, 0, 64, wl.factors)
    qh = O.quantize_history(Kd, Vd, 4)
    for j in (0, 1):   # the mapped pages hold group 0
        slot = int(holes[1, j])
        off = st["pool_offset"] + slot * 2 * st["record_bytes"]
        assert np.array_equal(ws[off:off + st["record_bytes"]].cpu().numpy(), O.pack_block(qh, j))
    assert math.isfinite(float(ws.float().sum()))


def test_gpu_out_of_range_slots_and_lengths():
    """A seq_slots entry outside [0, max_seqs) gives its decode rows NaN (other rows untouched)
    and makes an append skip that sequence, as does a negative length in an append."""
    _need_gpu()
    import quantized_kv_cache_loopkv_amd as lkv
    lengths = [300, 77, 40]
    cfg = R.small_config("badslots", 1, 1, 2, 64, lengths, [0.01], shuffled=True)
    wl = Workload(cfg, gpu_synth=False)
    wl.fill()
    q = wl.q_all()
    slots = torch.tensor([0, 99, 2], dtype=torch.int32, device="cuda")
    good = wl.ctx.decode(q, wl.bt, wl.seq_lens, wl.max_len(), 0.01, sel_mask=True)
    got = wl.ctx.decode(q, wl.bt, wl.seq_lens, wl.max_len(), 0.01, sel_mask=True, seq_slots=slots)
    torch.cuda.synchronize()
    assert torch.isnan(got[0][0, 1]).all() and not got[1][0, 1].any()
    for b in (0, 2):
        assert torch.equal(got[0][0, b], good[0][0, b]) and torch.equal(got[1][0, b], good[1][0, b])

    ctx = lkv.Context(1, 1, 2, 64, wl.nb, 3)
    ctx.plan([0])
    ws = torch.zeros(ctx.workspace_bytes(), dtype=torch.uint8, device="cuda")
    ctx.bind(ws)
    K, V = wl.kv_chunk(0, 0, 40, seqs=[0])
    for n in (1, 40):   # the one-kernel append and the prefill path
        ctx.append(K[:, :n].contiguous(), V[:, :n].contiguous(), wl.bt[0:1].contiguous(),
                   torch.zeros(1, dtype=torch.int32, device="cuda"), cell=(0, 0),
                   seq_slots=torch.tensor([3], dtype=torch.int32, device="cuda"))
        ctx.append(K[:, :n].contiguous(), V[:, :n].contiguous(), wl.bt[0:1].contiguous(),
                   torch.full((1,), -5, dtype=torch.int32, device="cuda"), cell=(0, 0))
    torch.cuda.synchronize()
    assert not ws.any(), "an invalid sequence must not be written"
