"""Quantization groups of 64 on the GPU (group_size = 64).

K is quantized per channel over 64 tokens and V per token over 64 channels; the last N mod 64
tokens stay exact in the tail. A group's K meta is split over its four 16-token records and
V meta is [D/64][16] per record (half the meta bytes of groups of 32). Checked against the
fp64 oracle at group 64: records bit for bit (padding excluded), tails, bulk against
token-by-token appends, decode rows over ragged lengths at every tau regime, the split and
token-skipping decodes, grouped queries with a mixed plan and the KIVI-4 layout, decode-time
appends in the per-(loop, layer) order, and the crafted correction rows (including the one
that recomputes the row's values). Method: "LoopKV: Loop-Aware KV Cache Compression for
Serving Looped Transformers" (arXiv:2611.04137), Abstract; the group width is a shape option
the pages leave open.
"""
import numpy as np
import pytest
import torch

import quantized_kv_cache_loopkv_amd as lkv
from oracle import loopkv_oracle as O
from synth import recipes as R
from tests.harness import Workload, oracle_row_inputs
from tests.test_gpu_parity import check_row

pytestmark = pytest.mark.gpu

G64 = 64


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("layout,plan", [(lkv.LAYOUT_PLANES, [0]), (lkv.LAYOUT_PLANES, [1]), (lkv.LAYOUT_KIVI4, [0])])
@pytest.mark.parametrize("D", [64, 128, 256])
def test_gpu_group64_records(layout, plan, D):
    _need_gpu()
    lengths = [1, 63, 64, 65, 100, 257]
    cfg = R.small_config("g64rec", 1, 1, 2, D, lengths, [0.01], plan=plan, outlier_count=3, outlier_mult=10.0,
                         shuffled=True, group=G64)
    wl = Workload(cfg, layout=layout, gpu_synth=False)
    wl.fill()
    bits = 2 if plan[0] == 1 else 4
    kind = O.KIND_Q2 if bits == 2 else O.KIND_Q4
    assert wl.ctx.cell_storage(0, 0)["record_bytes"] == O.record_bytes(D, kind, layout, G64)
    for b, N in enumerate(lengths):
        for h in range(cfg.n_heads):
            kb, vb, K, V = oracle_row_inputs(cfg, 0, b, h, N, wl.factors)
            qh = O.quantize_history(K, V, bits, G64)
            for j in range(qh["n_q"] // 16):
                want = O.pack_block(qh, j, layout)
                got = wl.record(0, b, h, j)[:want.size]
                assert np.array_equal(got, want), f"record D={D} b={b} h={h} j={j}"
            n_q, tk, tv = O.tail_tokens(kb, vb, G64)
            tail = wl.tail(0, b, h)
            for i in range(N - n_q):
                p = n_q + i
                assert np.array_equal(tail[0, p % G64], tk[i]) and np.array_equal(tail[1, p % G64], tv[i])


def test_gpu_group64_bulk_equals_incremental():
    _need_gpu()
    lengths = [140, 140]
    cfg = R.small_config("g64inc", 1, 1, 2, 128, lengths, [0.01], shuffled=True, group=G64)
    bulk = Workload(cfg, gpu_synth=False)
    bulk.fill()
    inc = Workload(cfg, gpu_synth=False)
    K, V = inc.kv_chunk(0, 0, 140)
    lens = torch.zeros(2, dtype=torch.int32, device="cuda")
    for t in range(140):   # one token at a time: groups complete at 64 and 128
        inc.ctx.append(K[:, t:t + 1].contiguous(), V[:, t:t + 1].contiguous(), inc.bt, lens, cell=(0, 0))
        lens += 1
    torch.cuda.synchronize()
    for b in range(2):
        for h in range(2):
            for j in range(128 // 16):
                assert np.array_equal(bulk.record(0, b, h, j), inc.record(0, b, h, j)), (b, h, j)
            assert np.array_equal(bulk.tail(0, b, h)[:, :12], inc.tail(0, b, h)[:, :12])


@pytest.mark.parametrize("tau", [0.0, 0.001, 0.01, 1.1])
@pytest.mark.parametrize("D", [64, 128, 256])
def test_gpu_group64_rows(tau, D):
    _need_gpu()
    lengths = [1, 63, 64, 65, 127, 128, 129, 640, 1000, 2049]
    cfg = R.small_config("g64rows", 1, 1, 2, D, lengths, [tau], outlier_count=3, outlier_mult=10.0, shuffled=True,
                         group=G64)
    wl = Workload(cfg, gpu_synth=False)
    wl.fill()
    q = wl.q_all() * 2
    q = q.to(torch.bfloat16).float().to(q.dtype)
    for n_split in (0, 3):
        out, sm = wl.ctx.decode(q, wl.bt, wl.seq_lens, wl.max_len(), tau, sel_mask=True, n_split=n_split)
        torch.cuda.synchronize()
        for b, N in enumerate(lengths):
            for h in range(2):
                check_row(wl, out, sm, q, 0, b, h, tau, N, f"g64 D={D} tau={tau} split={n_split} b={b} h={h}")
    if 0 < tau <= 1:
        from tests.test_gpu_skip import _check_skip_row
        out, sm = wl.ctx.decode(q, wl.bt, wl.seq_lens, wl.max_len(), tau, sel_mask=True, skip=True)
        torch.cuda.synchronize()
        for b, N in enumerate(lengths):
            for h in range(2):
                _check_skip_row(wl, out, sm, q, 0, b, h, tau, N, f"g64 skip D={D} tau={tau} b={b} h={h}")


def test_gpu_group64_mixed_plan_gqa_and_kivi():
    _need_gpu()
    plan = np.array([[0, 2], [1, 0]], dtype=np.uint8)
    lengths = [95, 517, 1000]
    cfg = R.small_config("g64mix", 2, 2, 4, 128, lengths, [0.01], plan=plan, cell_scales=True, shuffled=True,
                         n_kv_heads=2, outlier_count=2, outlier_mult=8.0, group=G64)
    wl = Workload(cfg, gpu_synth=False)
    wl.fill()
    q = wl.q_all()
    for tau in (0.0, 0.01, 1.1):
        out, sm = wl.ctx.decode(q, wl.bt, wl.seq_lens, wl.max_len(), tau, sel_mask=True)
        torch.cuda.synchronize()
        for c in range(4):
            for b, N in enumerate(lengths):
                for h in range(4):
                    check_row(wl, out, sm, q, c, b, h, tau, N, f"g64 mixed tau={tau} c={c} b={b} h={h}")
    kw = Workload(cfg, layout=lkv.LAYOUT_KIVI4, gpu_synth=False)
    kw.fill()
    out, sm = kw.ctx.decode(q, kw.bt, kw.seq_lens, kw.max_len(), 0.01, sel_mask=True)
    torch.cuda.synchronize()
    for c in range(4):
        for b, N in enumerate(lengths):
            for h in range(4):
                check_row(kw, out, sm, q, c, b, h, 0.01, N, f"g64 kivi c={c} b={b} h={h}")


def test_gpu_group64_serving_appends():
    """Decode-time appends in the per-(loop, layer) order, crossing a 64-token boundary."""
    _need_gpu()
    steps = 4
    plan = np.array([[0, 2], [1, 0]], dtype=np.uint8)
    lengths = [62, 300]   # the first sequence completes its group during the steps
    cfg = R.small_config("g64serve", 2, 2, 2, 128, lengths, [0.01], plan=plan, cell_scales=True, shuffled=True,
                         append_steps=steps, group=G64)
    wl = Workload(cfg, gpu_synth=False)
    wl.fill()
    C, B, H, D = cfg.n_cells, cfg.batch, cfg.n_heads, cfg.head_dim
    max_len = max(lengths) + steps
    lb = torch.tensor(lengths, dtype=torch.int32, device="cuda")
    la = lb + 1
    out = torch.zeros((C, B, H, D), dtype=torch.float32, device="cuda")
    sm = torch.zeros((C, B, H, (max_len + 31) // 32), dtype=torch.int32, device="cuda")
    for s in range(steps):
        K, V, _, _ = wl.append_inputs(s)
        q = wl.q_all(s)
        wl.serving_step(K, V, q, lb, la, max_len, 0.01, out, sm)
    torch.cuda.synchronize()
    for c in range(C):
        share = wl.plan[c] == R.SHARE
        for b, n0 in enumerate(lengths):
            n = n0 + steps - (1 if share else 0)
            for h in range(H):
                check_row(wl, out, sm, q, c, b, h, 0.01, n, f"g64 serving c={c} b={b} h={h} n={n}")


@pytest.mark.parametrize("mode", ["drop", "rise"])
@pytest.mark.parametrize("D", [64, 128, 256])
def test_gpu_group64_correction_rows(D, mode):
    _need_gpu()
    from tests.test_gpu_corrections import _check, _winner_row
    K, V, q = _winner_row(D, 512 + 7, mode, seed=11)
    for n_split in (0, 3):
        err, n_sel = _check(K, V, q, 0.01, f"g64 {mode} D={D} split={n_split}", n_split=n_split, group=G64)
        assert n_sel >= 1
        print(f"g64 {mode} D={D} split={n_split}: rel err {err:.2e}, selected {n_sel}", flush=True)
