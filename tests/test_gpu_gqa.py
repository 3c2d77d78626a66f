"""Grouped queries (n_kv_heads < n_heads) on the GPU.

Each query head h reads KV head h // (n_heads / n_kv_heads); pools, tails and appends hold the
KV heads only. Rows are checked against the fp64 oracle over their KV head's history, and the
whole decode is checked bit for bit against an MHA cache that stores each KV head once per
query head (same records, same arithmetic per row). Method: "LoopKV: Loop-Aware KV Cache
Compression for Serving Looped Transformers" (arXiv:2611.04137), Abstract (decoding sentence).
"""
import numpy as np
import pytest
import torch

import quantized_kv_cache_loopkv_amd as lkv
from synth import recipes as R
from tests.harness import Workload
from tests.test_gpu_parity import check_row

pytestmark = pytest.mark.gpu


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("H,Hkv,D", [(8, 2, 128), (4, 1, 64), (6, 3, 128), (4, 2, 256)])
def test_gpu_gqa_rows(H, Hkv, D):
    _need_gpu()
    lengths = [33, 640, 1000]   # 3 sequences: KV-head groups not a multiple of 8 (grid padding)
    cfg = R.small_config("gqa", 1, 1, H, D, lengths, [0.01], outlier_count=3, outlier_mult=10.0, shuffled=True,
                         n_kv_heads=Hkv)
    wl = Workload(cfg, gpu_synth=False)
    wl.fill()
    q = wl.q_all() * 2
    q = q.to(torch.bfloat16).float().to(q.dtype)
    for tau in (0.0, 0.01, 1.1):
        out, sm = wl.decode(q, tau)
        torch.cuda.synchronize()
        for b, N in enumerate(lengths):
            for h in range(H):
                check_row(wl, out, sm, q, 0, b, h, tau, N, f"H={H} Hkv={Hkv} b={b} h={h} tau={tau}")


def test_gpu_gqa_mixed_plan_split_and_skip():
    """4-bit, 2-bit and reuse cells with 8 query heads over 2 KV heads: the one-workgroup,
    split and skip decodes of every row against the oracle (skip rows in their own test)."""
    _need_gpu()
    plan = np.array([[0, 2], [1, 0]], dtype=np.uint8)
    lengths = [300, 517]
    cfg = R.small_config("gqaplan", 2, 2, 8, 128, lengths, [0.01], plan=plan, cell_scales=True, shuffled=True,
                         n_kv_heads=2)
    wl = Workload(cfg, gpu_synth=False)
    wl.fill()
    q = wl.q_all()
    for n_split in (0, 3):
        out, sm = wl.ctx.decode(q, wl.bt, wl.seq_lens, wl.max_len(), 0.01, sel_mask=True, n_split=n_split)
        torch.cuda.synchronize()
        for c in range(4):
            for b, N in enumerate(lengths):
                for h in range(8):
                    check_row(wl, out, sm, q, c, b, h, 0.01, N, f"split={n_split} cell={c} b={b} h={h}")
    from tests.test_gpu_skip import _check_skip_row
    out, sm = wl.ctx.decode(q, wl.bt, wl.seq_lens, wl.max_len(), 0.01, sel_mask=True, skip=True)
    torch.cuda.synchronize()
    for c in range(4):
        for b, N in enumerate(lengths):
            for h in range(8):
                _check_skip_row(wl, out, sm, q, c, b, h, 0.01, N, f"skip cell={c} b={b} h={h}")


def test_gpu_gqa_equals_duplicated_mha():
    _need_gpu()
    H, Hkv, D = 8, 2, 128
    lengths = [700, 129, 2000]
    cfg = R.small_config("gqadup", 1, 1, H, D, lengths, [0.01], outlier_count=2, outlier_mult=8.0, n_kv_heads=Hkv)
    g = Workload(cfg, gpu_synth=False)
    g.fill()
    # the same histories in an MHA context: KV head k stored once for each of its query heads
    m = lkv.Context(1, 1, H, D, g.nb, cfg.batch)
    m.plan([0])
    ws = torch.zeros(m.workspace_bytes(), dtype=torch.uint8, device="cuda")
    m.bind(ws)
    for b, N in enumerate(lengths):
        K, V = g.kv_chunk(0, 0, N, seqs=[b])
        K = K[:, :N].repeat_interleave(H // Hkv, dim=2).contiguous()
        V = V[:, :N].repeat_interleave(H // Hkv, dim=2).contiguous()
        lens = torch.zeros(1, dtype=torch.int32, device="cuda")
        slots = torch.tensor([b], dtype=torch.int32, device="cuda")
        m.append(K, V, g.bt[b:b + 1].contiguous(), lens, cell=(0, 0), seq_slots=slots)
    q = g.q_all() * 2
    for tau in (0.0, 0.01, 0.5, 1.1):
        og, sg = g.decode(q, tau)
        om, smm = m.decode(q, g.bt, g.seq_lens, g.max_len(), tau, sel_mask=True)
        torch.cuda.synchronize()
        assert torch.equal(og, om) and torch.equal(sg, smm), f"tau={tau}"
