"""The largest supported sizes. max_len = LOOPKV_MAX_LEN (32768 tokens), whose coarse scores
fill most of a workgroup's LDS (one workgroup per CU), with the largest split
(LOOPKV_MAX_SPLIT workgroups per row). Rows of a 4-bit and a 2-bit cell at 32768 tokens (no
tail), 32767 (a 31-token tail) and 1 token are checked against the fp64 oracle; the selection
mask covers all 1024 words of a row. Method: "LoopKV: Loop-Aware KV Cache Compression for
Serving Looped Transformers" (arXiv:2611.04137), Abstract (decoding sentence). And the largest
plan, LOOPKV_MAX_CELLS cells, in one whole-plan append and decode.
"""
import numpy as np
import pytest
import torch

import quantized_kv_cache_loopkv_amd as lkv
from synth import recipes as R
from tests.harness import Workload
from tests.test_gpu_parity import check_row

pytestmark = pytest.mark.gpu

MAX_LEN = 32768
LENGTHS = [MAX_LEN, MAX_LEN - 1, 1]


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


_cache = {}


def _workload(D):
    if D not in _cache:
        _cache.clear()
        cfg = R.small_config("maxlen", 1, 2, 2, D, LENGTHS, [0.01], plan=np.array([[0, 1]], dtype=np.uint8),
                             outlier_count=3, outlier_mult=10.0, cell_scales=True, shuffled=True, seed=7)
        wl = Workload(cfg, gpu_synth=True)
        wl.fill()
        torch.cuda.synchronize()
        _cache[D] = wl
    return _cache[D]


@pytest.mark.parametrize("D,tau", [(128, 0.0), (128, 0.01), (128, 1.1), (256, 0.01), (64, 0.01), (64, 0.0)])
def test_gpu_max_len_rows(D, tau):
    _need_gpu()
    wl = _workload(D)
    assert wl.max_len() == MAX_LEN
    q = wl.q_all() * 2
    q = q.to(torch.bfloat16).float().to(q.dtype)
    splits = (0, lkv.MAX_SPLIT) if tau == 0.01 else (0, 8)
    for n_split in splits:
        out, sm = wl.ctx.decode(q, wl.bt, wl.seq_lens, MAX_LEN, tau, sel_mask=True, n_split=n_split)
        torch.cuda.synchronize()
        assert sm.shape[-1] == MAX_LEN // 32
        print(f"D={D} tau={tau} n_split={n_split}: decoded", flush=True)
        for c in range(2):
            for b, N in enumerate(LENGTHS):
                for h in range(2):
                    if n_split and (h or b == 2):   # split rows: the two long sequences, head 0
                        continue
                    check_row(wl, out, sm, q, c, b, h, tau, N, f"D={D} tau={tau} split={n_split} c={c} b={b} h={h}")


def test_gpu_max_cells():
    """The largest plan, LOOPKV_MAX_CELLS = 128 cells (8 loops x 16 layers), in one whole-plan
    append and decode: every row of every cell against the oracle (the kernel arguments carry
    all 128 cell descriptors)."""
    _need_gpu()
    L, NL = 8, 16
    assert L * NL == lkv.MAX_CELLS
    rng = np.random.default_rng(5)
    plan = rng.integers(0, 3, size=(L, NL)).astype(np.uint8)
    plan[L - 1][plan[L - 1] == 2] = 1
    lengths = [40, 97]
    cfg = R.small_config("maxcells", L, NL, 2, 64, lengths, [0.01], plan=plan, cell_scales=True, shuffled=True,
                         append_steps=1)
    wl = Workload(cfg, gpu_synth=False)
    wl.fill()
    wl.append_step(0)   # one whole-plan append over every storing cell
    q = wl.q_all(1)
    out, sm = wl.ctx.decode(q, wl.bt, wl.seq_lens, wl.max_len(1), 0.01, sel_mask=True)
    torch.cuda.synchronize()
    for c in range(L * NL):
        for b, N in enumerate(lengths):
            for h in range(2):
                check_row(wl, out, sm, q, c, b, h, 0.01, N + 1, f"max cells c={c} b={b} h={h}")
