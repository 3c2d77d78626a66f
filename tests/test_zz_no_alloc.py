"""The no-allocation split decode (loopkv_decode_attn_split_noalloc) against the split decode
with a caller buffer (loopkv_decode_attn_split): the same kernels on the same inputs, so the
outputs and selection masks must agree bit for bit. Two calls in a row, the second with a
smaller input (fewer cells, sequences and splits, a shorter max_len), so the second reads the
fixed array as the first left it; a call whose scratch would exceed the array is refused and
leaves the next call unaffected. Both are checked against the fp64 oracle on sampled rows."""
import numpy as np
import pytest
import torch

import quantized_kv_cache_loopkv_amd as lkv
from quantized_kv_cache_loopkv_amd import loopkv as B
from synth import recipes as R
from tests.harness import Workload
from tests.test_gpu_parity import check_row

pytestmark = pytest.mark.gpu


def test_noalloc_split_matches_caller_scratch():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    plan = np.array([[0, 2], [1, 0]], dtype=np.uint8)
    lengths = [1500, 700, 33, 2100]
    cfg = R.small_config("noalloc", 2, 2, 4, 128, lengths, [0.01], plan=plan, cell_scales=True, shuffled=True,
                         outlier_count=3, outlier_mult=10.0)
    wl = Workload(cfg, gpu_synth=False)
    wl.fill()
    q = (wl.q_all().float() * 3).to(torch.bfloat16)
    max_len = max(lengths)
    # first call: the whole plan, every sequence, 6 splits
    for tau in (0.01, 0.0):
        ref, sm_ref = wl.ctx.decode(q, wl.bt, wl.seq_lens, max_len, tau, sel_mask=True, n_split=6)
        got, sm_got = wl.ctx.decode(q, wl.bt, wl.seq_lens, max_len, tau, sel_mask=True, n_split=6, no_alloc=True)
        torch.cuda.synchronize()
        assert torch.equal(got, ref) and torch.equal(sm_got, sm_ref), f"whole plan tau={tau}"
        for (c, b, h) in [(0, 0, 1), (1, 3, 2), (2, 1, 0), (3, 2, 3), (3, 3, 0)]:
            check_row(wl, got, sm_got, q, c, b, h, tau, lengths[b], f"noalloc c={c} b={b} h={h} tau={tau}")
    # a call too large for the fixed array is refused before anything is enqueued
    big = torch.zeros((4, 64, 4, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(lkv.LoopKVError) as e:
        wl.ctx.decode(big, torch.zeros((64, 2048), dtype=torch.int32, device="cuda"),
                      torch.ones(64, dtype=torch.int32, device="cuda"), 32768, 0.01, n_split=2, no_alloc=True)
    assert e.value.status == B.ERR_WORKSPACE
    # second call: one cell, the first two sequences, a shorter max_len, 3 splits
    lens2 = wl.seq_lens[:2].clone()
    bt2 = wl.bt[:2].contiguous()
    q2 = q[3, :2].contiguous()
    ref2, s2r = wl.ctx.decode(q2, bt2, lens2, 1500, 0.01, cell=(1, 1), sel_mask=True, n_split=3)
    got2, s2g = wl.ctx.decode(q2, bt2, lens2, 1500, 0.01, cell=(1, 1), sel_mask=True, n_split=3, no_alloc=True)
    torch.cuda.synchronize()
    assert torch.equal(got2, ref2) and torch.equal(s2g, s2r), "second, smaller call"
    full, fsm = wl.decode(q, 0.01)
    torch.cuda.synchronize()
    for b in range(2):
        for h in range(4):
            check_row(wl, full, fsm, q, 3, b, h, 0.01, lengths[b], f"one-workgroup b={b} h={h}")
    assert (got2 - full[3, :2]).abs().max().item() <= 2e-3 * full[3, :2].abs().max().item()
