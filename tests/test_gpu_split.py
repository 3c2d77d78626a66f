"""The split decode (loopkv_decode_attn_split): each row's tokens streamed by n_split
workgroups, then one finishing launch per row that merges the partials, selects over the
whole row and corrects the selected tokens.

Every row is checked against the fp64 oracle at the parity bar (selection bit-exact outside
the 1e-5 tie band, output within 2e-3), across the tau regimes, both layouts, 2-bit and reuse
cells, ragged lengths (rows with only a tail, rows shorter than one split's share, more splits
than chunks) and the corrections' cancellation guard. Method: "LoopKV: Loop-Aware KV Cache
Compression for Serving Looped Transformers" (arXiv:2611.04137), Abstract (decoding sentence).
"""
import numpy as np
import pytest
import torch

import quantized_kv_cache_loopkv_amd as lkv
from synth import recipes as R
from synth.philox import f32_to_bf16_bits
from tests.harness import Workload, rel_err
from tests.test_gpu_parity import TOL, check_row

pytestmark = pytest.mark.gpu


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _split(wl, q, tau, n_split, cell=None, out_dtype=torch.float32, max_len=None):
    qq = q if cell is None else q[cell[0] * wl.cfg.n_layers + cell[1]].contiguous()
    ml = wl.max_len() if max_len is None else max_len
    return wl.ctx.decode(qq, wl.bt, wl.seq_lens, ml, tau, cell=cell, out_dtype=out_dtype, sel_mask=True,
                         n_split=n_split)


@pytest.mark.parametrize("tau", [0.0, 0.001, 0.01, 1.1])
@pytest.mark.parametrize("D", [64, 128, 256])
def test_gpu_split_ragged(tau, D):
    _need_gpu()
    lengths = [1, 31, 32, 33, 97, 640, 1000, 2049]
    cfg = R.small_config("srag", 1, 1, 2, D, lengths, [tau], outlier_count=3, outlier_mult=10.0, shuffled=True)
    wl = Workload(cfg, gpu_synth=False)
    wl.fill()
    q = wl.q_all() * 3
    q = q.to(torch.bfloat16).float().to(q.dtype)
    o1, s1 = wl.decode(q, tau)
    for n_split in (1, 3, 8, 64):
        print(f"D={D} tau={tau} n_split={n_split}", flush=True)
        out, sm = _split(wl, q, tau, n_split)
        torch.cuda.synchronize()
        for b, N in enumerate(lengths):
            for h in range(2):
                check_row(wl, out, sm, q, 0, b, h, tau, N, f"split={n_split} b={b} N={N} h={h} tau={tau}")
        # same coarse scores and codes as the one-workgroup decode; only fp32 summation order differs
        assert rel_err(out.cpu().numpy(), o1.cpu().numpy()) < TOL


def test_gpu_split_whole_plan_and_cells():
    """Mixed 4-bit / 2-bit / reuse plan: a whole-plan split call equals per-cell split calls
    bit for bit (rows are independent), and every row matches the oracle."""
    _need_gpu()
    plan = np.array([[0, 2, 1], [2, 0, 0], [0, 1, 0]], dtype=np.uint8)
    lengths = [300, 64, 517]
    cfg = R.small_config("splan", 3, 3, 2, 128, lengths, [0.01], plan=plan, cell_scales=True, shuffled=True)
    wl = Workload(cfg, gpu_synth=False)
    wl.fill()
    q = wl.q_all()
    for tau in (0.0, 0.01, 1.1):
        out, sm = _split(wl, q, tau, 5)
        torch.cuda.synchronize()
        for c in range(9):
            for b, N in enumerate(lengths):
                for h in range(2):
                    check_row(wl, out, sm, q, c, b, h, tau, N, f"cell={c} b={b} h={h} tau={tau}")
        for c in range(9):
            o1, s1 = _split(wl, q, tau, 5, cell=divmod(c, 3))
            assert torch.equal(o1, out[c]) and torch.equal(s1, sm[c])


def test_gpu_split_kivi4_and_bf16_output():
    _need_gpu()
    lengths = [333, 1024, 40]
    cfg = R.small_config("sk4", 1, 1, 4, 128, lengths, [0.0], outlier_count=3, outlier_mult=10.0)
    k = Workload(cfg, layout=lkv.LAYOUT_KIVI4, gpu_synth=False)
    k.fill()
    q = k.q_all()
    out, sm = _split(k, q, 0.37, 6)
    ob, smb = _split(k, q, 0.37, 6, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    for b, N in enumerate(lengths):
        for h in range(4):
            check_row(k, out, sm, q, 0, b, h, 0.37, N, f"kivi split b={b} h={h}")
    assert np.array_equal(ob.view(torch.int16).cpu().numpy().view(np.uint16), f32_to_bf16_bits(out.cpu().numpy()))
    assert torch.equal(sm, smb)


def test_gpu_split_edge_lengths():
    """Empty rows give zeros and rows longer than max_len give NaN, as in the one-workgroup decode."""
    _need_gpu()
    cfg = R.small_config("sedge", 1, 1, 2, 64, [1, 40, 200], [0.01])
    wl = Workload(cfg, gpu_synth=False)
    wl.fill()
    q = wl.q_all()[0].contiguous()
    lens = torch.tensor([1, 0, 200], dtype=torch.int32, device="cuda")
    a = wl.ctx.decode(q, wl.bt, lens, 200, 0.01, cell=(0, 0))
    s = wl.ctx.decode(q, wl.bt, lens, 200, 0.01, cell=(0, 0), n_split=4)
    torch.cuda.synchronize()
    assert torch.all(s[1] == 0)
    assert rel_err(s[0].cpu().numpy(), a[0].cpu().numpy()) == 0.0   # one token: v itself
    assert rel_err(s[2].cpu().numpy(), a[2].cpu().numpy()) < TOL
    lens = torch.tensor([1, 40, 300], dtype=torch.int32, device="cuda")
    s = wl.ctx.decode(q, wl.bt, lens, 200, 0.01, cell=(0, 0), n_split=4)
    torch.cuda.synchronize()
    assert torch.isnan(s[2]).all() and not torch.isnan(s[0]).any() and not torch.isnan(s[1]).any()


@pytest.mark.parametrize("mode", ["drop", "rise"])
def test_gpu_split_corrections(mode):
    """The crafted rows of the correction tests (a coarse winner whose low bits move its score by
    ~13 nats either way) through the split decode: the finishing launch's corrections and its
    cancellation guard."""
    _need_gpu()
    from tests.test_gpu_corrections import _winner_row, _check
    K, V, q = _winner_row(128, 512 + 7, mode, seed=11)
    for n_split in (1, 3):
        err, n_sel = _check(K, V, q, 0.01, f"split={n_split} {mode}", n_split=n_split)
        assert n_sel >= 1
