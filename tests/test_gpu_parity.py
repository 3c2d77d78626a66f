"""GPU parity of the HIP path against the fp64 oracle, through the C ABI.

Bars: packed codes, scales/zeros, tails and the selected-token set are
bit-exact (selection excuses only tokens whose oracle coarse weight lies within
1e-5 of tau); outputs accumulated in fp32 are within 2e-3 max relative error
(max |o - ref| / max |ref| over the row). Method: "LoopKV: Loop-Aware KV Cache
Compression for Serving Looped Transformers" (arXiv:2611.04137), Abstract.
"""
import math

import numpy as np
import pytest
import torch

import quantized_kv_cache_loopkv_amd as lkv
from oracle import loopkv_oracle as O
from synth import recipes as R
from synth.philox import f32_to_bf16_bits
from tests.harness import Workload, kv_head, oracle_row_inputs, rel_err, sel_bits_from_mask

pytestmark = pytest.mark.gpu

TOL = 2e-3
TIE = 1e-5


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def check_row(wl: Workload, out, sm, q, cell, b, h, tau, n_tokens, label="", inputs=None):
    """Compare one row of a decode call with the oracle. Returns the relative error.
    inputs: optional (K, V, qh) of the row's storage (qh: the oracle's quantized history, or
    None), so that one row can be checked at several tau without drawing it again."""
    cfg = wl.cfg
    st = O.storage_cell(wl.plan.reshape(cfg.n_loops, cfg.n_layers), cell)
    kind = O.target_kind(wl.plan.reshape(cfg.n_loops, cfg.n_layers), cell)
    if wl.layout == lkv.LAYOUT_KIVI4:
        kind = "kivi4"
    if inputs is None:
        _, _, K, V = oracle_row_inputs(cfg, st, b, kv_head(cfg, h), n_tokens, wl.factors)
        qh = None
    else:
        K, V, qh = inputs
    qv = q[cell, b, h].float().cpu().numpy().astype(np.float64)
    sig = np.float32(1.0 / math.sqrt(cfg.head_dim))
    G = cfg.group
    o_ref, sel_ref, phat = O.decode_row(qv, K, V, kind, tau, float(sig), qh=qh, group=G)
    n_q = G * (n_tokens // G)
    o_gpu = out[cell, b, h].float().cpu().numpy()
    sel_gpu = sel_bits_from_mask(sm[cell, b, h].cpu().numpy(), n_q)
    if kind == "kivi4" or (kind == O.KIND_Q4 and tau == 0.0):
        assert sel_gpu.all(), label
    elif kind == O.KIND_Q2 or tau > 1.0:
        assert not sel_gpu.any(), label
    else:
        excused = np.abs(phat[:n_q] - tau) <= TIE
        bad = (sel_gpu != sel_ref) & ~excused
        assert not bad.any(), f"{label}: selection differs at {np.flatnonzero(bad)[:10]}"
        if (sel_gpu != sel_ref).any():
            o_ref, _, _ = O.decode_row(qv, K, V, kind, tau, float(sig), qh=qh, sel_override=sel_gpu, group=G)
    err = rel_err(o_gpu, o_ref)
    assert err <= TOL, f"{label}: rel err {err:.3e}"
    return err


# --------------------------------------------------------------------------- generator
def test_gpu_synth_matches_host():
    _need_gpu()
    from synth import gpu as G
    cfg = R.make_config("C2")
    f = R.factor_table(cfg)
    K = torch.empty((cfg.batch, 40, cfg.n_heads, cfg.head_dim), dtype=torch.bfloat16, device="cuda")
    G.kv_bf16(cfg.seed, 1, cfg.batch, 40, 100, cfg.token_stride, cfg.n_heads, cfg.head_dim,
              torch.from_numpy(f[0, 0]).cuda(), K)
    kb, _ = R.kv_tensor_bits(cfg, 0, 100, 140, f)
    got = K.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, kb)
    q = torch.empty((cfg.batch, cfg.n_heads, cfg.head_dim), dtype=torch.bfloat16, device="cuda")
    G.normal(cfg.seed, 3, 2 * q.numel(), q)
    want = R.q_values(cfg, 0, 2)
    assert np.array_equal(q.float().cpu().numpy(), want)


# --------------------------------------------------------------------------- quantize + pack
@pytest.mark.parametrize("layout,plan", [(lkv.LAYOUT_PLANES, [0]), (lkv.LAYOUT_PLANES, [1]), (lkv.LAYOUT_KIVI4, [0])])
@pytest.mark.parametrize("D", [64, 128, 256])
def test_gpu_records_bit_exact(layout, plan, D):
    _need_gpu()
    lengths = [1, 31, 32, 33, 100, 257]
    cfg = R.small_config("rec", 1, 1, 3, D, lengths, [0.01], plan=plan, outlier_count=3, outlier_mult=10.0,
                         shuffled=True)
    wl = Workload(cfg, layout=layout, gpu_synth=False)
    wl.fill()
    bits = 2 if plan[0] == 1 else 4
    for b, N in enumerate(lengths):
        for h in range(cfg.n_heads):
            kb, vb, K, V = oracle_row_inputs(cfg, 0, b, h, N, wl.factors)
            qh = O.quantize_history(K, V, bits)
            for j in range(qh["n_q"] // 16):
                want = O.pack_block(qh, j, layout)
                got = wl.record(0, b, h, j)
                assert np.array_equal(got, want), f"record b={b} h={h} j={j}"
            n_q, tk, tv = O.tail_tokens(kb, vb)
            tail = wl.tail(0, b, h)
            for i in range(N - n_q):
                p = n_q + i
                assert np.array_equal(tail[0, p % 32], tk[i]) and np.array_equal(tail[1, p % 32], tv[i])


def test_gpu_bulk_equals_incremental_append():
    """P10: one bulk append and token-by-token appends give identical records and tails."""
    _need_gpu()
    lengths = [70, 70]
    cfg = R.small_config("inc", 1, 1, 2, 64, lengths, [0.01], shuffled=True)
    a = Workload(cfg, gpu_synth=False)
    a.fill()
    b_ = Workload(cfg, gpu_synth=False)
    K, V = b_.kv_chunk(0, 0, 70)
    for t in range(0, 70, 1 if False else 7):
        n = min(7, 70 - t)
        lens = torch.full((2,), t, dtype=torch.int32, device="cuda")
        b_.ctx.append(K[:, t:t + n].contiguous(), V[:, t:t + n].contiguous(), b_.bt, lens, cell=(0, 0))
    c = Workload(cfg, gpu_synth=False)
    for t in range(70):
        lens = torch.full((2,), t, dtype=torch.int32, device="cuda")
        c.ctx.append(K[:, t:t + 1].contiguous(), V[:, t:t + 1].contiguous(), c.bt, lens, cell=(0, 0))
    torch.cuda.synchronize()
    for other in (b_, c):
        for bb in range(2):
            for h in range(2):
                for j in range(4):
                    assert np.array_equal(a.record(0, bb, h, j), other.record(0, bb, h, j))
                ta, to = a.tail(0, bb, h), other.tail(0, bb, h)
                assert np.array_equal(ta[:, :6], to[:, :6])


def test_gpu_f32_input_rounds_to_bf16():
    _need_gpu()
    cfg = R.small_config("f32", 1, 1, 2, 64, [64], [0.01])
    a = Workload(cfg, gpu_synth=False)
    a.fill()
    b_ = Workload(cfg, gpu_synth=False)
    K, V = b_.kv_chunk(0, 0, 64)
    # add sub-bf16 noise that rounds away
    Kf = K.float() * (1 + 2 ** -12)
    Vf = V.float()
    lens = torch.zeros(1, dtype=torch.int32, device="cuda")
    b_.ctx.append(Kf.contiguous(), Vf.contiguous(), b_.bt, lens, cell=(0, 0))
    torch.cuda.synchronize()
    for h in range(2):
        for j in range(4):
            assert np.array_equal(a.record(0, 0, h, j), b_.record(0, 0, h, j))


@pytest.mark.gpu
def test_gpu_append_unaligned_input_same_records():
    """K and V whose data start 2 bytes past a 16-byte boundary take the element-wise gathers of
    the append kernels (aligned bf16 inputs take 16-byte loads): the same records and tails, for a
    bulk append and for one-token appends that complete a group."""
    _need_gpu()
    cfg = R.small_config("unal", 1, 1, 2, 128, [70], [0.01])
    a = Workload(cfg, gpu_synth=False)
    a.fill()
    b_ = Workload(cfg, gpu_synth=False)
    K, V = b_.kv_chunk(0, 0, 70)

    def shifted(x):
        buf = torch.empty(x.numel() + 8, dtype=x.dtype, device=x.device)
        y = buf[1:1 + x.numel()].view(x.shape)
        y.copy_(x)
        assert y.data_ptr() % 16 == 2 and y.is_contiguous()
        return y

    lens = torch.zeros(1, dtype=torch.int32, device="cuda")
    b_.ctx.append(shifted(K[:, :63].contiguous()), shifted(V[:, :63].contiguous()), b_.bt, lens, cell=(0, 0))
    for t in range(63, 70):   # token 63 completes group 1 through the one-token kernel
        lens = torch.full((1,), t, dtype=torch.int32, device="cuda")
        b_.ctx.append(shifted(K[:, t:t + 1].contiguous()), shifted(V[:, t:t + 1].contiguous()), b_.bt, lens,
                      cell=(0, 0))
    torch.cuda.synchronize()
    for h in range(2):
        for j in range(4):
            assert np.array_equal(a.record(0, 0, h, j), b_.record(0, 0, h, j)), f"record h={h} j={j}"
        assert np.array_equal(a.tail(0, 0, h)[:, :6], b_.tail(0, 0, h)[:, :6])


# --------------------------------------------------------------------------- decode
def test_gpu_decode_c1():
    _need_gpu()
    cfg = R.make_config("C1")
    wl = Workload(cfg, gpu_synth=False)
    wl.fill()
    q = wl.q_all()
    out, sm = wl.decode(q, 0.01)
    out_b, sm_b = wl.decode(q, 0.01, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    for h in range(2):
        check_row(wl, out, sm, q, 0, 0, h, 0.01, 256, f"C1 h={h}")
    # bf16 output is the nearest-even rounding of the fp32 output of the same computation
    want = f32_to_bf16_bits(out.cpu().numpy())
    got = out_b.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, want)
    assert torch.equal(sm, sm_b)


@pytest.mark.parametrize("tau", [0.0, 0.001, 0.01, 0.2, 1.1])
@pytest.mark.parametrize("D", [64, 128, 256])
def test_gpu_decode_ragged_tau_sweep(tau, D):
    _need_gpu()
    lengths = [1, 2, 31, 32, 33, 95, 96, 97, 640, 1000, 2049]
    cfg = R.small_config("rag", 1, 1, 2, D, lengths, [tau], outlier_count=3, outlier_mult=10.0, shuffled=True)
    wl = Workload(cfg, gpu_synth=False)
    wl.fill()
    q = wl.q_all() * 3  # sharpen the attention so that selections are non-trivial
    q = q.to(torch.bfloat16).float().to(q.dtype)
    out, sm = wl.decode(q, tau)
    torch.cuda.synchronize()
    for b, N in enumerate(lengths):
        for h in range(2):
            check_row(wl, out, sm, q, 0, b, h, tau, N, f"b={b} N={N} h={h} tau={tau}")


def test_gpu_decode_whole_plan_small():
    """Mixed plan with 4-bit, 2-bit and reuse cells; whole-plan call == per-cell calls (bitwise);
    a reuse cell equals the final-loop cell for the same query (P3, bitwise)."""
    _need_gpu()
    plan = np.array([[0, 2, 1], [2, 0, 0], [0, 1, 0]], dtype=np.uint8)
    lengths = [300, 64, 517]
    cfg = R.small_config("plan", 3, 3, 2, 128, lengths, [0.01], plan=plan, cell_scales=True, shuffled=True)
    wl = Workload(cfg, gpu_synth=False)
    wl.fill()
    q = wl.q_all()
    for tau in (0.0, 0.01, 1.1):
        out, sm = wl.decode(q, tau)
        for c in range(9):
            for b, N in enumerate(lengths):
                for h in range(2):
                    check_row(wl, out, sm, q, c, b, h, tau, N, f"cell={c} b={b} h={h} tau={tau}")
        for c in range(9):
            loop, layer = divmod(c, 3)
            o1, s1 = wl.decode(q, tau, cell=(loop, layer))
            assert torch.equal(o1, out[c]) and torch.equal(s1, sm[c])
        # P3: reuse cell with the final loop's query
        q2 = q.clone()
        for c in (1, 3):
            q2[c] = q[6 + c % 3]
        out2, sm2 = wl.decode(q2, tau)
        for c in (1, 3):
            assert torch.equal(out2[c], out2[6 + c % 3]) and torch.equal(sm2[c], sm2[6 + c % 3])


@pytest.mark.parametrize("D", [64, 128, 256])
def test_gpu_kivi4_equals_planes_tau0(D):
    """P12: the KIVI-4 layout matches the planes layout at tau = 0 (same codes, same selection)."""
    _need_gpu()
    lengths = [333, 1024]
    cfg = R.small_config("k4", 1, 1, 4, D, lengths, [0.0], outlier_count=3, outlier_mult=10.0)
    a = Workload(cfg, gpu_synth=False)
    a.fill()
    k = Workload(cfg, layout=lkv.LAYOUT_KIVI4, gpu_synth=False)
    k.fill()
    q = a.q_all()
    oa, sa = a.decode(q, 0.0)
    ok_, sk = k.decode(q, 0.37)
    torch.cuda.synchronize()
    assert torch.equal(sa, sk)
    # Same codes, scales and selection; the two layouts read their 4-bit codes from different
    # words (one 4-bit plane vs two 2-bit planes) and sum in a different order, so the outputs
    # agree to the parity bar rather than bit for bit (typically ~1e-7).
    d = rel_err(ok_.cpu().numpy(), oa.cpu().numpy())
    print(f"kivi vs planes rel diff {d:.3e}", flush=True)
    assert d < TOL
    for b, N in enumerate(lengths):
        for h in range(4):
            check_row(k, ok_, sk, q, 0, b, h, 0.37, N, f"kivi b={b} h={h}")


def test_gpu_paging_invariance():
    """P9: identity vs shuffled block table give bitwise-identical outputs and records."""
    _need_gpu()
    lengths = [500, 77]
    c1 = R.small_config("id", 1, 1, 2, 128, lengths, [0.01], shuffled=False)
    c2 = R.small_config("sh", 1, 1, 2, 128, lengths, [0.01], shuffled=True)
    a, b_ = Workload(c1, gpu_synth=False), Workload(c2, gpu_synth=False)
    a.fill()
    b_.fill()
    q = a.q_all()
    for tau in (0.0, 0.005, 1.1):
        oa, sa = a.decode(q, tau)
        ob, sb = b_.decode(q, tau)
        assert torch.equal(oa, ob) and torch.equal(sa, sb)
    for bb, N in enumerate(lengths):
        for j in range(32 * (N // 32) // 16):
            assert np.array_equal(a.record(0, bb, 1, j), b_.record(0, bb, 1, j))


def test_gpu_edge_lengths():
    """Empty rows give zeros, rows longer than max_len give NaN, one token gives v exactly."""
    _need_gpu()
    cfg = R.small_config("edge", 1, 1, 2, 64, [1, 40], [0.01])
    wl = Workload(cfg, gpu_synth=False)
    wl.fill()
    q = wl.q_all()
    lens = torch.tensor([1, 0], dtype=torch.int32, device="cuda")
    out = wl.ctx.decode(q[0], wl.bt, lens, 40, 0.01, cell=(0, 0))
    torch.cuda.synchronize()
    kb, vb = R.kv_row_bits(cfg, 0, 0, 0, 0, 1, wl.factors)
    from synth.philox import bf16_bits_to_f32
    assert np.array_equal(out[0, 0].cpu().numpy(), bf16_bits_to_f32(vb[0]))
    assert torch.all(out[1] == 0)
    lens = torch.tensor([1, 40], dtype=torch.int32, device="cuda")
    out = wl.ctx.decode(q[0], wl.bt, lens, 33, 0.01, cell=(0, 0))
    torch.cuda.synchronize()
    assert torch.isnan(out[1]).all() and not torch.isnan(out[0]).any()


def test_gpu_c2_full():
    """C2 (16 heads x 128, batch 8, 4096 tokens, tau 0.005), every row against the oracle,
    and the same cell in the KIVI-4 layout."""
    _need_gpu()
    cfg = R.make_config("C2")
    wl = Workload(cfg, gpu_synth=True)
    wl.fill()
    q = wl.q_all()
    out, sm = wl.decode(q, 0.005)
    torch.cuda.synchronize()
    errs = []
    for b in range(cfg.batch):
        for h in range(cfg.n_heads):
            errs.append(check_row(wl, out, sm, q, 0, b, h, 0.005, 4096, f"C2 b={b} h={h}"))
    print(f"C2 max rel err {max(errs):.2e}, mean selected per row "
          f"{np.unpackbits(sm.cpu().numpy().view(np.uint8)).sum() / (cfg.batch * cfg.n_heads):.1f}")
    k = Workload(cfg, layout=lkv.LAYOUT_KIVI4, gpu_synth=True)
    k.fill()
    ok_, sk = k.decode(q, 0.005)
    torch.cuda.synchronize()
    for b in range(0, cfg.batch, 3):
        for h in range(0, cfg.n_heads, 5):
            check_row(k, ok_, sk, q, 0, b, h, 0.005, 4096, f"C2-kivi b={b} h={h}")
