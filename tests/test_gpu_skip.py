"""The token-skipping ablation (loopkv_decode_attn_skip) on the GPU.

"LoopKV: Loop-Aware KV Cache Compression for Serving Looped Transformers" (arXiv:2611.04137),
Abstract, sentence on skipping: leaving out the values of weakly attended tokens saves reads
but its error grows from loop to loop, so the method reads the unselected tokens at 2 bits
instead of leaving them out.

* rows of the skip kernel match the oracle's skip mode (selection bit-exact outside the 1e-5
  tie band, output within 2e-3), over tau regimes, head dims, ragged lengths and a mixed plan;
* a synthetic looped chain (one shared block applied over 4 loops, a separate cache per loop)
  run through the kernels: the hidden state's error against the exact chain, per loop, for the
  method and for skipping. Skipping's error is far larger and grows across the loops.
"""
import math

import numpy as np
import pytest
import torch

import quantized_kv_cache_loopkv_amd as lkv
from oracle import loopkv_oracle as O
from synth import recipes as R
from tests.harness import Workload, kv_head, oracle_row_inputs, rel_err, sel_bits_from_mask
from tests.test_gpu_parity import TIE, TOL

pytestmark = pytest.mark.gpu


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _check_skip_row(wl, out, sm, q, cell, b, h, tau, n_tokens, label):
    cfg = wl.cfg
    plan = wl.plan.reshape(cfg.n_loops, cfg.n_layers)
    st = O.storage_cell(plan, cell)
    kind = O.target_kind(plan, cell)
    _, _, K, V = oracle_row_inputs(cfg, st, b, kv_head(cfg, h), n_tokens, wl.factors)
    qv = q[cell, b, h].float().cpu().numpy().astype(np.float64)
    sig = float(np.float32(1.0 / math.sqrt(cfg.head_dim)))
    skip = kind == O.KIND_Q4
    G = cfg.group
    o_ref, sel_ref, phat = O.decode_row(qv, K, V, kind, tau, sig, skip=skip, group=G)
    n_q = G * (n_tokens // G)
    o_gpu = out[cell, b, h].float().cpu().numpy()
    sel_gpu = sel_bits_from_mask(sm[cell, b, h].cpu().numpy(), n_q)
    if kind == O.KIND_Q4 and tau > 0:
        excused = np.abs(phat[:n_q] - tau) <= TIE
        bad = (sel_gpu != sel_ref) & ~excused
        assert not bad.any(), f"{label}: selection differs at {np.flatnonzero(bad)[:10]}"
        if (sel_gpu != sel_ref).any():
            o_ref, _, _ = O.decode_row(qv, K, V, kind, tau, sig, sel_override=sel_gpu, skip=True, group=G)
    if not np.any(o_ref):
        assert not np.any(o_gpu), f"{label}: nothing kept, output must be 0"
        return 0.0
    err = rel_err(o_gpu, o_ref)
    assert err <= TOL, f"{label}: rel err {err:.3e}"
    return err


@pytest.mark.parametrize("tau", [0.0, 0.003, 0.02, 1.5])
@pytest.mark.parametrize("D", [64, 128, 256])
def test_gpu_skip_rows(tau, D):
    _need_gpu()
    lengths = [1, 31, 32, 33, 96, 640, 1000, 2049]
    cfg = R.small_config("skip", 1, 1, 2, D, lengths, [tau], outlier_count=3, outlier_mult=10.0, shuffled=True)
    wl = Workload(cfg, gpu_synth=False)
    wl.fill()
    q = wl.q_all() * 3
    q = q.to(torch.bfloat16).float().to(q.dtype)
    out, sm = wl.ctx.decode(q, wl.bt, wl.seq_lens, wl.max_len(), tau, sel_mask=True, skip=True)
    torch.cuda.synchronize()
    for b, N in enumerate(lengths):
        for h in range(2):
            _check_skip_row(wl, out, sm, q, 0, b, h, tau, N, f"skip b={b} N={N} h={h} tau={tau}")


def test_gpu_skip_mixed_plan():
    """4-bit, 2-bit and reuse cells: 4-bit targets skip, 2-bit targets decode as the method."""
    _need_gpu()
    plan = np.array([[0, 2, 1], [2, 0, 0], [0, 1, 0]], dtype=np.uint8)
    lengths = [300, 64, 517]
    cfg = R.small_config("skplan", 3, 3, 2, 128, lengths, [0.01], plan=plan, cell_scales=True, shuffled=True)
    wl = Workload(cfg, gpu_synth=False)
    wl.fill()
    q = wl.q_all() * 2
    out, sm = wl.ctx.decode(q, wl.bt, wl.seq_lens, wl.max_len(), 0.01, sel_mask=True, skip=True)
    torch.cuda.synchronize()
    for c in range(9):
        for b, N in enumerate(lengths):
            for h in range(2):
                _check_skip_row(wl, out, sm, q, c, b, h, 0.01, N, f"cell={c} b={b} h={h}")


def test_gpu_skip_rejected_with_kivi4():
    _need_gpu()
    cfg = R.small_config("skk", 1, 1, 2, 64, [64], [0.01])
    k = Workload(cfg, layout=lkv.LAYOUT_KIVI4, gpu_synth=False)
    with pytest.raises(lkv.LoopKVError) as e:
        k.ctx.decode(k.q_all(), k.bt, k.seq_lens, 64, 0.01, skip=True)
    assert e.value.status == lkv.loopkv.ERR_UNSUPPORTED


def looped_chain(n_loops=4, B=2, H=4, D=128, N=4090, tau=0.01, q_gain=1.0, seed=1):
    """A shared attention block applied n_loops times, each loop with its own cache (one cell
    per loop): h <- h + W_o attn(W_q h, cache_loop). Runs the exact chain (fp64 over the bf16
    history) and the chains of the method and of skipping (the decode kernels; projections in
    fp64 on the host). Returns per-loop relative errors of h for each, plus each loop's error
    when fed the exact hidden state (no compounding)."""
    plan = np.zeros((n_loops, 1), dtype=np.uint8)
    cfg = R.small_config("chain", n_loops, 1, H, D, [N] * B, [tau], plan=plan, shuffled=True, seed=seed)
    wl = Workload(cfg, gpu_synth=False)
    wl.fill()
    rng = np.random.default_rng(seed)
    dm = H * D
    Wq = rng.standard_normal((dm, dm)) * (q_gain / math.sqrt(dm))
    Wo = rng.standard_normal((dm, dm)) * (1.0 / math.sqrt(dm))
    h0 = rng.standard_normal((B, dm))
    sig = float(np.float32(1.0 / math.sqrt(D)))
    hist = {(i, b): [oracle_row_inputs(cfg, i, b, hh, N, wl.factors)[2:] for hh in range(H)]
            for i in range(n_loops) for b in range(B)}

    def q_of(h):   # [B][dm] -> fp32 [B][H][D] (what the kernel and the reference both use)
        return (h @ Wq.T).reshape(B, H, D).astype(np.float32)

    def exact_attn(i, q):
        o = np.zeros((B, H, D))
        for b in range(B):
            for hh in range(H):
                K, V = hist[(i, b)][hh]
                o[b, hh] = O.attention_reference(q[b, hh].astype(np.float64), K, V, sig)
        return o

    def kernel_attn(i, q, skip):
        qd = torch.from_numpy(q).cuda().contiguous()
        out = wl.ctx.decode(qd, wl.bt, wl.seq_lens, N, tau, cell=(i, 0), skip=skip)
        torch.cuda.synchronize()
        return out.cpu().numpy().astype(np.float64)

    h_ex = [h0]
    for i in range(n_loops):
        h_ex.append(h_ex[-1] + exact_attn(i, q_of(h_ex[-1])).reshape(B, dm) @ Wo.T)
    res = {}
    for name, skip in (("method", False), ("skip", True)):
        h = h0
        chained, single = [], []
        for i in range(n_loops):
            o = kernel_attn(i, q_of(h), skip)
            h = h + o.reshape(B, dm) @ Wo.T
            chained.append(float(np.linalg.norm(h - h_ex[i + 1]) / np.linalg.norm(h_ex[i + 1])))
            o1 = kernel_attn(i, q_of(h_ex[i]), skip)   # this loop alone, from the exact state
            h1 = h_ex[i] + o1.reshape(B, dm) @ Wo.T
            single.append(float(np.linalg.norm(h1 - h_ex[i + 1]) / np.linalg.norm(h_ex[i + 1])))
        res[name] = {"chained": chained, "single_loop": single}
    return res


def test_gpu_skipping_errors_compound_across_loops():
    """Scores of unit scale (q gain 1, no outlier channels), tau 0.01, 4090-token caches: the
    method's error stays at the quantizer's few percent while skipping's grows loop by loop."""
    _need_gpu()
    res = looped_chain()
    for name, r in res.items():
        print(name, "chained:", " ".join(f"{e:.2e}" for e in r["chained"]),
              "| single loop:", " ".join(f"{e:.2e}" for e in r["single_loop"]), flush=True)
    m, s = res["method"]["chained"], res["skip"]["chained"]
    assert s[-1] > 10 * m[-1]            # skipping is far less accurate than 2-bit reads
    assert s[-1] > s[0]                  # and its error grows across the loops
    assert s[-1] > max(res["skip"]["single_loop"])   # beyond what any single loop adds
