"""Full-size configurations on the GPU, checked row by row against the fp64 oracle on sampled rows.

* C3: 4 loops x 24 layers (48 4-bit / 29 2-bit / 19 reuse), 16 heads x 128, batch 32,
  8192 tokens, identity block table, tau in {0, 0.001, 0.01, 1.1}.
* C4: the same plan at 16384 tokens with a shuffled block table (the benchmarked
  workload), tau in {0, 0.001, 0.01, 1.1}, plus the bf16 output of the same launch.
* C5: batch 128, lengths uniform in [1024, 16384], shuffled table, 40 decode steps each
  preceded by a one-token append to every storing cell; tau 0.01.

The same bars as the small tests: selection bit-exact outside the 1e-5 tie band,
outputs within 2e-3 (max |o - ref| / max |ref| per row), records bit-exact.
"""
import numpy as np
import pytest
import torch

import quantized_kv_cache_loopkv_amd as lkv
from oracle import loopkv_oracle as O
from synth import recipes as R
from synth.philox import f32_to_bf16_bits
from tests.harness import Workload, kv_head, oracle_row_inputs
from tests.test_gpu_parity import check_row

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def _log(*a):
    print(*a, flush=True)


def _sample_rows(cfg, n_per_kind=2):
    plan = cfg.plan.reshape(-1)
    rows = []
    for kind in (R.Q4, R.Q2, R.SHARE):
        cells = [c for c in range(cfg.n_cells) if plan[c] == kind][:n_per_kind]
        for i, c in enumerate(cells):
            b = (7 * c + 3 * i) % cfg.batch
            h = (5 * c + i) % cfg.n_heads
            rows.append((c, b, h))
    rows.append((cfg.n_cells - 1, cfg.batch - 1, cfg.n_heads - 1))
    return rows


def _check_records(wl, cell, b, h, n_tokens, blocks):
    cfg = wl.cfg
    st = O.storage_cell(cfg.plan, cell)
    bits = 2 if cfg.plan.reshape(-1)[st] == R.Q2 else 4
    _, _, K, V = oracle_row_inputs(cfg, st, b, kv_head(cfg, h), n_tokens, wl.factors)
    qh = O.quantize_history(K, V, bits)
    for j in blocks:
        if 16 * (j + 1) <= qh["n_q"]:
            assert np.array_equal(wl.record(cell, b, h, j), O.pack_block(qh, j)), f"record {cell},{b},{h},{j}"


def _run_sweep(wl, rows, taus, n_tokens_of):
    q = wl.q_all()
    for tau in taus:
        out, sm = wl.decode(q, tau)
        torch.cuda.synchronize()
        errs = [check_row(wl, out, sm, q, c, b, h, tau, n_tokens_of(b), f"{wl.cfg.name} c={c} b={b} h={h} tau={tau}")
                for (c, b, h) in rows]
        _log(f"{wl.cfg.name} tau={tau}: max rel err {max(errs):.2e} over {len(rows)} rows")
    return q


def test_c3_sampled_rows():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cfg = R.make_config("C3")
    wl = Workload(cfg, gpu_synth=True, log=_log)
    wl.fill()
    rows = _sample_rows(cfg)
    _run_sweep(wl, rows, cfg.taus, lambda b: cfg.lengths[b])
    for (c, b, h) in rows[:3]:
        _check_records(wl, c, b, h, cfg.lengths[b], [0, 1, 255, 511])
    del wl
    torch.cuda.empty_cache()


def test_c4_sampled_rows_and_bf16_output():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cfg = R.make_config("C4")
    wl = Workload(cfg, gpu_synth=True, log=_log)
    wl.fill()
    rows = _sample_rows(cfg)
    q = _run_sweep(wl, rows, cfg.taus, lambda b: cfg.lengths[b])
    # the benchmarked launch writes bf16: nearest-even rounding of the fp32 result of the same launch
    out32, sm32 = wl.decode(q, 0.01)
    out16, sm16 = wl.decode(q, 0.01, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(sm32, sm16)
    for (c, b, h) in rows:
        want = f32_to_bf16_bits(out32[c, b, h].cpu().numpy())
        got = out16[c, b, h].view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(got, want)
    for (c, b, h) in rows[:3]:
        _check_records(wl, c, b, h, cfg.lengths[b], [0, 3, 1000, 1023])
    del wl
    torch.cuda.empty_cache()


def test_c5_mixed_lengths_with_appends():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cfg = R.make_config("C5")
    steps = 40
    cfg.append_steps = steps   # token indexing stride covers the appended tokens
    wl = Workload(cfg, gpu_synth=True, log=_log)
    wl.fill()
    _log("C5 filled")
    for s in range(steps):
        wl.append_step(s)
    torch.cuda.synchronize()
    _log(f"C5 appended {steps} tokens per sequence")
    rows = _sample_rows(cfg)
    final = [n + steps for n in cfg.lengths]
    wl.seq_lens = torch.tensor(final, dtype=torch.int32, device="cuda")
    q = wl.q_all(step=steps)
    out, sm = wl.ctx.decode(q, wl.bt, wl.seq_lens, max(final), 0.01, out_dtype=torch.float32, sel_mask=True)
    torch.cuda.synchronize()
    errs = [check_row(wl, out, sm, q, c, b, h, 0.01, final[b], f"C5 c={c} b={b} h={h}") for (c, b, h) in rows]
    _log(f"C5: max rel err {max(errs):.2e} over {len(rows)} rows")
    for (c, b, h) in rows[:2]:
        n_q = 32 * (final[b] // 32)
        _check_records(wl, c, b, h, final[b], [n_q // 16 - 2, n_q // 16 - 1])
    del wl
    torch.cuda.empty_cache()
