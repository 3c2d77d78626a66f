"""Benchmark: loop-aware decode attention over the full 4-loop x 24-layer plan at 16K context.

Workload (the long-context configuration): 96 cells (seeded 48 4-bit / 29 2-bit /
19 reuse-final-loop plan), 16 heads x 128, batch 32, 16384-token context, paged
16-token blocks with a shuffled block table, bf16 inputs, per-cell K/V scales
log-uniform in [0.5, 4]. One step = a one-token append to every storing cell of
every sequence (quantizing completed 32-token groups) followed by the
whole-plan decode at tau = 0.01. Lengths start at 16384 - (warmup + steps) so
the last step decodes exactly 16384 tokens.

Prints one JSON line. ``value`` is the algorithmic HBM rate of the step (bytes
the method must move / step time); ``roofline`` is the decode kernel's
algorithmic bytes per launch over its mean duration (HIP events on the launch
stream) against the 8 TB/s HBM peak; ``cpu_baseline`` times the fp64 oracle on a
few sampled rows of the same workload on the host.

Extra fields: the tau sweep, the token-skipping ablation (unselected tokens dropped instead of
read at 2 bits), the KIVI-4 layout on the same kernel, a read-ceiling probe, and
the per-(loop, layer) serving order under a graph (each cell appends its token and decodes in
turn, as a looped model calls it): at batch 32 beside the whole-plan step, and at batch 1 with
the split decode (each row over n_split workgroups) against one workgroup per row.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
SERVING_WARM, SERVING_REPS = 2, 5     # graph replays of the per-(loop, layer) legs
SERVING_SPLITS = (0, 8, 16, 32)       # workgroups per row tried at batch 1
COUNTERS = os.path.join(ROOT, "profiles", "k_decode_c4_tau0.01_counters.json")
KERNEL_SOURCES = ["quantized_kv_cache_loopkv_amd/csrc/decode.hip", "quantized_kv_cache_loopkv_amd/csrc/layout.h"]


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def counter_traffic():
    """HBM bytes per decode launch from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE summary
    (copy-calibrated), or None when the decode kernel's source has changed since."""
    try:
        with open(COUNTERS) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("source_sha256") != kernel_source_hash():
        return None
    return d.get("traffic_bytes_per_launch")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(plan, lengths, H, D, sel_counts=None, layout_kivi=False, out_bytes=2, q_bytes=2, group=32):
    """Bytes one whole-plan decode must move.

    Per (cell, sequence, head) row with N tokens, n_q = G floor(N/G) (G = group):
      quantized prefix: D/2 + 8D/G B/token (D=128, G=32: K_hi 32 + K_meta 16 + V_hi 32 +
      V_meta 16 = 96; G=64: 80), plus D/2 B (K_lo + V_lo) per selected token on a 4-bit
      target; KIVI-4 reads D + 8D/G B/token (160 at D=128, G=32);
      tail: 4*D B/token (bf16 K and V); query and output: D * dtype bytes each;
      block table: 4 B per 16-token block; length: 4 B.
    sel_counts[c][b][h] is the number of selected tokens (4-bit targets only).
    """
    import numpy as np
    plan = np.asarray(plan).reshape(-1)
    n_loops_layers = plan.size
    per_tok_base = D // 2 + 8 * D // group
    per_tok_lo = D // 2
    per_tok_kivi = D + 8 * D // group
    total = 0
    n_layers = None
    for c in range(n_loops_layers):
        kind = plan[c]
        for b, N in enumerate(lengths):
            n_q = group * (N // group)
            row = (N - n_q) * 4 * D + D * q_bytes + D * out_bytes + 4 * ((N + 15) // 16) + 4
            if layout_kivi:
                row += n_q * per_tok_kivi
                total += H * row
                continue
            row += n_q * per_tok_base
            total += H * row
            if sel_counts is not None:
                total += per_tok_lo * int(sel_counts[c, b].sum())
    return total


def algorithmic_bytes_skip(tk, lengths, H, D, sel_counts, out_bytes=2, q_bytes=2, group=32):
    """Bytes of the token-skipping ablation's whole-plan decode: rows with a 4-bit target read
    D/4 + 4D/G B/token (D=128, G=32: K_hi 32 + K_meta 16) plus 3D/4 + 4D/G per selected token
    (K_lo 32 + V_hi 32 + V_lo 32 + V_meta 16); 2-bit targets, tails, q, output and block table
    as in the method."""
    import numpy as np
    tk = np.asarray(tk).reshape(-1)
    total = 0
    for c in range(tk.size):
        for b, N in enumerate(lengths):
            n_q = group * (N // group)
            row = (N - n_q) * 4 * D + D * q_bytes + D * out_bytes + 4 * ((N + 15) // 16) + 4
            row += n_q * ((D // 4 + 4 * D // group) if tk[c] == 0 else (D // 2 + 8 * D // group))
            total += H * row
            if tk[c] == 0:
                total += (3 * D // 4 + 4 * D // group) * int(sel_counts[c, b].sum())
    return total


def target_kinds(plan, n_loops, n_layers):
    import numpy as np
    p = np.asarray(plan).reshape(-1)
    out = p.copy()
    for c in range(p.size):
        if p[c] == 2:
            out[c] = p[(n_loops - 1) * n_layers + c % n_layers]
    return out


def append_bytes(n_storing, B, H, D, lengths_before, group=32):
    """Bytes of a one-token append: bf16 K and V in, one tail slot out; a completed group
    also reads its G - 1 tail tokens and writes its G / 16 4-bit records (G D + 8 D bytes)."""
    import numpy as np
    tok = 2 * H * D * 2
    total = n_storing * B * (tok + tok)
    done = sum(1 for n in lengths_before if n % group == group - 1)
    return total + n_storing * done * H * ((group - 1) * 2 * D * 2 + group * D + 8 * D)


def sel_counts_from_mask(sm, n_q):
    """Per-row selected counts from the u32 mask tensor [cells][B][H][words]."""
    import numpy as np
    w = sm.cpu().numpy().view(np.uint32)
    bits = np.unpackbits(w.view(np.uint8), axis=-1, bitorder="little")
    return bits.sum(axis=-1)


def cpu_baseline(cfg, plan, tau, rows, log, min_seconds=10.0, max_evals=400):
    """Time the fp64 oracle (quantize + loop-aware decode of one row) on sampled rows.

    The distinct rows' inputs are drawn first (untimed); the oracle then evaluates the
    rows round-robin until about ``min_seconds`` of CPU time has accumulated."""
    import numpy as np
    from oracle import loopkv_oracle as O
    from synth import recipes as R
    from synth.philox import bf16_bits_to_f32
    try:
        from threadpoolctl import threadpool_info
        cores = max([1] + [i.get("num_threads", 1) for i in threadpool_info()])
    except Exception:
        cores = 1
    factors = R.factor_table(cfg)
    sig = float(np.float32(1.0 / math.sqrt(cfg.head_dim)))
    inputs = []
    for (c, b, h) in rows:
        st = O.storage_cell(plan.reshape(cfg.n_loops, cfg.n_layers), c)
        kind = O.target_kind(plan.reshape(cfg.n_loops, cfg.n_layers), c)
        N = cfg.lengths[b]
        kb, vb = R.kv_row_bits(cfg, st, b, h, 0, N, factors)
        K = bf16_bits_to_f32(kb).astype(np.float64)
        V = bf16_bits_to_f32(vb).astype(np.float64)
        q = R.q_values(cfg, c, 0, b, h).astype(np.float64)
        inputs.append((q, K, V, kind, N))
    t_total = 0.0
    bytes_total = 0
    evals = 0
    while evals < max_evals and (t_total < min_seconds or evals < len(inputs)):
        q, K, V, kind, N = inputs[evals % len(inputs)]
        t0 = time.perf_counter()
        o, sel, _ = O.decode_row(q, K, V, kind, tau, sig, group=cfg.group)
        t_total += time.perf_counter() - t0
        D, G = cfg.head_dim, cfg.group
        n_q = G * (N // G)
        bytes_total += n_q * (D // 2 + 8 * D // G) + (N - n_q) * 4 * D + 4 * D + 4 * ((N + 15) // 16) + 4
        if kind == 0:
            bytes_total += D // 2 * int(sel.sum())
        evals += 1
    log(f"cpu oracle: {evals} row evaluations ({len(inputs)} distinct rows) in {t_total:.2f}s")
    cpu_model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": bytes_total / t_total / 1e9, "unit": "GB/s", "cores": int(cores), "kind": "oracle",
            "host_cpus": os.cpu_count(), "cpu_model": cpu_model,
            "sample": f"{len(inputs)} distinct (cell, seq, head) rows of the 16K-context plan (4-bit, 2-bit and "
                      f"reuse cells), evaluated round-robin {evals} times: fp64 quantize + loop-aware decode "
                      f"per row, {t_total:.2f} s measured, input generation excluded; value = the rows' "
                      f"algorithmic bytes / oracle time"}


def serving_graph(wl, q, tau, first_step, n_rep, n_split, log, warm=2):
    """Per-(loop, layer) serving order (each cell: append the new token, decode the cell) captured
    once in a HIP graph by the library (loopkv_step_graph_create) and launched once per step;
    returns the mean and per-launch ms. Appends n_rep + warm tokens."""
    import torch
    cfg = wl.cfg
    C, B, H, D = cfg.n_cells, cfg.batch, cfg.n_heads, cfg.head_dim
    max_len = cfg.max_len
    stream = torch.cuda.current_stream()
    K0, V0, before, _ = wl.append_inputs(first_step)
    sK, sV = K0.clone(), V0.clone()
    lb = before.clone()
    la = lb + 1
    out = torch.empty((C, B, H, D), dtype=torch.bfloat16, device="cuda")
    scratch = None
    if n_split:
        scratch = torch.empty(wl.ctx.split_scratch_bytes(B, max_len, n_split, cell=(0, 0)), dtype=torch.uint8,
                              device="cuda")
    g = wl.ctx.step_graph(sK, sV, q, wl.bt, lb, la, max_len, tau, out, n_split=n_split, scratch=scratch)
    torch.cuda.synchronize()
    ms = []
    for k in range(warm + n_rep):
        if k > 0:
            K, V, _, _ = wl.append_inputs(first_step + k)
            sK.copy_(K)
            sV.copy_(V)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.launch()
        e1.record(stream)
        torch.cuda.synchronize()
        if k >= warm:
            ms.append(e0.elapsed_time(e1))
    g.close()
    return float(sum(ms) / len(ms)), ms


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--tau", type=float, default=0.01)
    ap.add_argument("--ctx", type=int, default=16384)
    ap.add_argument("--batch", type=int, default=32)
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-kivi", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-serving", action="store_true",
                    help="skip the per-(loop, layer) graph legs (batch 32 and batch 1)")
    ap.add_argument("--cpu-rows", type=int, default=6)
    ap.add_argument("--group", type=int, choices=[32, 64], default=32,
                    help="quantization group (tokens per K group, channels per V group); the pages' is 32")
    ap.add_argument("--table", choices=["shuffled", "identity"], default="shuffled",
                    help="block table of the workload (the configuration uses a shuffled one)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a device-to-device copy of 4 GiB three times (counter calibration)")
    args = ap.parse_args()
    if args.calibrate_copy:
        import torch
        n = 4 << 30
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 3}))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path (asked for --gpus {args.gpus}). "
              "Rows of the decode are independent; see the sharding notes for how it would split.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import quantized_kv_cache_loopkv_amd as lkv
    from synth import recipes as R
    from tests.harness import Workload

    torch.cuda.set_device(0)
    lkv.lib()
    S = args.warmup + args.steps
    GS = 0 if args.no_serving else SERVING_WARM + SERVING_REPS   # tokens the serving leg appends
    cfg = R.make_config("C4")
    cfg.batch = args.batch
    cfg.lengths = [args.ctx - S] * args.batch
    cfg.append_steps = S + GS
    cfg.shuffled = args.table == "shuffled"
    cfg.group = GQ = args.group
    plan = cfg.plan.reshape(-1)
    H, D, C, B = cfg.n_heads, cfg.head_dim, cfg.n_cells, cfg.batch

    t0 = time.time()
    wl = Workload(cfg, gpu_synth=True, log=log)
    log(f"workspace {wl.ws.numel() / 1e9:.2f} GB; filling {len(wl.storing_cells())} storing cells")
    wl.fill()
    log(f"filled in {time.time() - t0:.1f}s")
    q = wl.q_all()
    out = torch.empty((C, B, H, D), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()

    inputs = [wl.append_inputs(s) for s in range(S)]   # drawn before the timed region
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(S)]
    lengths_before = []
    for s in range(S):
        if s == args.warmup:
            torch.cuda.synchronize()
            t_wall0 = time.perf_counter()
        lengths_before.append(wl.current_lengths(s))
        e0, e1, e2 = ev[s]
        e0.record(stream)
        wl.append_step(s, inputs[s])
        e1.record(stream)
        wl.ctx.decode(q, wl.bt, wl.seq_lens, wl.max_len(s + 1), args.tau, out=out, out_dtype=torch.bfloat16)
        e2.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall0
    step_ms = [ev[s][0].elapsed_time(ev[s][2]) for s in range(args.warmup, S)]
    dec_ms = [ev[s][1].elapsed_time(ev[s][2]) for s in range(args.warmup, S)]
    app_ms = [ev[s][0].elapsed_time(ev[s][1]) for s in range(args.warmup, S)]
    ms_per_step = t_wall * 1e3 / args.steps

    # selected tokens at the final state (untimed), for the byte count
    final_lens = wl.current_lengths(S)
    _, sm = wl.ctx.decode(q, wl.bt, wl.seq_lens, max(final_lens), args.tau, out_dtype=torch.bfloat16,
                          sel_mask=True)
    torch.cuda.synchronize()
    tk = target_kinds(plan, cfg.n_loops, cfg.n_layers)
    counts = sel_counts_from_mask(sm, None)
    counts[tk != 0] = 0
    dec_bytes = algorithmic_bytes(plan, final_lens, H, D, counts, group=GQ)
    n_storing = len(wl.storing_cells())
    step_bytes = [algorithmic_bytes(plan, wl.current_lengths(s + 1), H, D, counts, group=GQ) +
                  append_bytes(n_storing, B, H, D, lengths_before[s], group=GQ) for s in range(args.warmup, S)]
    value = float(np.mean(step_bytes)) / (ms_per_step * 1e-3) / 1e9
    dec_mean_ms = float(np.mean(dec_ms))
    achieved = dec_bytes / (dec_mean_ms * 1e-3) / 1e9
    sel_frac = float(counts.sum()) / max(1, sum(int(H * B * (GQ * (final_lens[0] // GQ))) for c in range(C) if tk[c] == 0))
    log(f"step {ms_per_step:.3f} ms (events {np.mean(step_ms):.3f}), decode {dec_mean_ms:.3f} ms, "
        f"append {np.mean(app_ms):.3f} ms; decode {achieved:.0f} GB/s algorithmic; selected fraction {sel_frac:.2e}")

    extra = {}
    if not args.no_sweep:
        sweep = {}
        for tau in (0.0, 0.001, 0.01, 1.1):
            _, smt = wl.ctx.decode(q, wl.bt, wl.seq_lens, max(final_lens), tau, out_dtype=torch.bfloat16,
                                   sel_mask=True)
            ct = sel_counts_from_mask(smt, None)
            ct[tk != 0] = 0
            bts = algorithmic_bytes(plan, final_lens, H, D, ct, group=GQ)
            e_a, e_b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            wl.ctx.decode(q, wl.bt, wl.seq_lens, max(final_lens), tau, out=out, out_dtype=torch.bfloat16)
            e_a.record(stream)
            for _ in range(3):
                wl.ctx.decode(q, wl.bt, wl.seq_lens, max(final_lens), tau, out=out, out_dtype=torch.bfloat16)
            e_b.record(stream)
            torch.cuda.synchronize()
            ms = e_a.elapsed_time(e_b) / 3
            sweep[str(tau)] = {"decode_ms": round(ms, 4), "algorithmic_GB": round(bts / 1e9, 3),
                               "GBps": round(bts / (ms * 1e-3) / 1e9, 1), "selected": int(ct.sum())}
            log(f"tau={tau}: {ms:.3f} ms, {bts / 1e9:.2f} GB, {bts / (ms * 1e-3) / 1e9:.0f} GB/s")
        extra["tau_sweep"] = sweep
        # the ablation the pages reject: drop the unselected tokens instead of reading them at 2 bits
        _, sms = wl.ctx.decode(q, wl.bt, wl.seq_lens, max(final_lens), args.tau, out_dtype=torch.bfloat16,
                               sel_mask=True, skip=True)
        cs = sel_counts_from_mask(sms, None)
        cs[tk != 0] = 0
        sb = algorithmic_bytes_skip(tk, final_lens, H, D, cs, group=GQ)
        e_a, e_b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e_a.record(stream)
        for _ in range(3):
            wl.ctx.decode(q, wl.bt, wl.seq_lens, max(final_lens), args.tau, out=out, out_dtype=torch.bfloat16,
                          skip=True)
        e_b.record(stream)
        torch.cuda.synchronize()
        sms_ms = e_a.elapsed_time(e_b) / 3
        extra["skip_ablation"] = {"decode_ms": round(sms_ms, 4), "algorithmic_GB": round(sb / 1e9, 3),
                                  "GBps": round(sb / (sms_ms * 1e-3) / 1e9, 1),
                                  "bytes_ratio_to_method": round(sb / dec_bytes, 4),
                                  "time_ratio_to_method": round(sms_ms / dec_mean_ms, 4)}
        log(f"skip ablation: {sms_ms:.3f} ms, {sb / 1e9:.2f} GB ({sb / dec_bytes:.3f} of the method's bytes)")
    if not args.no_serving:
        # the same cache in the order a looped model calls it (96 cells one by one), under a graph
        ms, per = serving_graph(wl, q, args.tau, S, SERVING_REPS, 0, log, warm=SERVING_WARM)
        extra["per_cell_graph"] = {
            "batch": B, "context": f"{args.ctx}..{args.ctx + GS}", "ms_per_step": round(ms, 4),
            "whole_plan_ms_per_step": round(float(np.mean(step_ms)), 4),
            "ratio_to_whole_plan": round(ms / float(np.mean(step_ms)), 4),
            "launches_per_step": n_storing + C + 1}   # appends, decodes, the length update
        log(f"per-cell graph, batch {B}: {ms:.3f} ms per step vs whole plan {np.mean(step_ms):.3f} ms")
        # one sequence: the per-cell launches hold 16 rows each, so the split decode fills the GPU
        scfg = R.make_config("C4")
        scfg.batch = 1
        scfg.lengths = [args.ctx]
        scfg.append_steps = len(SERVING_SPLITS) * (SERVING_WARM + SERVING_REPS)
        scfg.group = GQ
        sw = Workload(scfg, gpu_synth=True, log=log)
        sw.fill()
        sq = sw.q_all()
        small = {"batch": 1, "context": args.ctx}
        first = 0
        for ns in SERVING_SPLITS:
            ms1, _ = serving_graph(sw, sq, args.tau, first, SERVING_REPS, ns, log, warm=SERVING_WARM)
            first += SERVING_WARM + SERVING_REPS
            small[f"ms_per_step_split{ns}"] = round(ms1, 4)
            log(f"per-cell graph, batch 1, n_split {ns}: {ms1:.3f} ms per step")
        extra["per_cell_graph_batch1"] = small
        del sw
        torch.cuda.empty_cache()
    if not args.no_kivi:
        kcfg = R.make_config("C4")
        kcfg.batch = B
        kcfg.lengths = list(final_lens)
        kcfg.group = GQ
        kcfg.append_steps = 0
        t1 = time.time()
        kw = Workload(kcfg, layout=lkv.LAYOUT_KIVI4, gpu_synth=True, log=log)
        kw.fill()
        log(f"KIVI-4 cache filled in {time.time() - t1:.1f}s")
        kb = algorithmic_bytes(plan, final_lens, H, D, layout_kivi=True, group=GQ)
        kw.decode(q, args.tau, out_dtype=torch.bfloat16, sel_mask=False)
        e_a, e_b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e_a.record(stream)
        for _ in range(3):
            kw.ctx.decode(q, kw.bt, kw.seq_lens, max(final_lens), args.tau, out=out, out_dtype=torch.bfloat16)
        e_b.record(stream)
        torch.cuda.synchronize()
        kms = e_a.elapsed_time(e_b) / 3
        extra["kivi4_same_kernel"] = {"decode_ms": round(kms, 4), "algorithmic_GB": round(kb / 1e9, 3),
                                      "GBps": round(kb / (kms * 1e-3) / 1e9, 1),
                                      "bytes_ratio_loopkv_over_kivi4": round(dec_bytes / kb, 4),
                                      "time_ratio_loopkv_over_kivi4": round(dec_mean_ms / kms, 4)}
        log(f"KIVI-4: {kms:.3f} ms, {kb / 1e9:.2f} GB, ratio bytes {dec_bytes / kb:.3f} time {dec_mean_ms / kms:.3f}")
        del kw
        torch.cuda.empty_cache()

    try:
        from synth import gpu as G
        extra["read_ceiling"] = G.read_ceiling(chunk_bytes=1536)   # the K and V spans of one 4-bit record
        log(f"read ceiling: {extra['read_ceiling']}")
    except Exception as e:  # the probe is context only
        log(f"read ceiling probe failed: {e}")

    cpu = None
    if not args.no_cpu:
        rows = []
        kinds_seen = {}
        for c in range(C):
            k = int(plan[c])
            if kinds_seen.get(k, 0) < max(1, args.cpu_rows // 3):
                rows.append((c, (7 * c) % B, (3 * c) % H))
                kinds_seen[k] = kinds_seen.get(k, 0) + 1
            if len(rows) >= args.cpu_rows:
                break
        ccfg = R.make_config("C4")
        ccfg.batch = B
        ccfg.lengths = [args.ctx - S] * B     # the initial histories of the timed workload
        ccfg.append_steps = S + GS
        ccfg.group = GQ
        cpu = cpu_baseline(ccfg, plan, args.tau, rows, log)

    line = {
        "metric": "achieved HBM GB/s (% of peak) + us per decode step, 4x24 plan, 16K ctx",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "us_per_decode_step": round(dec_mean_ms * 1e3, 1),
        "pct_of_peak": round(100 * value / PEAK_HBM_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8 dot products into i32, f32 softmax and accumulators (bf16 q/K/V in, bf16 out)",
        "data": "synthetic (seeded Philox normal draws, shapes of the pages' Ouro-1.4B 16K serving workload)",
        "config": {"workload": "4 loops x 24 layers, 48 q4 / 29 q2 / 19 reuse, 16 heads x 128, batch 32, "
                               f"context {args.ctx} (last step), 16-token blocks shuffled, tau {args.tau}, "
                               "1-token append + whole-plan decode per step"
                               + ("" if GQ == 32 else f", quantization groups of {GQ}"),
                   "global_batch": B, "seq_len": args.ctx, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": counter_traffic() if GQ == 32 else None,   # the counters cover groups of 32
                     "kernel": f"k_decode<128, {GQ}, tau regime, PH_ROW>", "bytes_per_launch": dec_bytes,
                     "mean_launch_ms": round(dec_mean_ms, 4)},
        "cpu_baseline": cpu,
        "selected_fraction_q4_targets": sel_frac,
        "append_ms": round(float(np.mean(app_ms)), 4),
    }
    line.update(extra)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
