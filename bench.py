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
stream) against the 8 TB/s HBM peak; ``cpu_baseline`` times the fp64 oracle's decode on a
row subset of the same workload (every cell x 2 sequences x every head) on the host's cores.

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
KERNEL_SOURCES = ["quantized_kv_cache_loopkv_amd/csrc/decode.hip", "quantized_kv_cache_loopkv_amd/csrc/layout.h",
                  "quantized_kv_cache_loopkv_amd/csrc/quantize.h"]


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
      tail: 4*D B/token (bf16 K and V); query and output: D * dtype bytes each.
    Per (cell, sequence): the block table, 4 B per 16-token block (the heads of a sequence
    share its row).
    sel_counts[c][b][h] is the number of selected tokens (4-bit targets only).
    """
    import numpy as np
    plan = np.asarray(plan).reshape(-1)
    per_tok_base = D // 2 + 8 * D // group
    per_tok_lo = D // 2
    per_tok_kivi = D + 8 * D // group
    total = 0
    for c in range(plan.size):
        for b, N in enumerate(lengths):
            n_q = group * (N // group)
            row = (N - n_q) * 4 * D + D * q_bytes + D * out_bytes
            row += n_q * (per_tok_kivi if layout_kivi else per_tok_base)
            total += H * row + 4 * ((N + 15) // 16)
            if sel_counts is not None and not layout_kivi:
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
            row = (N - n_q) * 4 * D + D * q_bytes + D * out_bytes
            row += n_q * ((D // 4 + 4 * D // group) if tk[c] == 0 else (D // 2 + 8 * D // group))
            total += H * row + 4 * ((N + 15) // 16)
            if tk[c] == 0:
                total += (3 * D // 4 + 4 * D // group) * int(sel_counts[c, b].sum())
    return total


def gathered_bytes(sm, tk, D, group=32):
    """Bytes the corrections load for the selected tokens, as the kernel reads them: per 32-token
    unit holding a selected token its K low plane (8 D) and its group's K meta (4 D: one word
    per channel), per 16-token block holding one its V high and low planes and V meta
    (8 D + 64 D / G). The algorithmic count charges D/2 per selected token instead; the
    difference is the gather's re-read granularity."""
    import torch
    w = sm.to(torch.int64) & 0xFFFFFFFF                       # [cells][B][H][units]
    rows_q4 = torch.as_tensor(tk == 0, device=sm.device).view(-1, 1, 1, 1)
    units = ((w != 0) & rows_q4).sum().item()
    blocks = ((((w & 0xFFFF) != 0).to(torch.int64) + (((w >> 16) & 0xFFFF) != 0).to(torch.int64))
              * rows_q4).sum().item()
    meta = 64 * D // group
    return int(units * (8 * D + 4 * D) + blocks * (8 * D + meta))


def target_kinds(plan, n_loops, n_layers):
    import numpy as np
    p = np.asarray(plan).reshape(-1)
    out = p.copy()
    for c in range(p.size):
        if p[c] == 2:
            out[c] = p[(n_loops - 1) * n_layers + c % n_layers]
    return out


def append_bytes(n_storing, B, H, D, lengths_before, group=32, n_q2=0):
    """Bytes of a one-token append: bf16 K and V in, one tail slot out; a completed group
    also reads its G - 1 tail tokens and writes its G / 16 records: G D + 8 D bytes at 4 bits,
    G D / 2 + 8 D bytes for the n_q2 storing cells kept at 2 bits."""
    tok = 2 * H * D * 2
    total = n_storing * B * (tok + tok)
    done = sum(1 for n in lengths_before if n % group == group - 1)
    tail_read = (group - 1) * 2 * D * 2
    flush = (n_storing - n_q2) * (tail_read + group * D + 8 * D) + n_q2 * (tail_read + group * D // 2 + 8 * D)
    return total + done * H * flush


def prefill_bytes(plan, lengths, H, D, group=32):
    """Bytes of the bulk appends that build the cache: for every storing cell and sequence of N
    tokens, bf16 K and V in (4 D B per token-head), the records of its N // G complete groups out
    (G D + 8 D B per group-head at 4 bits, G D / 2 + 8 D at 2 bits) and its last N mod G tokens
    into the tail (4 D B per token-head)."""
    import numpy as np
    plan = np.asarray(plan).reshape(-1)
    total = 0
    for kind in plan:
        if kind == 2:   # reuse: nothing stored
            continue
        flush = group * D + 8 * D if kind == 0 else group * D // 2 + 8 * D
        for N in lengths:
            total += H * (N * 4 * D + (N // group) * flush + (N % group) * 4 * D)
    return total


def append_figures(app_ms, lengths_before, n_storing, B, H, D, group=32, n_q2=0):
    """The timed steps' one-token appends, split into steps that only write the token to the tail
    and steps whose token completes a group of every sequence (each then quantizes and writes the
    group's records): mean ms, algorithmic bytes (append_bytes) and GB/s of each kind. The append
    is latency-bound (a few KB per workgroup); the fraction of the 8 TB/s peak is given anyway."""
    import numpy as np
    out = {}
    for kind, pick in (("token_only", lambda L: all(n % group != group - 1 for n in L)),
                       ("group_completing", lambda L: any(n % group == group - 1 for n in L))):
        idx = [i for i, L in enumerate(lengths_before) if pick(L)]
        if not idx:
            continue
        ms = float(np.mean([app_ms[i] for i in idx]))
        by = float(np.mean([append_bytes(n_storing, B, H, D, lengths_before[i], group, n_q2) for i in idx]))
        gbs = by / (ms * 1e-3) / 1e9
        out[kind] = {"steps": len(idx), "ms": round(ms, 4), "algorithmic_GB": round(by / 1e9, 4),
                     "GBps": round(gbs, 1), "frac_of_peak": round(gbs / PEAK_HBM_GBS, 4)}
    return out


def sel_counts_from_mask(sm, n_q):
    """Per-row selected counts from the u32 mask tensor [cells][B][H][words]."""
    import numpy as np
    w = sm.cpu().numpy().view(np.uint32)
    bits = np.unpackbits(w.view(np.uint8), axis=-1, bitorder="little")
    return bits.sum(axis=-1)


CPU_SEQS = 2    # sequences of the oracle's row subset: every cell and head of each
CPU_REPS = 3    # timed repetitions of every row (the subset's time is the median pass)


def cpu_workers():
    """Worker processes for the oracle: the host's CPU share for this process, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _cpu_worker_init():
    """One BLAS thread per worker process: the rows run in parallel across processes."""
    for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ[k] = "1"
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:
        pass


def cpu_rows_task(kpath, vpath, rows, tau, sig, group, bits, reps):
    """The oracle's decode of every row reading one storage chunk (one cell and sequence, bf16
    K and V bits [N][KV heads][D] in two .npy files, removed once read). Per KV head the history
    is converted and quantized once (untimed); each row (head, query, kind) is then decoded
    ``reps`` times, each timed. Returns [(head, [seconds per repetition], selected count)]."""
    import numpy as np
    from oracle import loopkv_oracle as O
    from synth.philox import bf16_bits_to_f32
    kb = np.load(kpath)
    vb = np.load(vpath)
    os.remove(kpath)
    os.remove(vpath)
    out = []
    cur, K, V, qh = None, None, None, None
    for h, q, kind in sorted(rows, key=lambda r: r[0]):
        if h != cur:
            K = bf16_bits_to_f32(np.ascontiguousarray(kb[:, h])).astype(np.float64)
            V = bf16_bits_to_f32(np.ascontiguousarray(vb[:, h])).astype(np.float64)
            qh = O.quantize_history(K, V, bits, group)
            cur = h
        ts = []
        for _ in range(reps):
            t0 = time.perf_counter()
            _, sel, _ = O.decode_row(q, K, V, kind, tau, sig, qh=qh, group=group)
            ts.append(time.perf_counter() - t0)
        out.append((h, ts, int(sel.sum())))
    return out


def _spool_dir(need_bytes):
    import shutil
    import tempfile
    for d in ("/dev/shm", tempfile.gettempdir()):
        try:
            if os.access(d, os.W_OK) and shutil.disk_usage(d).free > 2 * need_bytes:
                return tempfile.mkdtemp(prefix="loopkv_cpu_", dir=d)
        except OSError:
            continue
    return tempfile.mkdtemp(prefix="loopkv_cpu_")


def cpu_baseline(pool, workers, wl, q, plan, tau, lengths, seqs, log):
    """The fp64 oracle's decode on a row subset of the timed workload: every cell x the given
    sequences x every head, on the same inputs (the seeded generator's draws of each row's
    history, the queries of the timed decode). Generation and quantization are excluded; each row
    is decoded CPU_REPS times in one of ``workers`` single-threaded processes. The subset's time
    is the median over the repetitions of the rows' summed time, divided over the workers (rows
    are independent); the per-step figure scales it by all rows / subset rows."""
    import numpy as np
    import torch
    from oracle import loopkv_oracle as O
    cfg = wl.cfg
    C, B, H, D, G = cfg.n_cells, cfg.batch, cfg.n_heads, cfg.head_dim, cfg.group
    P = plan.reshape(cfg.n_loops, cfg.n_layers)
    sig = float(np.float32(1.0 / math.sqrt(D)))
    qh_ = q.float().cpu().numpy().astype(np.float64)
    chunks = {}
    for c in range(C):
        st, kind = O.storage_cell(P, c), O.target_kind(P, c)
        for b in seqs:
            for h in range(H):
                chunks.setdefault((st, b), []).append((h, qh_[c, b, h], kind))
    n_rows = sum(len(r) for r in chunks.values())
    chunk_bytes = 2 * max(lengths) * cfg.kv_heads * D * 2
    spool = _spool_dir(2 * workers * chunk_bytes)
    t_wall = time.perf_counter()
    results, pending = [], []
    try:
        for i, ((st, b), rows) in enumerate(chunks.items()):
            N = lengths[b]
            K, V = wl.kv_seq_gpu(st, b, 0, N)
            kp, vp = os.path.join(spool, f"k{i}.npy"), os.path.join(spool, f"v{i}.npy")
            np.save(kp, K[0].view(torch.int16).cpu().numpy().view(np.uint16))
            np.save(vp, V[0].view(torch.int16).cpu().numpy().view(np.uint16))
            del K, V
            bits = 2 if int(plan[st]) == 1 else 4
            pending.append((N, st, pool.apply_async(cpu_rows_task, (kp, vp, rows, tau, sig, G, bits, CPU_REPS))))
            while len(pending) >= 2 * workers:   # bound the spooled chunks
                N0, st0, r0 = pending.pop(0)
                results.append((N0, st0, r0.get()))
        for N, st, r in pending:
            results.append((N, st, r.get()))
    finally:
        import shutil
        shutil.rmtree(spool, ignore_errors=True)
    t_wall = time.perf_counter() - t_wall
    pass_s = np.zeros(CPU_REPS)
    sub_bytes = 0
    for N, st, res in results:
        n_q = G * (N // G)
        for h, ts, n_sel in res:
            pass_s += np.asarray(ts)
            sub_bytes += n_q * (D // 2 + 8 * D // G) + (N - n_q) * 4 * D + 4 * D + (D // 2) * n_sel
    sub_bytes += sum(4 * ((lengths[b] + 15) // 16) for b in seqs) * C   # block table per (cell, sequence)
    cpu_s = float(np.median(pass_s))
    sub_s = cpu_s / workers
    scale = (C * B * H) / n_rows
    log(f"cpu oracle: {n_rows} rows x {CPU_REPS} on {workers} workers, {t_wall:.1f} s wall "
        f"(drawing and quantization included); rows' decode time {cpu_s:.1f} cpu-s per pass (median)")
    cpu_model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": sub_bytes / sub_s / 1e9, "unit": "GB/s", "cores": workers, "kind": "oracle",
            "subset_rows": n_rows, "subset_cpu_seconds_median": round(cpu_s, 3),
            "subset_seconds_on_cores": round(sub_s, 3),
            "us_per_step_extrapolated": round(sub_s * scale * 1e6, 1),
            "host_cpus": os.cpu_count(), "cpu_model": cpu_model,
            "sample": f"fp64 oracle decode (numpy) of {n_rows} rows of the timed workload: all {C} cells x "
                      f"{len(seqs)} sequences x {H} heads at {max(lengths)} tokens, tau {tau}, the same seeded "
                      f"inputs and queries; quantization and input generation excluded; each row decoded "
                      f"{CPU_REPS} times, the subset time is the median pass ({cpu_s:.1f} cpu-s) over "
                      f"{workers} single-threaded worker processes ({sub_s:.2f} s); value = the subset's "
                      f"algorithmic bytes / that time; us_per_step_extrapolated scales it by "
                      f"{C * B * H} / {n_rows} rows"}


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


def workload_name(wk, cfg, args, group):
    import numpy as np
    p = cfg.plan.reshape(-1)
    kinds = f"{int((p == 0).sum())} q4 / {int((p == 1).sum())} q2 / {int((p == 2).sum())} reuse"
    if wk == "c5":
        ctx = f"lengths uniform in [1024, 16384] (mean {int(np.mean(cfg.lengths)) + cfg.append_steps})"
    else:
        ctx = f"context {args.ctx} (last step)"
    table = "shuffled" if cfg.shuffled else "identity"
    return (f"{cfg.n_loops} loops x {cfg.n_layers} layers, {kinds}, {cfg.n_heads} heads x {cfg.head_dim}, "
            f"batch {cfg.batch}, {ctx}, 16-token blocks {table}, tau {args.tau}, "
            "1-token append + whole-plan decode per step" + ("" if group == 32 else f", quantization groups of {group}"))


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
    ap.add_argument("--group", type=int, choices=[32, 64], default=32,
                    help="quantization group (tokens per K group, channels per V group); the pages' is 32")
    ap.add_argument("--table", choices=["shuffled", "identity"], default="shuffled",
                    help="block table of the workload (the configuration uses a shuffled one)")
    ap.add_argument("--workload", choices=["c4", "c3", "c5", "c5-16k-half"], default="c4",
                    help="c4: the headline (4x24 plan, batch 32, 16K, shuffled table); c3: 8K context, identity "
                         "table; c5: batch 128, lengths uniform in [1024, 16384]; c5-16k-half: batch 128 at 16K "
                         "on the plan's last two loops (48 cells; pools above 4 GiB)")
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

    # the oracle's worker processes start before anything touches the GPU
    pool, workers = None, 0
    if not args.no_cpu:
        import multiprocessing as mp
        workers = cpu_workers()
        pool = mp.get_context("spawn").Pool(workers, initializer=_cpu_worker_init)

    import numpy as np
    import torch
    import quantized_kv_cache_loopkv_amd as lkv
    from synth import recipes as R
    from tests.harness import Workload

    torch.cuda.set_device(0)
    lkv.lib()
    S = args.warmup + args.steps
    wk = args.workload
    if wk == "c3":
        args.ctx, args.table = 8192, "identity"
    if wk in ("c5", "c5-16k-half"):
        args.batch = 128
        args.no_kivi = True      # the KIVI-4 cache of these batches does not fit beside the LoopKV one
        args.no_serving = True   # the per-cell serving legs are measured on the headline workload
    GS = 0 if args.no_serving else SERVING_WARM + SERVING_REPS   # tokens the serving leg appends
    if wk == "c5":
        cfg = R.make_config("C5")   # lengths uniform in [1024, 16384]: the first step's
        cfg.lengths = [n - S for n in cfg.lengths]
        args.ctx = max(cfg.lengths) + S
    else:
        cfg = R.make_config("C4")
        cfg.batch = args.batch
        cfg.lengths = [args.ctx - S] * args.batch
        if wk == "c5-16k-half":   # loops 2 and 3: reuse cells of loop 2 read loop 3
            cfg.n_loops = 2
            cfg.plan = cfg.plan[2:4].copy()
    cfg.batch = args.batch
    cfg.append_steps = S + GS
    cfg.shuffled = args.table == "shuffled"
    cfg.group = GQ = args.group
    plan = cfg.plan.reshape(-1)
    H, D, C, B = cfg.n_heads, cfg.head_dim, cfg.n_cells, cfg.batch

    t0 = time.time()
    wl = Workload(cfg, gpu_synth=True, log=log)
    log(f"workspace {wl.ws.numel() / 1e9:.2f} GB; filling {len(wl.storing_cells())} storing cells")
    fill_ev = []
    wl.fill(events=fill_ev)
    log(f"filled in {time.time() - t0:.1f}s")
    fill_ms = sum(e0.elapsed_time(e1) for e0, e1, _ in fill_ev)
    pre_by = prefill_bytes(plan, cfg.lengths, cfg.kv_heads, D, GQ)
    prefill = {"tokens_per_sequence": int(max(cfg.lengths)), "append_calls": len(fill_ev),
               "ms": round(fill_ms, 3), "algorithmic_GB": round(pre_by / 1e9, 3),
               "GBps": round(pre_by / (fill_ms * 1e-3) / 1e9, 1),
               "frac_of_peak": round(pre_by / (fill_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    log(f"prefill appends: {prefill}")
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
    n_q2 = int((plan == 1).sum())   # storing cells kept at 2 bits
    step_bytes = [algorithmic_bytes(plan, wl.current_lengths(s + 1), H, D, counts, group=GQ) +
                  append_bytes(n_storing, B, H, D, lengths_before[s], group=GQ, n_q2=n_q2) for s in range(args.warmup, S)]
    value = float(np.mean(step_bytes)) / (ms_per_step * 1e-3) / 1e9
    dec_mean_ms = float(np.mean(dec_ms))
    achieved = dec_bytes / (dec_mean_ms * 1e-3) / 1e9
    sel_frac = float(counts.sum()) / max(1, sum(H * GQ * (n // GQ) for n in final_lens) * int((tk == 0).sum()))
    log(f"step {ms_per_step:.3f} ms (events {np.mean(step_ms):.3f}), decode {dec_mean_ms:.3f} ms, "
        f"append {np.mean(app_ms):.3f} ms; decode {achieved:.0f} GB/s algorithmic; selected fraction {sel_frac:.2e}")
    append_fig = append_figures(app_ms, [lengths_before[s] for s in range(args.warmup, S)], n_storing, B,
                                cfg.kv_heads, D, GQ, n_q2)
    log(f"append: {append_fig}")

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
            if 0.0 < tau <= 1.0:   # what the corrections load for the selected tokens, as read
                gb = gathered_bytes(smt, tk, D, GQ)
                sweep[str(tau)]["gathered_GB"] = round(gb / 1e9, 4)
                sweep[str(tau)]["algorithmic_selected_GB"] = round((D // 2) * int(ct.sum()) / 1e9, 4)
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
            "launches_per_step": n_storing + C + 1,   # appends, decodes, the length update
            # the whole-plan decode's algorithmic bytes (the serving steps run up to GS tokens
            # longer, a few 1e-4 more bytes; the appends' few KB are not counted)
            "algorithmic_GBps": round(dec_bytes / (ms * 1e-3) / 1e9, 1),
            "frac_of_peak": round(dec_bytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
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
        # algorithmic bytes of one batch-1 step (selected tokens' low planes, ~1e-4 of the
        # bytes at tau 0.01, not counted)
        b1 = algorithmic_bytes(plan, [args.ctx], H, D, group=GQ)
        small = {"batch": 1, "context": args.ctx, "algorithmic_GB": round(b1 / 1e9, 4)}
        first = 0
        for ns in SERVING_SPLITS:
            ms1, _ = serving_graph(sw, sq, args.tau, first, SERVING_REPS, ns, log, warm=SERVING_WARM)
            first += SERVING_WARM + SERVING_REPS
            small[f"ms_per_step_split{ns}"] = round(ms1, 4)
            small[f"GBps_split{ns}"] = round(b1 / (ms1 * 1e-3) / 1e9, 1)
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
    if pool is not None:
        seqs = sorted({0, B // 2})[:CPU_SEQS]
        cpu = cpu_baseline(pool, workers, wl, q, plan, args.tau, final_lens, seqs, log)
        pool.close()
        pool.join()

    default_workload = (wk == "c4" and GQ == 32 and B == 32 and args.ctx == 16384 and args.tau == 0.01
                        and cfg.shuffled)
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
        "config": {"workload": workload_name(wk, cfg, args, GQ),
                   "global_batch": B, "seq_len": args.ctx, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4),
                     # the counters were taken on the default workload (C4, groups of 32, tau 0.01)
                     "traffic": counter_traffic() if default_workload else None,
                     "kernel": f"k_decode<128, {GQ}, tau regime, PH_ROW>", "bytes_per_launch": dec_bytes,
                     "mean_launch_ms": round(dec_mean_ms, 4)},
        "cpu_baseline": cpu,
        "selected_fraction_q4_targets": sel_frac,
        "append_ms": round(float(np.mean(app_ms)), 4),
        "append": append_fig,
        "prefill": prefill,
    }
    line.update(extra)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
