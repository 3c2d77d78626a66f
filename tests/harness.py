"""Helpers shared by the GPU tests and bench.py.

Builds a LoopKV cache for a synthetic configuration through the library's own
append entry point, draws queries, reads records back for bit-exact
comparisons, and evaluates oracle rows from host-regenerated inputs (the oracle
never sees a value produced by the library).
"""
from __future__ import annotations

import math
import time
from typing import Optional

import numpy as np
import torch

import quantized_kv_cache_loopkv_amd as lkv
from synth import recipes as R
from synth.philox import bf16_bits_to_f32


def bits_to_bf16_tensor(bits: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)


class Workload:
    """A configuration materialised on the GPU: context, workspace, tables, lengths."""

    def __init__(self, cfg: R.Config, layout: int = lkv.LAYOUT_PLANES, plan=None, device="cuda",
                 gpu_synth: Optional[bool] = None, log=None):
        self.cfg = cfg
        self.layout = layout
        self.device = device
        self.log = log or (lambda *a: None)
        plan = np.asarray(cfg.plan if plan is None else plan, dtype=np.uint8).reshape(-1)
        if layout == lkv.LAYOUT_KIVI4:
            plan = np.zeros_like(plan)
        self.plan = plan
        self.nb = R.num_blocks(cfg)
        self.ctx = lkv.Context(cfg.n_loops, cfg.n_layers, cfg.n_heads, cfg.head_dim, self.nb, cfg.batch, layout,
                               n_kv_heads=cfg.n_kv_heads, block_tokens=cfg.block_tokens, group_size=cfg.group)
        self.ctx.plan(plan.tolist())
        self.ws = torch.empty(self.ctx.workspace_bytes(), dtype=torch.uint8, device=device)
        self.ctx.bind(self.ws)
        self.bt_np = R.block_table(cfg)
        self.bt = torch.from_numpy(self.bt_np).to(device)
        self.lengths = np.array(cfg.lengths, dtype=np.int64)
        self.seq_lens = torch.zeros(cfg.batch, dtype=torch.int32, device=device)
        self.factors = R.factor_table(cfg)
        big = cfg.batch * max(cfg.lengths) * cfg.kv_heads * cfg.head_dim > (1 << 24)
        self.gpu_synth = big if gpu_synth is None else gpu_synth
        self.factors_dev = torch.from_numpy(self.factors).to(device) if self.gpu_synth else None

    # ------------------------------------------------------------------ cache
    def storing_cells(self):
        return [c for c in range(self.cfg.n_cells) if self.plan[c] != R.SHARE]

    def cell_ll(self, c):
        return divmod(c, self.cfg.n_layers)

    def kv_chunk(self, cell, t0, n, seqs=None):
        """bf16 K, V [len(seqs)][n][H][D] of one cell for tokens t0..t0+n-1."""
        cfg = self.cfg
        if self.gpu_synth:
            from synth import gpu as G
            B = cfg.batch if seqs is None else len(seqs)
            assert seqs is None, "GPU draw covers every sequence"
            K = torch.empty((B, n, cfg.kv_heads, cfg.head_dim), dtype=torch.bfloat16, device=self.device)
            V = torch.empty_like(K)
            G.kv_bf16(cfg.seed, 4 * cell + R.STREAM_K, B, n, t0, cfg.token_stride, cfg.kv_heads, cfg.head_dim,
                      self.factors_dev[cell, 0].contiguous(), K)
            G.kv_bf16(cfg.seed, 4 * cell + R.STREAM_V, B, n, t0, cfg.token_stride, cfg.kv_heads, cfg.head_dim,
                      self.factors_dev[cell, 1].contiguous(), V)
            return K, V
        kb, vb = R.kv_tensor_bits(cfg, cell, t0, t0 + n, self.factors)
        if seqs is not None:
            kb, vb = kb[seqs], vb[seqs]
        return bits_to_bf16_tensor(kb, self.device), bits_to_bf16_tensor(vb, self.device)

    def kv_seq_gpu(self, cell, b, t0, n):
        from synth import gpu as G
        cfg = self.cfg
        K = torch.empty((1, n, cfg.kv_heads, cfg.head_dim), dtype=torch.bfloat16, device=self.device)
        V = torch.empty_like(K)
        t0s = torch.tensor([t0], dtype=torch.int32, device=self.device)
        # draw with the sequence index b: use a one-sequence view whose element index uses b
        G.kv_bf16(cfg.seed, 4 * cell + R.STREAM_K, 1, n, 0, cfg.token_stride, cfg.kv_heads, cfg.head_dim,
                  self.factors_dev[cell, 0].contiguous(), K, t0s=t0s + b * cfg.token_stride)
        G.kv_bf16(cfg.seed, 4 * cell + R.STREAM_V, 1, n, 0, cfg.token_stride, cfg.kv_heads, cfg.head_dim,
                  self.factors_dev[cell, 1].contiguous(), V, t0s=t0s + b * cfg.token_stride)
        return K, V

    def fill(self, chunk_tokens: Optional[int] = None, events: Optional[list] = None):
        """Append every sequence's initial history to every storing cell (bulk appends). With
        ``events`` (a list), each append call is bracketed by a pair of timing events on the
        current stream, appended as (start, end, cell)."""
        cfg = self.cfg
        stream = torch.cuda.current_stream() if events is not None else None

        def timed_append(*args, **kw):
            if events is None:
                self.ctx.append(*args, **kw)
                return
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            self.ctx.append(*args, **kw)
            e1.record(stream)
            events.append((e0, e1, c))

        equal = len(set(cfg.lengths)) == 1
        t_start = time.time()
        for i, c in enumerate(self.storing_cells()):
            loop, layer = self.cell_ll(c)
            if equal:
                N = cfg.lengths[0]
                step = N if chunk_tokens is None else chunk_tokens
                for t0 in range(0, N, step):
                    n = min(step, N - t0)
                    K, V = self.kv_chunk(c, t0, n)
                    lens = torch.full((cfg.batch,), t0, dtype=torch.int32, device=self.device)
                    timed_append(K, V, self.bt, lens, cell=(loop, layer))
                    del K, V
            else:
                for b in range(cfg.batch):
                    N = cfg.lengths[b]
                    if self.gpu_synth:
                        K, V = self.kv_seq_gpu(c, b, 0, N)
                    else:
                        K, V = self.kv_chunk(c, 0, N, seqs=[b])
                        K, V = K[:, :N].contiguous(), V[:, :N].contiguous()
                    lens = torch.zeros(1, dtype=torch.int32, device=self.device)
                    slots = torch.tensor([b], dtype=torch.int32, device=self.device)
                    timed_append(K, V, self.bt[b:b + 1].contiguous(), lens, cell=(loop, layer), seq_slots=slots)
            if (i + 1) % 8 == 0:
                torch.cuda.synchronize()
                self.log(f"  filled {i + 1}/{len(self.storing_cells())} cells ({time.time() - t_start:.1f}s)")
        torch.cuda.synchronize()
        self.seq_lens = torch.tensor(cfg.lengths, dtype=torch.int32, device=self.device)

    def append_inputs(self, step: int):
        """Inputs of the one-token append before decode step ``step``: bf16 K, V
        [cells][B][1][KV heads][D] (token lengths[b] + step of each sequence), lengths before and after."""
        cfg = self.cfg
        C, B, H, D = cfg.n_cells, cfg.batch, cfg.kv_heads, cfg.head_dim
        K = torch.zeros((C, B, 1, H, D), dtype=torch.bfloat16, device=self.device)
        V = torch.zeros_like(K)
        pos = torch.tensor([n + step for n in cfg.lengths], dtype=torch.int32, device=self.device)
        for c in self.storing_cells():
            if self.gpu_synth:
                from synth import gpu as G
                for kv, out in ((0, K), (1, V)):
                    G.kv_bf16(cfg.seed, 4 * c + (R.STREAM_K if kv == 0 else R.STREAM_V), B, 1, 0, cfg.token_stride,
                              H, D, self.factors_dev[c, kv].contiguous(), out[c], t0s=pos)
            else:
                bits_k = np.zeros((B, 1, H, D), dtype=np.uint16)
                bits_v = np.zeros((B, 1, H, D), dtype=np.uint16)
                for b in range(B):
                    t = cfg.lengths[b] + step
                    for h in range(H):
                        kb, vb = R.kv_row_bits(self.cfg, c, b, h, t, t + 1, self.factors)
                        bits_k[b, 0, h] = kb[0]
                        bits_v[b, 0, h] = vb[0]
                K[c] = bits_to_bf16_tensor(bits_k, self.device)
                V[c] = bits_to_bf16_tensor(bits_v, self.device)
        return K, V, pos, pos + 1

    def append_step(self, step: int, inputs=None):
        """Append token lengths[b] + step of every sequence to every storing cell (whole-plan call)."""
        K, V, before, after = self.append_inputs(step) if inputs is None else inputs
        self.ctx.append(K, V, self.bt, before)
        self.seq_lens = after

    def current_lengths(self, step: int = 0):
        return [n + step for n in self.cfg.lengths]

    # ------------------------------------------------------------------ queries
    def q_all(self, step: int = 0) -> torch.Tensor:
        cfg = self.cfg
        C, B, H, D = cfg.n_cells, cfg.batch, cfg.n_heads, cfg.head_dim
        dt = torch.float32 if cfg.q_fp32 else torch.bfloat16
        q = torch.empty((C, B, H, D), dtype=dt, device=self.device)
        if self.gpu_synth:
            from synth import gpu as G
            for c in range(C):
                G.normal(cfg.seed, 4 * c + R.STREAM_Q, step * B * H * D, q[c])
        else:
            for c in range(C):
                qv = R.q_values(cfg, c, step)
                q[c] = torch.from_numpy(qv).to(self.device).to(dt)
        return q

    def max_len(self, step=0):
        return max(self.current_lengths(step))

    def decode(self, q, tau, out_dtype=torch.float32, sel_mask=True, step=0, cell=None):
        qq = q if cell is None else q[cell[0] * self.cfg.n_layers + cell[1]].contiguous()
        return self.ctx.decode(qq, self.bt, self.seq_lens, self.max_len(step), tau, cell=cell,
                               out_dtype=out_dtype, sel_mask=sel_mask)

    def serving_step(self, K, V, q, lens_before, lens_after, max_len, tau, out, sm=None, n_split=0, scratch=None):
        """One decode step in the order a looped model runs it: for each (loop, layer) cell in turn,
        append the new token's K, V (storing cells; K, V: [cells][B][1][H][D]) and decode that cell
        with its query. A reuse cell reads the final loop's cache as it stands, which does not hold
        the current token yet (the final loop runs later in the step), so it decodes over
        lens_before tokens; every other cell over lens_after. Advances both length tensors in
        place, so the step can be captured in a graph and replayed."""
        cfg = self.cfg
        for c in range(cfg.n_cells):
            cell = divmod(c, cfg.n_layers)
            share = self.plan[c] == R.SHARE
            if not share:
                self.ctx.append(K[c], V[c], self.bt, lens_before, cell=cell)
            self.ctx.decode(q[c], self.bt, lens_before if share else lens_after, max_len, tau, cell=cell,
                            out=out[c], sel_mask=sm[c] if sm is not None else False, n_split=n_split,
                            scratch=scratch)
        lens_before.add_(1)
        lens_after.add_(1)

    # ------------------------------------------------------------------ oracle inputs
    def oracle_inputs(self, cell_store: int, b: int, kvh: int, n_tokens: int):
        """float64 K, V [n_tokens][D] of one (storage cell, sequence, KV head), drawn by the seeded
        generator for the oracle. Workloads that draw on the GPU draw here on the GPU too (the same
        bits as the host draw; every head of the sequence at once, the last two kept); the library
        plays no part."""
        if not self.gpu_synth:
            _, _, K, V = oracle_row_inputs(self.cfg, cell_store, b, kvh, n_tokens, self.factors)
            return K, V
        cache = self.__dict__.setdefault("_row_cache", {})
        key = (cell_store, b, n_tokens)
        if key not in cache:
            K, V = self.kv_seq_gpu(cell_store, b, 0, n_tokens)
            kb = K[0].view(torch.int16).cpu().numpy().view(np.uint16)
            vb = V[0].view(torch.int16).cpu().numpy().view(np.uint16)
            while len(cache) >= 2:
                cache.pop(next(iter(cache)))
            cache[key] = (kb, vb)
        kb, vb = cache[key]
        return (bf16_bits_to_f32(np.ascontiguousarray(kb[:, kvh])).astype(np.float64),
                bf16_bits_to_f32(np.ascontiguousarray(vb[:, kvh])).astype(np.float64))

    # ------------------------------------------------------------------ inspection
    def record(self, cell: int, b: int, h: int, j: int) -> np.ndarray:
        """Bytes of the record of 16-token block j of (cell, sequence b, KV head h): pages of
        32 tokens hold two consecutive record slots."""
        loop, layer = self.cell_ll(cell)
        st = self.ctx.cell_storage(loop, layer)
        rb = st["record_bytes"]
        per = self.cfg.block_tokens // 16
        slot = int(self.bt_np[b, j // per]) * per + j % per
        off = st["pool_offset"] + (slot * self.cfg.kv_heads + h) * rb
        return self.ws[off:off + rb].cpu().numpy()

    def tail(self, cell: int, b: int, h: int) -> np.ndarray:
        """bf16 bits [2][group][D] of the tail of (cell, slot b, head h)."""
        loop, layer = self.cell_ll(cell)
        st = self.ctx.cell_storage(loop, layer)
        D, G = self.cfg.head_dim, self.cfg.group
        n = 2 * G * D * 2
        off = st["tail_offset"] + (b * self.cfg.kv_heads + h) * n
        return self.ws[off:off + n].cpu().numpy().view(np.uint16).reshape(2, G, D)


def kv_head(cfg: R.Config, h: int) -> int:
    """The KV head query head h reads (grouped queries: h // (query heads per KV head))."""
    return h // (cfg.n_heads // cfg.kv_heads)


def oracle_row_inputs(cfg: R.Config, cell_store: int, b: int, h: int, n_tokens: int, factors=None):
    """History (bf16 bits and float64 values of K and V) of KV head h of a storage cell."""
    kb, vb = R.kv_row_bits(cfg, cell_store, b, h, 0, n_tokens, factors)
    K = bf16_bits_to_f32(kb).astype(np.float64)
    V = bf16_bits_to_f32(vb).astype(np.float64)
    return kb, vb, K, V


def rel_err(o, ref):
    o = np.asarray(o, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.abs(ref).max()
    return float(np.abs(o - ref).max() / (den if den > 0 else 1.0))


def selected_counts(sm: torch.Tensor) -> torch.Tensor:
    """Selected tokens per row of a mask tensor [..][words] (int32 words, on the device)."""
    x = sm.to(torch.int64) & 0xFFFFFFFF
    x = x - ((x >> 1) & 0x55555555)
    x = (x & 0x33333333) + ((x >> 2) & 0x33333333)
    x = (x + (x >> 4)) & 0x0F0F0F0F
    x = ((x * 0x01010101) & 0xFFFFFFFF) >> 24
    return x.sum(-1)


def sel_bits_from_mask(mask_words: np.ndarray, n_q: int) -> np.ndarray:
    w = np.asarray(mask_words, dtype=np.uint32)
    bits = np.unpackbits(w.view(np.uint8), bitorder="little")
    return bits[:n_q].astype(bool)
