"""The one-token append of a decode step on the GPU.

A decode step appends one token per sequence to every storing cell before the cell is read
("LoopKV: Loop-Aware KV Cache Compression for Serving Looped Transformers",
arXiv:2611.04137, Abstract: every cell keeps its own KV cache, 4-bit or 2-bit). Such an
append runs in its own kernel: one workgroup per (cell, sequence) for every KV head, writing
the token into its tail slot, or, when the token completes a group, quantizing and packing
the group of each head. Built token by token this way, a cache must hold, byte for byte, the
records and live tail slots of the same history appended in bulk (the group kernels): per
cell and over a whole plan in one call, bf16 and f32 inputs (f32 rounded to bf16), groups of
32 and 64, head dims 64, 128 and 256, grouped queries, ragged lengths (a sequence past its
length gets a negative length: the append skips it).
"""
import numpy as np
import pytest
import torch

from synth import recipes as R
from tests.harness import Workload

pytestmark = pytest.mark.gpu

LENGTHS = [70, 97, 64, 33]


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("D,group,Hkv,f32,whole", [(64, 32, 0, False, False), (128, 64, 2, True, True),
                                                   (256, 32, 0, False, True), (128, 32, 4, True, False)])
def test_gpu_one_token_appends_equal_bulk(D, group, Hkv, f32, whole):
    _need_gpu()
    plan = np.array([[2, 1], [0, 1]], dtype=np.uint8)   # a reuse cell, 2-bit and 4-bit storage
    cfg = R.small_config("token", 2, 2, 4, D, LENGTHS, [0.01], plan=plan, n_kv_heads=Hkv, group=group,
                         shuffled=True)
    bulk = Workload(cfg, gpu_synth=False)
    bulk.fill()
    tok = Workload(cfg, gpu_synth=False)
    B, N, G = cfg.batch, max(LENGTHS), cfg.group
    cells = tok.storing_cells()
    chunks = {c: tok.kv_chunk(c, 0, N) for c in cells}   # bf16 [B][N][KV heads][D]

    def as_input(x):
        # f32 input with sub-bf16 noise that the append's rounding removes
        return (x.float() * (1 + 2 ** -12)).contiguous() if f32 else x.contiguous()

    for t in range(N):
        lens = torch.tensor([t if t < n else -1 for n in LENGTHS], dtype=torch.int32, device="cuda")
        if whole:
            K = torch.zeros((cfg.n_cells, B, 1, cfg.kv_heads, D), dtype=torch.bfloat16, device="cuda")
            V = torch.zeros_like(K)
            for c in cells:
                K[c] = chunks[c][0][:, t:t + 1]
                V[c] = chunks[c][1][:, t:t + 1]
            tok.ctx.append(as_input(K), as_input(V), tok.bt, lens)
        else:
            for c in cells:
                tok.ctx.append(as_input(chunks[c][0][:, t:t + 1]), as_input(chunks[c][1][:, t:t + 1]), tok.bt, lens,
                               cell=tok.cell_ll(c))
    torch.cuda.synchronize()
    print(f"D={D} group={group} Hkv={Hkv} f32={f32} whole={whole}: {N} one-token appends", flush=True)
    for c in cells:
        for b, n in enumerate(LENGTHS):
            for h in range(cfg.kv_heads):
                for j in range(G * (n // G) // 16):
                    assert np.array_equal(bulk.record(c, b, h, j), tok.record(c, b, h, j)), f"record c={c} b={b} h={h} j={j}"
                tb, tt = bulk.tail(c, b, h), tok.tail(c, b, h)
                for s in range(n % G):   # the live tail slots
                    assert np.array_equal(tb[:, s], tt[:, s]), f"tail c={c} b={b} h={h} slot={s}"
