"""The native serving-step graph (loopkv_step_graph_create / _launch) on the GPU.

One decode step of a looped model calls the cache cell by cell: for each (loop, layer) in
order, the append of the step's token and the decode of that cell ("LoopKV: Loop-Aware KV
Cache Compression for Serving Looped Transformers", arXiv:2611.04137, Abstract, serving
sentence: the fused kernel runs under a graph). The library captures the whole step (every
append, every decode, the length update) into a HIP graph once; each launch replays it.

Checks: every launch equals the same step run call by call on an identical cache, bit for
bit, with eager work and synchronizations between launches; one-workgroup and split decodes,
grouped queries and groups of 64; the records and tails the graph's appends wrote (inside the
decode launches when every KV head has one query head) equal those of the append calls; rows of
the final state against the fp64 oracle (a reuse cell over the final loop's history without the
step's token).

The split decode inside the graph (a partial and a finishing launch per cell) is checked in
every selection regime, each its own kernel (tau 0, tau > 1, tau 0.01 and 0.001, the KIVI-4
layout), and with rows that read nothing (an unmapped page: NaN rows in every launch).
"""
import numpy as np
import pytest
import torch

from quantized_kv_cache_loopkv_amd import loopkv as lkv
from synth import recipes as R
from tests.harness import Workload
from tests.test_gpu_parity import check_row

pytestmark = pytest.mark.gpu

STEPS = 4


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _workload(Hkv, group, D=128, layout=lkv.LAYOUT_PLANES, lengths=None):
    plan = np.array([[0, 2, 1], [2, 1, 0], [0, 1, 0]], dtype=np.uint8)
    if lengths is None:
        lengths = [95, 517] if group == 32 else [62, 517]   # the first sequence completes a group
    cfg = R.small_config("stepgraph", 3, 3, 2, D, lengths, [0.01], plan=plan, cell_scales=True, shuffled=True,
                         append_steps=STEPS, n_kv_heads=Hkv, group=group)
    wl = Workload(cfg, layout=layout, gpu_synth=False)
    wl.fill()
    return wl


def _bits_equal(x, y):
    """Bit-for-bit equality of two float32 tensors (NaN rows included)."""
    return torch.equal(x.view(torch.int32), y.view(torch.int32))


@pytest.mark.parametrize("n_split,Hkv,group,D", [(0, 0, 32, 128), (3, 0, 32, 128), (0, 1, 64, 128), (2, 1, 64, 128),
                                                 (0, 0, 32, 64), (3, 0, 64, 64), (0, 0, 32, 256), (2, 0, 64, 256)])
def test_gpu_step_graph_launches_equal_eager(n_split, Hkv, group, D):
    """Head dims 64 and 256 run their own step geometries (128- and 32-token steps) and their own
    in-launch appends."""
    _need_gpu()
    _graph_vs_eager(_workload(Hkv, group, D), _workload(Hkv, group, D), 0.01, n_split, Hkv, group)


@pytest.mark.parametrize("layout,tau", [(lkv.LAYOUT_PLANES, 0.0), (lkv.LAYOUT_PLANES, 1.1),
                                        (lkv.LAYOUT_PLANES, 0.001), (lkv.LAYOUT_KIVI4, 0.01)])
def test_gpu_step_graph_split_regimes(layout, tau):
    """The graph's split decode in every selection regime (each its own kernel)."""
    _need_gpu()
    _graph_vs_eager(_workload(0, 32, 128, layout), _workload(0, 32, 128, layout), tau, 4, 0, 32)


def test_gpu_step_graph_split_unmapped_page():
    """A sequence whose first page is unmapped: its rows are NaN in every launch (partials
    marked invalid, rows written by the finishing launch); the other sequences' rows stay exact
    over every launch."""
    _need_gpu()
    lengths = [95, 517, 300]
    ea, gb = _workload(0, 32, 128, lengths=lengths), _workload(0, 32, 128, lengths=lengths)
    for wl in (ea, gb):
        wl.bt[2, 0] = -1
    _graph_vs_eager(ea, gb, 0.01, 5, 0, 32, nan_seqs=(2,))


def _graph_vs_eager(ea, gb, tau, n_split, Hkv, group, nan_seqs=()):
    cfg = ea.cfg
    C, B, H, D = cfg.n_cells, cfg.batch, cfg.n_heads, cfg.head_dim
    max_len = max(cfg.lengths) + STEPS
    words = (max_len + 31) // 32
    inputs = [ea.append_inputs(s) for s in range(STEPS)]
    qs = [ea.q_all(s) for s in range(STEPS)]
    scratch = None
    if n_split:
        scratch = torch.empty(ea.ctx.split_scratch_bytes(B, max_len, n_split, cell=(0, 0)), dtype=torch.uint8,
                              device="cuda")

    # call by call on cache A
    lb = torch.tensor(cfg.lengths, dtype=torch.int32, device="cuda")
    la = lb + 1
    ref = []
    for s in range(STEPS):
        out = torch.zeros((C, B, H, D), dtype=torch.float32, device="cuda")
        sm = torch.zeros((C, B, H, words), dtype=torch.int32, device="cuda")
        K, V, _, _ = inputs[s]
        ea.serving_step(K, V, qs[s], lb, la, max_len, tau, out, sm, n_split=n_split, scratch=scratch)
        ref.append((out.clone(), sm.clone()))
    torch.cuda.synchronize()

    # the same steps on cache B through one native graph
    sK = torch.zeros_like(inputs[0][0])
    sV = torch.zeros_like(inputs[0][1])
    sq = torch.zeros_like(qs[0])
    slb = torch.tensor(cfg.lengths, dtype=torch.int32, device="cuda")
    sla = slb + 1
    out = torch.zeros((C, B, H, D), dtype=torch.float32, device="cuda")
    sm = torch.zeros((C, B, H, words), dtype=torch.int32, device="cuda")
    g = gb.ctx.step_graph(sK, sV, sq, gb.bt, slb, sla, max_len, tau, out, sel_mask=sm, n_split=n_split,
                          scratch=scratch)
    torch.cuda.synchronize()
    assert torch.equal(slb.cpu(), torch.tensor(cfg.lengths, dtype=torch.int32))   # creation ran nothing
    for s in range(STEPS):
        K, V, _, _ = inputs[s]
        sK.copy_(K)
        sV.copy_(V)
        sq.copy_(qs[s])
        out.fill_(float("nan"))   # eager work between launches
        g.launch()
        torch.cuda.synchronize()
        print(f"n_split={n_split} Hkv={Hkv} group={group} D={D} tau={tau} launch {s}", flush=True)
        assert _bits_equal(out, ref[s][0]), f"launch {s}: outputs differ"
        assert torch.equal(sm, ref[s][1]), f"launch {s}: selections differ"
    assert torch.equal(slb.cpu(), torch.tensor([n + STEPS for n in cfg.lengths], dtype=torch.int32))
    assert torch.equal(sla.cpu(), torch.tensor([n + STEPS + 1 for n in cfg.lengths], dtype=torch.int32))
    g.close()
    # the graph's appends (inside the decode launches with one query head per KV head) wrote the
    # same records and tails as the append calls
    G = cfg.group
    kivi = ea.layout == lkv.LAYOUT_KIVI4
    for c in ea.storing_cells():
        # the record's data (planes and meta); the bytes after it pad the record to a 256-byte
        # multiple (D = 64 with groups of 64) and are never written
        used = (8 * D if ea.plan[c] == R.Q2 and not kivi else 16 * D) + 2 * (64 * D // G)
        for b, n0 in enumerate(cfg.lengths):
            if b in nan_seqs:   # unmapped pages: nothing to compare
                continue
            n = n0 + STEPS
            for h in range(cfg.kv_heads):
                for j in range(G * (n // G) // 16):
                    assert np.array_equal(ea.record(c, b, h, j)[:used], gb.record(c, b, h, j)[:used]), \
                        f"record c={c} b={b} h={h} j={j}"
                ta, tb = ea.tail(c, b, h), gb.tail(c, b, h)
                for t in range(G * (n // G), n):
                    assert np.array_equal(ta[:, t % G], tb[:, t % G]), f"tail c={c} b={b} h={h} t={t}"

    q = qs[-1]
    o_last, s_last = ref[-1]
    for c in range(C):
        share = ea.plan[c] == R.SHARE
        for b, n0 in enumerate(cfg.lengths):
            if b in nan_seqs:
                assert torch.isnan(o_last[c, b]).all(), f"cell={c} b={b}: expected NaN rows"
                continue
            n = n0 + STEPS - (1 if share else 0)
            for h in range(H):
                check_row(ea, o_last, s_last, q, c, b, h, tau, n, f"cell={c} b={b} h={h} n={n}")
