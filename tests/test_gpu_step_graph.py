"""The native serving-step graph (loopkv_step_graph_create / _launch) on the GPU.

One decode step of a looped model calls the cache cell by cell: for each (loop, layer) in
order, the append of the step's token and the decode of that cell ("LoopKV: Loop-Aware KV
Cache Compression for Serving Looped Transformers", arXiv:2611.04137, Abstract, serving
sentence: the fused kernel runs under a graph). The library captures the whole step (every
append, every decode, the length update) into a HIP graph once; each launch replays it.

Checks: every launch equals the same step run call by call on an identical cache, bit for
bit, with eager work and synchronizations between launches; one-workgroup and split decodes,
grouped queries and groups of 64; rows of the final state against the fp64 oracle (a reuse
cell over the final loop's history without the step's token).
"""
import numpy as np
import pytest
import torch

from synth import recipes as R
from tests.harness import Workload
from tests.test_gpu_parity import check_row

pytestmark = pytest.mark.gpu

STEPS = 4


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _workload(Hkv, group):
    plan = np.array([[0, 2, 1], [2, 1, 0], [0, 1, 0]], dtype=np.uint8)
    lengths = [95, 517] if group == 32 else [62, 517]   # the first sequence completes a group
    cfg = R.small_config("stepgraph", 3, 3, 2, 128, lengths, [0.01], plan=plan, cell_scales=True, shuffled=True,
                         append_steps=STEPS, n_kv_heads=Hkv, group=group)
    wl = Workload(cfg, gpu_synth=False)
    wl.fill()
    return wl


@pytest.mark.parametrize("n_split,Hkv,group", [(0, 0, 32), (3, 0, 32), (0, 1, 64), (2, 1, 64)])
def test_gpu_step_graph_launches_equal_eager(n_split, Hkv, group):
    _need_gpu()
    tau = 0.01
    ea, gb = _workload(Hkv, group), _workload(Hkv, group)
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
        print(f"n_split={n_split} Hkv={Hkv} group={group} launch {s}", flush=True)
        assert torch.equal(out, ref[s][0]), f"launch {s}: outputs differ"
        assert torch.equal(sm, ref[s][1]), f"launch {s}: selections differ"
    assert torch.equal(slb.cpu(), torch.tensor([n + STEPS for n in cfg.lengths], dtype=torch.int32))
    assert torch.equal(sla.cpu(), torch.tensor([n + STEPS + 1 for n in cfg.lengths], dtype=torch.int32))
    g.close()

    q = qs[-1]
    o_last, s_last = ref[-1]
    for c in range(C):
        share = ea.plan[c] == R.SHARE
        for b, n0 in enumerate(cfg.lengths):
            n = n0 + STEPS - (1 if share else 0)
            for h in range(H):
                check_row(ea, o_last, s_last, q, c, b, h, tau, n, f"cell={c} b={b} h={h} n={n}")
