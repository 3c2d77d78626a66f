"""Per-(loop, layer) serving order captured in a HIP graph (torch.cuda.CUDAGraph).

A looped model calls the cache one cell at a time: loop i's queries depend on the layers
before it, so a decode step is, for every (loop, layer) in turn, the append of the new
token's K, V and the decode of that cell. The pages run their fused kernel under a graph
("LoopKV: Loop-Aware KV Cache Compression for Serving Looped Transformers",
arXiv:2611.04137, Abstract, serving sentence); here the whole step (all appends, decodes
and the length updates) is captured once and replayed.

Checks: every replay equals the same step run eagerly on an identical cache, bit for bit,
with eager work and synchronizations between replays; the one-workgroup and split decodes
both run under capture; rows of the final state match the fp64 oracle (a reuse cell over the
final loop's history without the current token).
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


def _workload():
    plan = np.array([[0, 2, 1], [2, 1, 0], [0, 1, 0]], dtype=np.uint8)
    lengths = [95, 517]   # the first sequence completes a group during the steps
    cfg = R.small_config("graph", 3, 3, 2, 128, lengths, [0.01], plan=plan, cell_scales=True, shuffled=True,
                         append_steps=STEPS)
    wl = Workload(cfg, gpu_synth=False)
    wl.fill()
    return wl


@pytest.mark.parametrize("n_split", [0, 3])
def test_gpu_serving_graph_replays_equal_eager(n_split):
    _need_gpu()
    tau = 0.01
    ea, gb = _workload(), _workload()
    cfg = ea.cfg
    C, B, H, D = cfg.n_cells, cfg.batch, cfg.n_heads, cfg.head_dim
    max_len = max(cfg.lengths) + STEPS   # one bound for every step, so that a graph can be reused
    words = (max_len + 31) // 32
    inputs = [ea.append_inputs(s) for s in range(STEPS)]
    qs = [ea.q_all(s) for s in range(STEPS)]
    scratch = None
    if n_split:
        scratch = torch.empty(ea.ctx.split_scratch_bytes(B, max_len, n_split, cell=(0, 0)), dtype=torch.uint8,
                              device="cuda")

    # eager reference on cache A
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

    # the same steps on cache B, captured once and replayed
    sK = torch.zeros_like(inputs[0][0])
    sV = torch.zeros_like(inputs[0][1])
    sq = torch.zeros_like(qs[0])
    slb = torch.tensor(cfg.lengths, dtype=torch.int32, device="cuda")
    sla = slb + 1
    out = torch.zeros((C, B, H, D), dtype=torch.float32, device="cuda")
    sm = torch.zeros((C, B, H, words), dtype=torch.int32, device="cuda")
    # one eager decode first (read only: the cache is unchanged), so that one-time launch
    # attributes are set outside the capture
    gb.ctx.decode(sq[0], gb.bt, sla, max_len, tau, cell=(0, 0), out=out[0], sel_mask=sm[0], n_split=n_split,
                  scratch=scratch)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        gb.serving_step(sK, sV, sq, slb, sla, max_len, tau, out, sm, n_split=n_split, scratch=scratch)
    torch.cuda.synchronize()
    assert torch.equal(slb.cpu(), torch.tensor(cfg.lengths, dtype=torch.int32))   # capture ran nothing
    for s in range(STEPS):
        K, V, _, _ = inputs[s]
        sK.copy_(K)
        sV.copy_(V)
        sq.copy_(qs[s])
        out.fill_(float("nan"))   # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        print(f"n_split={n_split} replay {s}", flush=True)
        assert torch.equal(out, ref[s][0]), f"replay {s}: outputs differ"
        assert torch.equal(sm, ref[s][1]), f"replay {s}: selections differ"
    assert torch.equal(slb.cpu(), torch.tensor([n + STEPS for n in cfg.lengths], dtype=torch.int32))

    # final state against the oracle: each row over its own history (a reuse cell: the final
    # loop's history without the current token)
    q = qs[-1]
    o_last, s_last = ref[-1]
    for c in range(C):
        share = ea.plan[c] == R.SHARE
        for b, n0 in enumerate(cfg.lengths):
            n = n0 + STEPS - (1 if share else 0)
            for h in range(H):
                check_row(ea, o_last, s_last, q, c, b, h, tau, n, f"cell={c} b={b} h={h} n={n}")
