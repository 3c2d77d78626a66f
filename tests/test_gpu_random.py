"""Seeded randomized parity sweep: combinations of plan, head dim, grouped queries, lengths,
tau, split, skip, output dtype, quantization group and page size, every row against the fp64
oracle.

The targeted tests cover each feature; this sweep covers their interactions (a constant-term
exchange that only broke at head dim 256 is the kind of mistake it is for). Each case is small
enough for the oracle; the cases are fixed by their seeds.
"""
import numpy as np
import pytest
import torch

from synth import recipes as R
from synth.philox import f32_to_bf16_bits
from tests.harness import Workload
from tests.test_gpu_parity import check_row

pytestmark = pytest.mark.gpu

N_CASES = 32


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _case(seed):
    rng = np.random.default_rng(1000 + seed)
    D = int(rng.choice([64, 128, 256]))
    Hkv = int(rng.choice([1, 2]))
    H = Hkv * int(rng.choice([1, 2, 4]))
    L, NL = int(rng.integers(1, 3)), int(rng.integers(1, 3))
    plan = rng.integers(0, 3, size=(L, NL)).astype(np.uint8)
    plan[L - 1][plan[L - 1] == 2] = 0                  # the final loop cannot reuse
    B = int(rng.integers(1, 4))
    lengths = [int(x) for x in rng.integers(1, 1500, size=B)]
    tau = float(rng.choice([0.0, 1e-3, 0.01, 0.05, 1.5]))
    n_split = int(rng.choice([0, 0, 2, 5]))
    bf16_out = bool(rng.integers(0, 2))
    outliers, q_gain = int(rng.choice([0, 3])), float(rng.choice([1.0, 2.5]))
    group, pages = int(rng.choice([32, 64])), int(rng.choice([16, 32]))
    return dict(D=D, H=H, Hkv=Hkv, plan=plan, lengths=lengths, tau=tau, n_split=n_split, bf16_out=bf16_out,
                outliers=outliers, q_gain=q_gain, group=group, pages=pages)


@pytest.mark.parametrize("seed", range(N_CASES))
def test_gpu_random_case(seed):
    _need_gpu()
    c = _case(seed)
    L, NL = c["plan"].shape
    cfg = R.small_config(f"rnd{seed}", L, NL, c["H"], c["D"], c["lengths"], [c["tau"]], plan=c["plan"],
                         outlier_count=c["outliers"], outlier_mult=10.0, cell_scales=True, shuffled=bool(seed % 2),
                         n_kv_heads=c["Hkv"], seed=seed, group=c["group"], block_tokens=c["pages"])
    print(f"case {seed}: {dict((k, v) for k, v in c.items() if k != 'plan')} plan={c['plan'].tolist()}", flush=True)
    wl = Workload(cfg, gpu_synth=False)
    wl.fill()
    q = wl.q_all() * c["q_gain"]
    q = q.to(torch.bfloat16).float().to(q.dtype)
    out, sm = wl.ctx.decode(q, wl.bt, wl.seq_lens, wl.max_len(), c["tau"], sel_mask=True, n_split=c["n_split"])
    torch.cuda.synchronize()
    for cell in range(L * NL):
        for b, N in enumerate(c["lengths"]):
            for h in range(c["H"]):
                check_row(wl, out, sm, q, cell, b, h, c["tau"], N, f"case {seed} cell={cell} b={b} h={h}")
    if c["bf16_out"]:
        ob = wl.ctx.decode(q, wl.bt, wl.seq_lens, wl.max_len(), c["tau"], out_dtype=torch.bfloat16,
                           n_split=c["n_split"])
        torch.cuda.synchronize()
        assert np.array_equal(ob.view(torch.int16).cpu().numpy().view(np.uint16), f32_to_bf16_bits(out.cpu().numpy()))
    if 0 < c["tau"] <= 1:   # the skip ablation on the same cache (4-bit targets skip)
        from tests.test_gpu_skip import _check_skip_row
        os_, ss = wl.ctx.decode(q, wl.bt, wl.seq_lens, wl.max_len(), c["tau"], sel_mask=True, skip=True)
        torch.cuda.synchronize()
        for cell in range(L * NL):
            for b, N in enumerate(c["lengths"]):
                for h in range(c["H"]):
                    _check_skip_row(wl, os_, ss, q, cell, b, h, c["tau"], N, f"skip case {seed} cell={cell}")
