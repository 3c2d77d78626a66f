"""A cell pool above 4 GiB: 131,072 16-token blocks x 16 KV heads x 2560-byte records (5.4 GB),
the pool a batch of 128 sequences reserved at 16K tokens needs. The decode then addresses
records with 64-bit offsets. Two sequences are paged into the top of the pool and across the
4 GiB boundary; their records are checked bit for bit and every row against the fp64 oracle
(one-workgroup and split decodes, tau 0, 0.01 and 1.1; the KIVI-4 layout)."""
import math

import numpy as np
import pytest
import torch

import quantized_kv_cache_loopkv_amd as lkv
from oracle import loopkv_oracle as O
from tests.harness import rel_err, sel_bits_from_mask

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

NUM_BLOCKS = 131072
H, D = 16, 128


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("layout", [lkv.LAYOUT_PLANES, lkv.LAYOUT_KIVI4])
def test_gpu_pool_above_4gib(layout):
    _need_gpu()
    rec = 20 * D
    boundary = (1 << 32) // (H * rec)          # first block whose records start past 4 GiB
    lengths = [3000, 2085]
    rng = np.random.default_rng(17)
    per = max(lengths) // 16 + 1
    top = rng.permutation(np.arange(NUM_BLOCKS - per, NUM_BLOCKS))
    across = rng.permutation(np.arange(boundary - per // 2, boundary - per // 2 + per))
    bt_np = np.stack([top, across]).astype(np.int32)
    assert bt_np.max() == NUM_BLOCKS - 1 and (bt_np[1] < boundary).any() and (bt_np[1] >= boundary).any()
    ctx = lkv.Context(1, 1, H, D, NUM_BLOCKS, 2, layout)
    ctx.plan([lkv.CELL_Q4])
    ws = torch.empty(ctx.workspace_bytes(), dtype=torch.uint8, device="cuda")
    assert ws.numel() > (1 << 32)
    ctx.bind(ws)
    bt = torch.from_numpy(bt_np).cuda()
    Ks = [rng.standard_normal((N, H, D)).astype(np.float32) for N in lengths]
    Vs = [rng.standard_normal((N, H, D)).astype(np.float32) for N in lengths]
    Ks = [torch.tensor(k).to(torch.bfloat16) for k in Ks]
    Vs = [torch.tensor(v).to(torch.bfloat16) for v in Vs]
    for b, N in enumerate(lengths):
        ctx.append(Ks[b].view(1, N, H, D).cuda(), Vs[b].view(1, N, H, D).cuda(), bt[b:b + 1].contiguous(),
                   torch.zeros(1, dtype=torch.int32, device="cuda"), cell=(0, 0),
                   seq_slots=torch.tensor([b], dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    Kd = [k.float().numpy().astype(np.float64) for k in Ks]
    Vd = [v.float().numpy().astype(np.float64) for v in Vs]
    # records far above 4 GiB, bit for bit
    st = ctx.cell_storage(0, 0)
    rb = st["record_bytes"]
    for b in range(2):
        for h in (0, H - 1):
            qh = O.quantize_history(Kd[b][:, h], Vd[b][:, h], 4)
            for j in (0, 7, qh["n_q"] // 16 - 1):
                off = st["pool_offset"] + (int(bt_np[b, j]) * H + h) * rb
                got = ws[off:off + rb].cpu().numpy()
                assert np.array_equal(got, O.pack_block(qh, j, layout)), f"record b={b} h={h} j={j}"
    lens = torch.tensor(lengths, dtype=torch.int32, device="cuda")
    q = (rng.standard_normal((2, H, D)) * 2.0).astype(np.float32)
    qd = torch.tensor(q).cuda()
    sig = float(np.float32(1.0 / math.sqrt(D)))
    kind = "kivi4" if layout == lkv.LAYOUT_KIVI4 else O.KIND_Q4
    for tau in (0.0, 0.01, 1.1):
        for ns in (0, 5):
            out, sm = ctx.decode(qd, bt, lens, max(lengths), tau, cell=(0, 0), sel_mask=True, n_split=ns)
            torch.cuda.synchronize()
            out, sm = out.cpu().numpy(), sm.cpu().numpy()
            worst = 0.0
            for b, N in enumerate(lengths):
                n_q = 32 * (N // 32)
                for h in range(H):
                    o_ref, sel_ref, phat = O.decode_row(q[b, h].astype(np.float64), Kd[b][:, h], Vd[b][:, h], kind,
                                                        tau, sig)
                    sel = sel_bits_from_mask(sm[b, h], n_q)
                    excused = np.abs(phat[:n_q] - tau) <= 1e-5
                    assert not ((sel != sel_ref) & ~excused).any(), f"selection b={b} h={h} tau={tau}"
                    if (sel != sel_ref).any():
                        o_ref, _, _ = O.decode_row(q[b, h].astype(np.float64), Kd[b][:, h], Vd[b][:, h], kind, tau,
                                                   sig, sel_override=sel)
                    err = rel_err(out[b, h], o_ref)
                    assert err <= 2e-3, f"b={b} h={h} tau={tau} split={ns}: rel err {err:.3e}"
                    worst = max(worst, err)
            print(f"pool {ws.numel() / 2**30:.2f} GiB layout={layout} tau={tau} split={ns}: max rel err {worst:.2e}",
                  flush=True)
