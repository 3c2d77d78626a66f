"""The correction paths of selected tokens (4-bit target, 0 < tau <= 1) on crafted rows.

The decode reads every token's high bits once, with a running softmax, and afterwards
corrects the selected tokens from their low bits. These rows push that scheme to its edges:

* drop:  a coarse winner whose low bits lower its score by about 13 nats, so the correction
         removes nearly all of the row's coarse weight (the kernel then recomputes the row's
         values from the final scores);
* rise:  a coarse winner whose low bits raise its score above the coarse maximum (a new
         running maximum during the corrections);
* many:  random rows at a small tau, so that many groups in several 64-group spans hold
         selected tokens.

Each row is compared with the fp64 oracle: selection bit-exact outside the 1e-5 tie band,
output within 2e-3 (max |o - ref| / max |ref|). K and V are built here, rounded to bf16 once,
and the same bf16 values feed both sides.
"""
import math

import numpy as np
import pytest
import torch

import quantized_kv_cache_loopkv_amd as lkv
from oracle import loopkv_oracle as O
from tests.harness import rel_err, sel_bits_from_mask

pytestmark = pytest.mark.gpu

TOL = 2e-3
TIE = 1e-5


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _bf16(x):
    return torch.tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)


def _decode_one(K, V, q, tau, n_split=0, group=32):
    """Append K, V ([N][D] bf16 tensors, one head) to a fresh one-cell 4-bit cache and decode q
    (n_split > 0: the split decode)."""
    N, D = K.shape
    nb = N // 16 + 2
    ctx = lkv.Context(1, 1, 1, D, nb, 1, group_size=group)
    ctx.plan([lkv.CELL_Q4])
    ws = torch.zeros(ctx.workspace_bytes(), dtype=torch.uint8, device="cuda")
    ctx.bind(ws)
    bt = torch.arange(nb, dtype=torch.int32, device="cuda").view(1, nb)
    lens = torch.zeros(1, dtype=torch.int32, device="cuda")
    ctx.append(K.view(1, N, 1, D).cuda().contiguous(), V.view(1, N, 1, D).cuda().contiguous(), bt, lens,
               cell=(0, 0))
    lens = torch.full((1,), N, dtype=torch.int32, device="cuda")
    qd = torch.tensor(np.asarray(q, dtype=np.float32)).view(1, 1, D).cuda()
    out, sm = ctx.decode(qd, bt, lens, N, tau, cell=(0, 0), sel_mask=True, n_split=n_split)
    torch.cuda.synchronize()
    return out.view(D).cpu().numpy(), sm.view(-1).cpu().numpy()


def _check(K, V, q, tau, label, n_split=0, group=32):
    N, D = K.shape
    o_gpu, sm = _decode_one(K, V, q, tau, n_split, group)
    Kd, Vd = K.float().numpy().astype(np.float64), V.float().numpy().astype(np.float64)
    sig = float(np.float32(1.0 / math.sqrt(D)))
    o_ref, sel_ref, phat = O.decode_row(np.asarray(q, np.float64), Kd, Vd, O.KIND_Q4, tau, sig, group=group)
    n_q = group * (N // group)
    sel_gpu = sel_bits_from_mask(sm, n_q)
    excused = np.abs(phat[:n_q] - tau) <= TIE
    bad = (sel_gpu != sel_ref) & ~excused
    assert not bad.any(), f"{label}: selection differs at {np.flatnonzero(bad)[:10]}"
    if (sel_gpu != sel_ref).any():
        o_ref, _, _ = O.decode_row(np.asarray(q, np.float64), Kd, Vd, O.KIND_Q4, tau, sig, sel_override=sel_gpu,
                                   group=group)
    err = rel_err(o_gpu, o_ref)
    assert err <= TOL, f"{label}: rel err {err:.3e}"
    return err, int(sel_ref.sum())


def _winner_row(D, N, mode, seed):
    """Group 0 holds a coarse winner (token 5) with every channel at code 12 ('drop': high bits 3,
    low bits 0, so the midpoint overestimates it) or code 15 ('rise': the midpoint
    underestimates it); the rest of group 0 pins each channel's range to [-A, A]; every other
    group is zero (its scores are exactly 0). q = 1 on all channels."""
    A = 13.0 / (0.2 * math.sqrt(D))   # coarse-to-refined score change of about 13 nats
    K = np.zeros((N, D), np.float32)
    K[:32] = -A
    if mode == "drop":
        for h in range(D // 32):   # tokens 8.. hold the maximum of 32 channels each
            K[8 + h, 32 * h:32 * (h + 1)] = A
        K[5] = -A + 12.0 * (2.0 * A / 15.0)
    else:
        K[5] = A
    rng = np.random.default_rng(seed)
    V = rng.standard_normal((N, D)).astype(np.float32)
    return _bf16(K), _bf16(V), np.ones(D, np.float32)


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("mode", ["drop", "rise"])
def test_gpu_correction_of_coarse_winner(D, mode):
    _need_gpu()
    N = 512 + 7   # a tail of 7 exact tokens as well
    K, V, q = _winner_row(D, N, mode, seed=11)
    err, n_sel = _check(K, V, q, 0.01, f"{mode} D={D}")
    assert n_sel >= 1
    print(f"{mode} D={D}: rel err {err:.2e}, selected {n_sel}", flush=True)


@pytest.mark.parametrize("D", [64, 128, 256])
def test_gpu_many_selected_groups(D):
    _need_gpu()
    rng = np.random.default_rng(5 + D)
    N = 6000
    K = _bf16(rng.standard_normal((N, D)) * 1.5)
    V = _bf16(rng.standard_normal((N, D)))
    q = (rng.standard_normal(D) * 2.0).astype(np.float32)
    for tau in (1e-4, 1e-3):
        err, n_sel = _check(K, V, q, tau, f"many D={D} tau={tau}")
        print(f"many D={D} tau={tau}: rel err {err:.2e}, selected {n_sel}", flush=True)


# Generator rows (seed, head dim, sequence, head, query gain, tau) whose selected coarse winner
# loses most of its weight to its low bits: the removed coarse weight is tens to hundreds of
# times the weight the row keeps. The values sum carries each weight at 16 bits against the
# largest weight of its 16-token block, so the winner's neighbours are rounded coarsely; these
# rows put that rounding, amplified by removed / kept, above the tolerance unless the row's
# values are recomputed from the final scores.
_PEAKED = [(25, 128, 0, 0, 5.0, 0.05), (38, 64, 0, 1, 5.0, 0.05), (27, 64, 0, 3, 5.0, 0.05),
           (18, 64, 0, 1, 3.0, 0.05), (29, 256, 0, 2, 5.0, 0.05)]


def _removed_over_kept(q, K, V, tau, sig):
    """Coarse weight of the selected tokens over the final weight of the row (oracle values)."""
    qh = O.quantize_history(K, V, 4)
    n_q = qh["n_q"]
    coarse = sig * (np.concatenate([O.dequant_hi(qh, "k"), K[n_q:]]) @ q)
    _, sel, _ = O.decode_row(q, K, V, O.KIND_Q4, tau, sig, qh=qh)
    refined = coarse.copy()
    refined[:n_q][sel] = sig * (O.dequant_full(qh, "k")[sel] @ q)
    m = coarse.max()
    return np.exp(coarse[:n_q][sel] - m).sum() / np.exp(refined - m).sum()


@pytest.mark.parametrize("n_split", [0, 3])
@pytest.mark.parametrize("row", _PEAKED)
def test_gpu_peaked_rows(row, n_split):
    _need_gpu()
    from synth import recipes as R
    from tests.harness import oracle_row_inputs
    seed, D, b, h, gain, tau = row
    cfg = R.small_config("peak", 1, 1, 4, D, [700, 1300], [tau], outlier_count=3, outlier_mult=10.0, seed=seed)
    N = cfg.lengths[b]
    _, _, K, V = oracle_row_inputs(cfg, 0, b, h, N, R.factor_table(cfg))
    q = (R.q_values(cfg, 0, 0, b, h) * gain).astype(np.float32)
    ratio = _removed_over_kept(q.astype(np.float64), K, V, tau, float(np.float32(1.0 / math.sqrt(D))))
    assert 20 < ratio < 1024, ratio
    err, n_sel = _check(_bf16(K), _bf16(V), q, tau, f"peaked {row} split={n_split}", n_split=n_split)
    print(f"peaked {row} split={n_split}: removed/kept {ratio:.0f}, rel err {err:.2e}, selected {n_sel}",
          flush=True)


# Generator rows (found by a search with the oracle alone) whose removed / kept coarse weight
# lies in [4, 8): just under the ratio at which the kernel recomputes a row's values, so the
# corrected values sum keeps the selected winner's block rounding, amplified by up to 8x.
_NEAR_GUARD = [(0, 128, 1, 0, 5.0, 0.05), (2, 128, 0, 2, 3.0, 0.05), (2, 128, 1, 2, 5.0, 0.05),
               (3, 128, 0, 3, 5.0, 0.05), (2, 256, 1, 0, 5.0, 0.05), (6, 256, 1, 3, 5.0, 0.05),
               (0, 256, 1, 0, 5.0, 0.05), (3, 64, 1, 3, 3.0, 0.05), (6, 64, 1, 2, 3.0, 0.05),
               (0, 64, 0, 3, 3.0, 0.05)]


@pytest.mark.parametrize("n_split", [0, 4])
@pytest.mark.parametrize("row", _NEAR_GUARD)
def test_gpu_rows_under_the_recompute_ratio(row, n_split):
    _need_gpu()
    from synth import recipes as R
    from tests.harness import oracle_row_inputs
    seed, D, b, h, gain, tau = row
    cfg = R.small_config("peak", 1, 1, 4, D, [700, 1300], [tau], outlier_count=3, outlier_mult=10.0, seed=seed)
    N = cfg.lengths[b]
    _, _, K, V = oracle_row_inputs(cfg, 0, b, h, N, R.factor_table(cfg))
    q = (R.q_values(cfg, 0, 0, b, h) * gain).astype(np.float32)
    ratio = _removed_over_kept(q.astype(np.float64), K, V, tau, float(np.float32(1.0 / math.sqrt(D))))
    assert 4.0 <= ratio < 8.0, ratio
    err, n_sel = _check(_bf16(K), _bf16(V), q, tau, f"near-guard {row} split={n_split}", n_split=n_split)
    print(f"near-guard {row} split={n_split}: removed/kept {ratio:.2f}, rel err {err:.2e}, selected {n_sel}",
          flush=True)
