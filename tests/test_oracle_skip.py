"""Pins of the oracle's token-skipping mode (the ablation of the abstract's sentence on
skipping low-attention values; CPU only).

"LoopKV: Loop-Aware KV Cache Compression for Serving Looped Transformers" (arXiv:2611.04137),
Abstract (sentence on skipping): dropping the values of small attention weight to save
reads lets errors grow from loop to loop, which is why the method reads unselected tokens
at 2 bits instead. The skip mode keeps the
same coarse pass and selection and drops the unselected quantized tokens.

* S1  tau = 0 keeps every token: equals full 4-bit attention (closed form);
* S2  tau > 1 keeps only the exact tail: equals textbook attention over the tail, and 0
      when there is no tail;
* S3  tiny rows: exact-rational quantizer and 50-digit softmax over the kept set;
* S4  the values of a dropped token do not reach the output (they do in the method);
* S5  keeping every token by override equals the method with the same override.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import loopkv_oracle as O
from tests import brute
from tests.test_oracle_pins import _row


@pytest.mark.parametrize("N", [64, 300, 1000])
def test_s1_tau0_keeps_everything(N):
    rng = np.random.default_rng(N + 1)
    q, K, V = _row(rng, N, 64, outliers=4)
    sig = 1 / 8
    o, sel, _ = O.decode_row(q, K, V, O.KIND_Q4, 0.0, sig, skip=True)
    qh = O.quantize_history(K, V, 4)
    n_q = qh["n_q"]
    Kt = np.concatenate([O.dequant_full(qh, "k"), K[n_q:]])
    Vt = np.concatenate([O.dequant_full(qh, "v"), V[n_q:]])
    ref = O.attention_reference(q, Kt, Vt, sig)
    assert sel.all()
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


@pytest.mark.parametrize("N", [64, 77, 300])
def test_s2_tau_above_one_keeps_the_tail(N):
    rng = np.random.default_rng(N + 2)
    q, K, V = _row(rng, N, 128, outliers=3, mult=10)
    sig = 128 ** -0.5
    o, sel, _ = O.decode_row(q, K, V, O.KIND_Q4, 1.5, sig, skip=True)
    assert not sel.any()
    n_q = 32 * (N // 32)
    if N == n_q:
        assert np.all(o == 0)
    else:
        ref = O.attention_reference(q, K[n_q:], V[n_q:], sig)
        np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


@pytest.mark.parametrize("N", [32, 33, 64, 65])
def test_s3_tiny_rows_brute_force(N):
    D = 32
    rng = np.random.default_rng(500 + N)
    q, K, V = _row(rng, N, D)
    q = q * 3.0
    sig = D ** -0.5
    tau = 0.03
    n_q = 32 * (N // 32)
    Kq, Khi, Vq = K.copy(), K.copy(), V.copy()
    for g in range(n_q // 32):
        for d in range(D):
            codes, s, z, flagged = brute.quantize_exact(K[32 * g:32 * g + 32, d], 4)
            assert not flagged
            for i, c in enumerate(codes):
                Kq[32 * g + i, d] = float(z + c * s)
                Khi[32 * g + i, d] = float(z + (4 * (c // 4) + Fraction(3, 2)) * s)
    for t in range(n_q):
        codes, s, z, flagged = brute.quantize_exact(V[t, :32], 4)
        assert not flagged
        for i, c in enumerate(codes):
            Vq[t, i] = float(z + c * s)
    _, phat = brute.attention_mp(q, Khi, V, sig)   # coarse weights need only the keys
    sel = [float(p) >= tau for p in phat[:n_q]]
    near = [abs(float(p) - tau) < 1e-12 for p in phat[:n_q]]
    keep = [t for t in range(N) if t >= n_q or sel[t]]
    o, osel, _ = O.decode_row(q, K, V, O.KIND_Q4, tau, sig, skip=True)
    for t in range(n_q):
        if not near[t]:
            assert osel[t] == sel[t]
    if not keep:
        assert np.all(o == 0)
        return
    ref, _ = brute.attention_mp(q, Kq[keep], Vq[keep], sig)
    ref = np.array([float(x) for x in ref])
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
    assert 0 < len(keep) < N


def test_s4_dropped_values_do_not_reach_the_output():
    rng = np.random.default_rng(9)
    q, K, V = _row(rng, 256, 64, outliers=2)
    q = q * 3
    sig = 1 / 8
    o, sel, _ = O.decode_row(q, K, V, O.KIND_Q4, 0.01, sig, skip=True)
    o_m, _, _ = O.decode_row(q, K, V, O.KIND_Q4, 0.01, sig)
    t = int(np.flatnonzero(~sel)[0])
    V2 = V.copy()
    V2[t] = V2[t] * 4 + 1   # changes only token t's own V groups
    o2, sel2, _ = O.decode_row(q, K, V2, O.KIND_Q4, 0.01, sig, skip=True)
    o2_m, _, _ = O.decode_row(q, K, V2, O.KIND_Q4, 0.01, sig)
    assert np.array_equal(sel, sel2)
    np.testing.assert_array_equal(o, o2)
    assert not np.allclose(o_m, o2_m)


def test_s5_override_all_equals_method():
    rng = np.random.default_rng(10)
    q, K, V = _row(rng, 200, 64)
    sig = 1 / 8
    ones = np.ones(192, dtype=bool)
    a, _, _ = O.decode_row(q, K, V, O.KIND_Q4, 0.01, sig, sel_override=ones, skip=True)
    b, _, _ = O.decode_row(q, K, V, O.KIND_Q4, 0.01, sig, sel_override=ones)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-15)
