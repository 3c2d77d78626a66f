"""Pins of the fp64 oracle against closed forms, brute force and invariants (CPU only).

The method comes from "LoopKV: Loop-Aware KV Cache Compression for Serving
Looped Transformers" (arXiv:2611.04137), Abstract: per-cell 4-bit / 2-bit /
reuse storage and loop-aware selective fetching of the low bits. The pages give
no formula or worked example, so the pins are:

* P1  tau = 0 selects every quantized token: output == full 4-bit attention;
* P2  tau > 1 selects nothing: output == high-2-bit-only attention;
* P3  a reuse cell gives the final-loop cell's output for the same query;
* P4  a 2-bit target ignores tau and equals attention over 2-bit values;
* P5  tiny rows agree with an exact-rational quantizer and 50-digit attention;
* P6  quantizer invariants; P7 constant values; P8 power-of-two scaling;
* P11 one-token and empty rows; P12 KIVI-4 equals tau = 0; P13 monotone Sel;
* P14 the analytic storage ratio of the 48/29/19 plan.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import loopkv_oracle as O
from tests import brute
from synth import recipes as R
from synth.philox import bf16_bits_to_f32


def _bf16(x):
    """Round a float64 array to bf16 values (exactly, through the bit pattern)."""
    f = np.asarray(x, dtype=np.float32)
    b = f.view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return bf16_bits_to_f32(b.astype(np.uint16)).astype(np.float64)


def _row(rng, N, D, outliers=0, mult=8.0, scale=1.0):
    K = rng.standard_normal((N, D)) * scale
    V = rng.standard_normal((N, D)) * scale
    if outliers:
        ch = rng.choice(D, outliers, replace=False)
        K[:, ch] *= mult
        ch = rng.choice(D, outliers, replace=False)
        V[:, ch] *= mult
    q = rng.standard_normal(D)
    return _bf16(q), _bf16(K), _bf16(V)


# ----------------------------------------------------------------- f16 rounding
def test_f16_round_single_rounding():
    rng = np.random.default_rng(1)
    xs = list(rng.standard_normal(2000) * 10.0 ** rng.uniform(-6, 4, 2000))
    # adversarial: just above / below float16 ties, where float32 would round twice
    for base in [1.0, 3.0, 1000.0, 0.001, 6.1e-5, 2.0 ** -20]:
        e = np.floor(np.log2(base))
        ulp = 2.0 ** (e - 10) if base >= 2.0 ** -14 else 2.0 ** -24
        for k in range(4):
            tie = base + (k + 0.5) * ulp
            xs += [tie, tie + 2.0 ** (e - 40), tie - 2.0 ** (e - 40), -tie]
    for x in xs:
        ref = brute.f16_exact(Fraction(float(x)))
        got = O.f16_round(np.float64(x))
        if ref is None:
            assert np.isinf(got)
        else:
            assert Fraction(float(got)) == ref, x


# ----------------------------------------------------------------- quantizer
@pytest.mark.parametrize("bits", [2, 4])
def test_quantizer_matches_exact_rational(bits):
    rng = np.random.default_rng(bits)
    n_checked = 0
    for trial in range(300):
        scale = 10.0 ** rng.uniform(-3, 3)
        xs = _bf16(rng.standard_normal(32) * scale)
        if trial % 7 == 0:
            xs[rng.integers(32)] *= 30
        codes, s, z = O.quantize_groups(xs[None, :], bits)
        rc, rs, rz, flagged = brute.quantize_exact(xs, bits)
        if flagged:
            continue
        n_checked += 1
        assert Fraction(float(s[0])) == rs and Fraction(float(z[0])) == rz
        assert list(codes[0]) == rc
    assert n_checked > 250


def test_quantizer_invariants():
    """P6: codes in range; extremes hit 0 and M; reconstruction error bounds."""
    rng = np.random.default_rng(7)
    for bits in (2, 4):
        M = (1 << bits) - 1
        for _ in range(200):
            xs = _bf16(rng.standard_normal(32) * 10.0 ** rng.uniform(-2, 2))
            c, s, z = O.quantize_groups(xs[None, :], bits)
            c, s, z = c[0], s[0], z[0]
            assert c.min() >= 0 and c.max() <= M
            assert c[np.argmin(xs)] == 0
            assert c[np.argmax(xs)] == M
            rec = z + s * c
            slack = 2.0 ** -10 * (abs(xs).max() + s * M)
            assert np.all(np.abs(xs - rec) <= s / 2 + slack)
            if bits == 4:
                hi = z + s * (4 * (c >> 2) + 1.5)
                assert np.all(np.abs(xs - hi) <= 2 * s + slack)
                # the full value is the high-only value plus s*(lo - 3/2)
                assert np.allclose(rec, hi + s * ((c & 3) - 1.5), rtol=0, atol=1e-12 * (abs(rec).max() + 1))


def test_quantizer_constant_group():
    xs = np.full(32, 0.75)
    c, s, z = O.quantize_groups(xs[None, :], 4)
    assert s[0] == 0.0 and z[0] == 0.75 and np.all(c == 0)


@pytest.mark.parametrize("G", [32, 64])
def test_history_grouping_axes(G):
    """K groups run over G tokens of one channel; V groups over G channels of one token."""
    rng = np.random.default_rng(3)
    q, K, V = _row(rng, 2 * G + 6, 128)
    qh = O.quantize_history(K, V, 4, G)
    assert qh["n_q"] == 2 * G and qh["ks"].shape == (2, 128) and qh["vs"].shape == (2 * G, 128 // G)
    for g in range(2):
        for d in (0, 17, 63, 127):
            c, s, z = O.quantize_groups(K[G * g:G * g + G, d][None, :], 4)
            assert np.array_equal(qh["kc"][G * g:G * g + G, d], c[0])
            assert qh["ks"][g, d] == s[0] and qh["kz"][g, d] == z[0]
    for t in (0, 31, G - 1, 2 * G - 1):
        for e in range(128 // G):
            c, s, z = O.quantize_groups(V[t, G * e:G * e + G][None, :], 4)
            assert np.array_equal(qh["vc"][t, G * e:G * e + G], c[0])
            assert qh["vs"][t, e] == s[0] and qh["vz"][t, e] == z[0]
    # dequantized values carry their own group's scale and zero
    full = O.dequant_full(qh, "k")
    assert full[G + 5, 9] == qh["kz"][1, 9] + qh["ks"][1, 9] * qh["kc"][G + 5, 9]
    full = O.dequant_full(qh, "v")
    assert full[7, 127] == qh["vz"][7, 127 // G] + qh["vs"][7, 127 // G] * qh["vc"][7, 127]


# ----------------------------------------------------------------- decode closed forms
def _full4(qh, K, V):
    n_q = qh["n_q"]
    Kt = np.concatenate([O.dequant_full(qh, "k"), K[n_q:]])
    Vt = np.concatenate([O.dequant_full(qh, "v"), V[n_q:]])
    return Kt, Vt


def _hi_only(qh, K, V):
    n_q = qh["n_q"]
    Kt = np.concatenate([O.dequant_hi(qh, "k"), K[n_q:]])
    Vt = np.concatenate([O.dequant_hi(qh, "v"), V[n_q:]])
    return Kt, Vt


@pytest.mark.parametrize("G", [32, 64])
@pytest.mark.parametrize("N", [32, 100, 256, 1000])
def test_p1_tau0_equals_full_4bit(N, G):
    rng = np.random.default_rng(N)
    q, K, V = _row(rng, N, 64, outliers=4)
    sig = 1 / 8
    o, sel, _ = O.decode_row(q, K, V, O.KIND_Q4, 0.0, sig, group=G)
    qh = O.quantize_history(K, V, 4, G)
    assert sel.size == G * (N // G)
    ref = O.attention_reference(q, *_full4(qh, K, V), sig)
    assert sel.all()
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


@pytest.mark.parametrize("G", [32, 64])
@pytest.mark.parametrize("tau", [1.0000001, 1.1, 5.0])
def test_p2_tau_above_one_equals_high_bits_only(tau, G):
    rng = np.random.default_rng(11)
    q, K, V = _row(rng, 300, 128, outliers=3, mult=10)
    sig = 128 ** -0.5
    o, sel, _ = O.decode_row(q, K, V, O.KIND_Q4, tau, sig, group=G)
    qh = O.quantize_history(K, V, 4, G)
    ref = O.attention_reference(q, *_hi_only(qh, K, V), sig)
    assert not sel.any()
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_p4_two_bit_target_ignores_tau():
    rng = np.random.default_rng(5)
    q, K, V = _row(rng, 200, 64)
    sig = 0.125
    outs = [O.decode_row(q, K, V, O.KIND_Q2, t, sig)[0] for t in (0.0, 0.01, 2.0)]
    qh = O.quantize_history(K, V, 2)
    n_q = qh["n_q"]
    Kt = np.concatenate([O.dequant_full(qh, "k"), K[n_q:]])
    Vt = np.concatenate([O.dequant_full(qh, "v"), V[n_q:]])
    ref = O.attention_reference(q, Kt, Vt, sig)
    for o in outs:
        assert np.array_equal(o, outs[0])
        np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12)


def test_p3_share_cell_equals_final_loop():
    plan = R.random_plan(4, 24, 0)
    rng = np.random.default_rng(9)
    q, K, V = _row(rng, 96, 64)
    share = [c for c in range(96) if plan.reshape(-1)[c] == O.KIND_SHARE]
    assert len(share) == 19 and all(c < 72 for c in share)
    for c in share[:5]:
        s = O.storage_cell(plan, c)
        assert s == 72 + c % 24
        kind = O.target_kind(plan, c)
        o_share = O.decode_row(q, K, V, kind, 0.01, 0.125)
        o_final = O.decode_row(q, K, V, int(plan.reshape(-1)[s]), 0.01, 0.125)
        assert np.array_equal(o_share[0], o_final[0])
        assert np.array_equal(o_share[1], o_final[1])


def test_p11_one_token_and_empty():
    rng = np.random.default_rng(2)
    q, K, V = _row(rng, 1, 64)
    o, sel, _ = O.decode_row(q, K, V, O.KIND_Q4, 0.01, 0.125)
    assert np.array_equal(o, V[0]) and sel.size == 0
    o, sel, _ = O.decode_row(q, K[:0], V[:0], O.KIND_Q4, 0.01, 0.125)
    assert np.array_equal(o, np.zeros(64))


def test_p7_constant_values():
    """A V group that is constant has scale 0 and dequantizes exactly to its value."""
    rng = np.random.default_rng(4)
    q, K, _ = _row(rng, 160, 64)
    c = _bf16(rng.standard_normal((160, 2)))
    V = np.repeat(c, 32, axis=1)                 # every (token, 32-channel group) constant
    qh = O.quantize_history(K, V, 4)
    assert np.all(qh["vs"] == 0) and np.array_equal(O.dequant_full(qh, "v"), V[:160])
    assert np.array_equal(O.dequant_hi(qh, "v"), V[:160] + 0.0)
    o, _, _ = O.decode_row(q, K, V, O.KIND_Q4, 0.02, 0.125)
    o1, _, _ = O.decode_row(q, K, V, O.KIND_Q4, 0.0, 0.125)
    o2, _, _ = O.decode_row(q, K, V, O.KIND_Q4, 1.1, 0.125)
    # with exact values the output is a convex combination of the rows of V
    assert np.all(o <= V.max(axis=0) + 1e-12) and np.all(o >= V.min(axis=0) - 1e-12)
    Vall = np.full((160, 64), 0.375)
    for tau in (0.0, 0.02, 1.1):
        o3, _, _ = O.decode_row(q, K, Vall, O.KIND_Q4, tau, 0.125)
        np.testing.assert_allclose(o3, 0.375, rtol=1e-14, atol=0)


def test_p8_power_of_two_scaling():
    rng = np.random.default_rng(8)
    q, K, V = _row(rng, 200, 64, outliers=4)
    o, sel, _ = O.decode_row(q, K, V, O.KIND_Q4, 0.01, 0.125)
    o2, sel2, _ = O.decode_row(q, K, V * 8.0, O.KIND_Q4, 0.01, 0.125)
    assert np.array_equal(o2, o * 8.0) and np.array_equal(sel, sel2)
    o3, sel3, _ = O.decode_row(q, K * 4.0, V, O.KIND_Q4, 0.01, 0.125 / 4)
    assert np.array_equal(sel3, sel)
    np.testing.assert_allclose(o3, o, rtol=0, atol=0)


def test_p12_kivi4_equals_tau0():
    rng = np.random.default_rng(12)
    q, K, V = _row(rng, 321, 128)
    a = O.decode_row(q, K, V, "kivi4", 0.5, 0.09)
    b = O.decode_row(q, K, V, O.KIND_Q4, 0.0, 0.09)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_p13_selection_monotone_in_tau():
    rng = np.random.default_rng(13)
    q, K, V = _row(rng, 512, 64, outliers=4)
    q = q * 3
    taus = [0.0, 1e-4, 1e-3, 5e-3, 1e-2, 0.05, 0.3, 1.0, 1.1]
    sels = [O.decode_row(q, K, V, O.KIND_Q4, t, 0.125)[1] for t in taus]
    for a, b in zip(sels, sels[1:]):
        assert np.all(b <= a)
    assert sels[0].all() and not sels[-1].any() and 0 < sels[3].sum() < 480


def test_selection_rule_against_probabilities():
    rng = np.random.default_rng(21)
    q, K, V = _row(rng, 300, 64, outliers=4)
    q = q * 4
    o, sel, phat = O.decode_row(q, K, V, O.KIND_Q4, 0.01, 0.125)
    assert abs(phat.sum() - 1) < 1e-12
    assert np.array_equal(sel, phat[:288] >= 0.01)
    assert 0 < sel.sum() <= 100          # at most 1/tau tokens can reach tau


def test_p14_storage_ratio():
    plan = R.random_plan(4, 24, 0).reshape(-1)
    n4, n2, ns = (plan == 0).sum(), (plan == 1).sum(), (plan == 2).sum()
    assert (n4, n2, ns) == (48, 29, 19)
    D = 128
    ours = n4 * O.record_bytes(D, O.KIND_Q4, O.LAYOUT_PLANES) + n2 * O.record_bytes(D, O.KIND_Q2, O.LAYOUT_PLANES)
    kivi = 96 * O.record_bytes(D, O.KIND_Q4, O.LAYOUT_KIVI4)
    assert O.record_bytes(D, O.KIND_Q4, O.LAYOUT_PLANES) == 16 * 160
    assert O.record_bytes(D, O.KIND_Q2, O.LAYOUT_PLANES) == 16 * 96
    # groups of 64 halve the meta: 144 and 80 bytes per token-head at D = 128
    assert O.record_bytes(D, O.KIND_Q4, O.LAYOUT_PLANES, 64) == 16 * 144
    assert O.record_bytes(D, O.KIND_Q2, O.LAYOUT_PLANES, 64) == 16 * 80
    # D = 64 with groups of 64: 1152 and 640 bytes, padded to 256-byte multiples
    assert O.record_bytes(64, O.KIND_Q4, O.LAYOUT_PLANES, 64) == 1280
    assert O.record_bytes(64, O.KIND_Q2, O.LAYOUT_PLANES, 64) == 768
    assert abs(ours / kivi - (48 * 160 + 29 * 96) / (96 * 160)) < 1e-15
    assert abs(ours / kivi - 0.68125) < 1e-12


# ----------------------------------------------------------------- P5 brute force
@pytest.mark.parametrize("D,G,N", [(D, 32, N) for D in (32, 64) for N in (1, 31, 32, 33, 64, 65)] +
                         [(64, 64, N) for N in (1, 63, 64, 65, 128, 129)])
def test_p5_tiny_rows_brute_force(D, G, N):
    rng = np.random.default_rng(100 * D + N + G)
    q, K, V = _row(rng, N, D, outliers=2 if D == 64 else 0)
    q = q * 2.5
    sig = D ** -0.5
    tau = 0.02
    n_q = G * (N // G)
    # exact-rational quantization over groups of G, independent of the oracle
    Kq = K.copy()
    Khi = K.copy()
    Vq = V.copy()
    Vhi = V.copy()
    for g in range(n_q // G):
        for d in range(D):
            codes, s, z, flagged = brute.quantize_exact(K[G * g:G * g + G, d], 4)
            assert not flagged
            for i, c in enumerate(codes):
                Kq[G * g + i, d] = float(z + c * s)
                Khi[G * g + i, d] = float(z + (4 * (c // 4) + Fraction(3, 2)) * s)
    for t in range(n_q):
        for e in range(D // G):
            codes, s, z, flagged = brute.quantize_exact(V[t, G * e:G * e + G], 4)
            assert not flagged
            for i, c in enumerate(codes):
                Vq[t, G * e + i] = float(z + c * s)
                Vhi[t, G * e + i] = float(z + (4 * (c // 4) + Fraction(3, 2)) * s)
    # coarse softmax in 50 digits, selection, then final attention in 50 digits
    _, phat = brute.attention_mp(q, Khi, Vhi, sig)
    sel = [float(p) >= tau for p in phat[:n_q]]
    near = [abs(float(p) - tau) < 1e-12 for p in phat[:n_q]]
    Kf = np.array([Kq[t] if t < n_q and sel[t] else Khi[t] for t in range(N)])
    Vf = np.array([Vq[t] if t < n_q and sel[t] else Vhi[t] for t in range(N)])
    ref, _ = brute.attention_mp(q, Kf, Vf, sig)
    ref = np.array([float(x) for x in ref])
    o, osel, _ = O.decode_row(q, K, V, O.KIND_Q4, tau, sig, group=G)
    assert osel.size == n_q
    for t in range(n_q):
        if not near[t]:
            assert osel[t] == sel[t]
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
