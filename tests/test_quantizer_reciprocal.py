"""The group quantizer's code rule without a division per element.

The quantizer's code is rint((x - z) / s) with the float64 quotient correctly rounded (the
KIVI-style group quantizer; "LoopKV: Loop-Aware KV Cache Compression for Serving Looped
Transformers", Abstract, sentence on the three storage choices). The kernels compute
y = (x - z) * fl(1 / s) and fall back to the division when y lies within 2^-40 of a rounding
tie k + 1/2. These checks run that rule in numpy float64 (IEEE, as on the GPU) and compare
it with rint of the quotient on quotients drawn at random, on exact ties and on quotients
one ulp from a tie, for the f16 scales the quantizer produces.
"""
import numpy as np


def code_div(d, s, M):
    with np.errstate(all="ignore"):
        q = np.rint(d / s)
    return np.clip(np.where(s == 0, 0.0, q), 0.0, M)


def code_recip(d, s, M):
    with np.errstate(all="ignore"):
        rs = 1.0 / s
        y = d * rs
        near = np.abs(y - np.floor(y) - 0.5) <= 2.0 ** -40
        y = np.where(near, d / s, y)
        r = np.rint(y)
    return np.clip(np.where(s == 0, 0.0, r), 0.0, M), near


def f16_scales(rng, n):
    """Positive finite float16 values (normal and subnormal), as float64."""
    bits = rng.integers(1, 0x7C00, size=n, dtype=np.uint16)
    return bits.view(np.float16).astype(np.float64)


def test_random_quotients_match_the_division():
    rng = np.random.default_rng(0)
    for M in (3.0, 15.0):
        s = f16_scales(rng, 400_000)
        # differences spanning the codes, a little below 0 and above M
        d = s * rng.uniform(-0.7, M + 0.7, size=s.size)
        got, _ = code_recip(d, s, M)
        assert np.array_equal(got, code_div(d, s, M))


def test_exact_ties_take_the_division():
    rng = np.random.default_rng(1)
    s = f16_scales(rng, 200_000)
    k = rng.integers(-1, 16, size=s.size).astype(np.float64)
    d = (k + 0.5) * s                      # exact in float64: few significant bits
    assert np.array_equal(d / s, k + 0.5)  # the quotient is the tie itself
    got, near = code_recip(d, s, 15.0)
    assert near.all()
    assert np.array_equal(got, code_div(d, s, 15.0))
    # ties to even: 2.5 -> 2, 3.5 -> 4
    assert code_recip(np.array([2.5, 3.5]), np.array([1.0, 1.0]), 15.0)[0].tolist() == [2.0, 4.0]


def test_quotients_next_to_ties():
    rng = np.random.default_rng(2)
    s = f16_scales(rng, 200_000)
    k = rng.integers(0, 15, size=s.size).astype(np.float64)
    tie = (k + 0.5) * s
    for d in (np.nextafter(tie, np.inf), np.nextafter(tie, -np.inf),
              np.nextafter(np.nextafter(tie, np.inf), np.inf)):
        got, _ = code_recip(d, s, 15.0)
        assert np.array_equal(got, code_div(d, s, 15.0))


def test_non_finite_and_zero_scale():
    d = np.array([np.inf, -np.inf, np.nan, 1.0, 1.0, np.inf])
    s = np.array([0.5, 0.5, 0.5, np.inf, 0.0, np.inf])
    got, _ = code_recip(d, s, 15.0)
    assert np.array_equal(got, code_div(d, s, 15.0), equal_nan=True)   # NaN stays NaN on both routes
