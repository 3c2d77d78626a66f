"""Brute-force references used to pin the oracle: exact rationals and 50-digit arithmetic.

Nothing here reuses the oracle's code. The float16 rounding enumerates every
finite float16 value; the quantizer searches the nearest level with exact
rational comparisons; attention runs in mpmath at 50 significant digits.
"""
from __future__ import annotations

from fractions import Fraction

import mpmath
import numpy as np

_F16_ALL = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)  # +0 .. 65504
_F16_POS = np.unique(_F16_ALL)   # sorted, exactly representable in float64


def f16_exact(x: Fraction) -> Fraction:
    """Round an exact rational to the nearest float16, ties to the even significand.

    Values at or beyond 65520 (the midpoint above the largest finite float16)
    round to infinity, returned as None."""
    neg = x < 0
    a = -x if neg else x
    if a >= Fraction(65520):
        return None
    vals = _F16_POS
    # find bracketing values lo <= a < hi
    i = int(np.searchsorted(vals, float(a), side="right")) - 1
    i = max(0, min(i, len(vals) - 1))
    # float(a) may round; correct the bracket with exact comparisons
    while i > 0 and Fraction(vals[i]) > a:
        i -= 1
    while i + 1 < len(vals) and Fraction(vals[i + 1]) <= a:
        i += 1
    lo = Fraction(vals[i])
    if lo == a or i + 1 >= len(vals):
        r = lo
    else:
        hi = Fraction(vals[i + 1])
        mid = (lo + hi) / 2
        if a < mid:
            r = lo
        elif a > mid:
            r = hi
        else:
            # tie: pick the one whose float16 significand is even
            bits_lo = int(np.float16(vals[i]).view(np.uint16))
            r = lo if bits_lo % 2 == 0 else hi
    return -r if neg else r


def quantize_exact(xs, bits):
    """Exact-rational quantizer of one group: (codes, scale, zero, flagged).

    zero = f16(min), scale = f16((max - min) / M) rounded from the exact
    quotient, code = nearest level z + k*s for k in 0..M (ties to even k).
    ``flagged`` is True when rounding the float64 quotient instead of the exact
    one could change a result (the two definitions then legitimately differ)."""
    M = (1 << bits) - 1
    fx = [Fraction(float(v)) for v in xs]
    mn, mx = min(fx), max(fx)
    z = f16_exact(mn)
    exact_q = (mx - mn) / M
    s = f16_exact(exact_q)
    s64 = f16_exact(Fraction(float((float(mx) - float(mn)) / M)))
    flagged = s64 != s
    codes = []
    for v in fx:
        if s == 0:
            codes.append(0)
            continue
        best_k, best_d = None, None
        for k in range(M + 1):
            d = abs(v - (z + k * s))
            if best_d is None or d < best_d or (d == best_d and k % 2 == 0):
                best_k, best_d = k, d
        # is the exact quotient within a hair of (but not at) a rounding boundary?
        # An exact tie is representable in float64 and rounds to even on both sides.
        t = (v - z) / s
        frac = t - int(t) if t >= 0 else t - int(t) + 1
        if 0 < abs(frac - Fraction(1, 2)) < Fraction(1, 10 ** 9):
            flagged = True
        codes.append(best_k)
    return codes, s, z, flagged


def attention_mp(q, K, V, sm_scale, dps=50):
    """Softmax attention in mpmath at ``dps`` digits; inputs are exact binary floats."""
    with mpmath.workdps(dps):
        sig = mpmath.mpf(float(sm_scale))
        s = [sig * mpmath.fsum(mpmath.mpf(float(a)) * mpmath.mpf(float(b)) for a, b in zip(q, k)) for k in K]
        m = max(s)
        e = [mpmath.exp(x - m) for x in s]
        tot = mpmath.fsum(e)
        D = len(V[0])
        return [mpmath.fsum(e[t] * mpmath.mpf(float(V[t][d])) for t in range(len(V))) / tot for d in range(D)], \
               [x / tot for x in e]
