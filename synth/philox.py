"""Counter-based random numbers: Philox4x32-10 and an exact-arithmetic normal draw.

Philox4x32-10 is the generator of Salmon, Moraes, Dror and Shaw, "Parallel
random numbers: as easy as 1, 2, 3" (SC'11): a 128-bit counter and a 64-bit
key go through ten rounds of two 32x32->64-bit multiplies with the constants
0xD2511F53 and 0xCD9E8D57, the key being bumped by the Weyl constants
0x9E3779B9 and 0xBB67AE85 between rounds.

Normal draw (the same definition is implemented in synth_kernel.hip):

* element ``i`` of stream ``s`` under ``seed`` evaluates Philox at the two
  counters ``(i mod 2^32, i div 2^32, s, 0)`` and ``(..., s, 1)`` with key
  ``(seed mod 2^32, seed div 2^32)``, giving eight 32-bit words, i.e. sixteen
  16-bit halves ``h_0..h_15`` (low half of each word first);
* the first twelve halves are twelve uniforms ``u_j = (h_j + 1/2) / 2^16`` and
  the value is the classic Irwin-Hall approximation ``sum_j u_j - 6`` (mean 0,
  variance 1, support [-6, 6]), which equals ``(sum_j h_j - 393210) / 65536``:
  an integer over a power of two, exact in float32;
* a scaled value ``bf16(z * f)`` multiplies by a float32 factor with one IEEE
  float32 multiply and rounds to bfloat16 to nearest-even on the bit pattern.

Every step is integer arithmetic or a single correctly rounded IEEE operation,
so the host and the GPU produce identical bits.
"""
from __future__ import annotations

import numpy as np

_M0 = np.uint64(0xD2511F53)
_M1 = np.uint64(0xCD9E8D57)
_W0 = np.uint32(0x9E3779B9)
_W1 = np.uint32(0xBB67AE85)
_MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Ten Philox4x32 rounds on uint32 arrays (broadcast together). Returns 4 uint32 arrays."""
    c0 = np.asarray(c0, dtype=np.uint32)
    c1 = np.asarray(c1, dtype=np.uint32)
    c2 = np.asarray(c2, dtype=np.uint32)
    c3 = np.asarray(c3, dtype=np.uint32)
    k0 = np.asarray(k0, dtype=np.uint32)
    k1 = np.asarray(k1, dtype=np.uint32)
    c0, c1, c2, c3, k0, k1 = np.broadcast_arrays(c0, c1, c2, c3, k0, k1)
    c0, c1, c2, c3 = (x.copy() for x in (c0, c1, c2, c3))
    k0 = k0.copy()
    k1 = k1.copy()
    with np.errstate(over="ignore"):
        for r in range(10):
            if r:
                k0 = k0 + _W0
                k1 = k1 + _W1
            p0 = _M0 * c0.astype(np.uint64)
            p1 = _M1 * c2.astype(np.uint64)
            hi0 = (p0 >> np.uint64(32)).astype(np.uint32)
            lo0 = (p0 & _MASK32).astype(np.uint32)
            hi1 = (p1 >> np.uint64(32)).astype(np.uint32)
            lo1 = (p1 & _MASK32).astype(np.uint32)
            c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return c0, c1, c2, c3


def normal_f32(seed: int, stream: int, idx) -> np.ndarray:
    """Irwin-Hall(12) draw for element indices ``idx`` (uint64 array) of ``stream``.

    Returns float32 values that are exact (integer / 65536)."""
    idx = np.asarray(idx, dtype=np.uint64)
    lo = (idx & _MASK32).astype(np.uint32)
    hi = (idx >> np.uint64(32)).astype(np.uint32)
    k0 = np.uint32(seed & 0xFFFFFFFF)
    k1 = np.uint32((seed >> 32) & 0xFFFFFFFF)
    s = np.uint32(stream & 0xFFFFFFFF)
    a = philox4x32_10(lo, hi, s, np.uint32(0), k0, k1)
    b = philox4x32_10(lo, hi, s, np.uint32(1), k0, k1)
    words = list(a) + list(b)
    total = np.zeros(idx.shape, dtype=np.int64)
    for j in range(12):
        w = words[j // 2].astype(np.int64)
        h = (w & 0xFFFF) if j % 2 == 0 else (w >> 16)
        total += h
    return ((total - 393210).astype(np.float32)) / np.float32(65536.0)


def f32_to_bf16_bits(x) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even) and return the uint16 patterns."""
    b = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (b >> np.uint64(16)) & np.uint64(1)
    r = (b + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return (r & np.uint64(0xFFFF)).astype(np.uint16)


def bf16_bits_to_f32(bits) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def scaled_bf16_bits(seed: int, stream: int, idx, factor) -> np.ndarray:
    """bf16(z * factor) with one float32 multiply; ``factor`` broadcasts against ``idx``."""
    z = normal_f32(seed, stream, idx)
    with np.errstate(over="ignore"):
        prod = z * np.asarray(factor, dtype=np.float32)
    return f32_to_bf16_bits(prod)
