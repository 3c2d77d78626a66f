// Group quantizer and record packer of the KV cache, shared by the append kernels and the
// decode's in-launch append (serving steps).
//
// Source: "LoopKV: Loop-Aware KV Cache Compression for Serving Looped Transformers"
// (arXiv:2611.04137), Abstract: a cell is stored as 4-bit (KIVI-4 style) or 2-bit, and a
// decoding loop reads the high 2 bits of a 4-bit value apart from its low bits, so 4-bit codes
// are split into a high and a low 2-bit plane.
//
// Quantizer (KIVI-style asymmetric groups of GS = 32, or 64): K per channel over GS consecutive
// tokens, V per token over GS consecutive channels; zero = f16(min), scale = f16((max - min) /
// (2^b - 1)), code = clamp(rint((x - zero) / scale), 0, 2^b - 1), scale 0 -> code 0. All of it in
// float64 with one round-to-nearest-even to f16, each operation rounded on its own (no
// contraction), so codes and meta are the same bits wherever this header is compiled.
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>
#include "layout.h"

namespace lkv {

// float64 -> float16 bits, round to nearest even, one rounding.
__device__ inline uint32_t f64_to_f16_bits(double x) {
  uint64_t b = (uint64_t)__double_as_longlong(x);
  uint32_t sign = (uint32_t)(b >> 48) & 0x8000u;
  int ex = (int)((b >> 52) & 0x7ff);
  uint64_t man = b & 0xFFFFFFFFFFFFFull;
  if (ex == 0x7ff) return sign | 0x7c00u | (man ? 0x200u : 0u);
  if (ex == 0) return sign;                       // below 2^-1022: rounds to zero
  int e = ex - 1023;
  if (e > 15) return sign | 0x7c00u;
  uint64_t m = man | (1ull << 52);
  int s = (e >= -14) ? 42 : (28 - e);             // bits dropped to reach the f16 ulp
  if (s > 60) return sign;
  uint64_t q = m >> s;
  uint64_t rem = m & ((1ull << s) - 1);
  uint64_t half = 1ull << (s - 1);
  if (rem > half || (rem == half && (q & 1))) q++;
  uint32_t bits = (e >= -14) ? (uint32_t)(((e + 15) << 10) + (int)q - 1024) : (uint32_t)q;
  if (bits >= 0x7c00u) bits = 0x7c00u;
  return sign | bits;
}

__device__ inline double f16_bits_to_f64(uint32_t h) {
  return (double)__half2float(__ushort_as_half((unsigned short)h));
}

__device__ inline float bf16_bits_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);   // NaN stays NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Quantize n values (n a power of two) read through get(i) with M = 2^bits - 1 levels. Step k
// takes element (k + rot) mod n: the minimum, the maximum and each element's code do not depend
// on the order, and callers whose lanes read elements at a stride that maps them to the same
// LDS bank give each lane its own rotation. U elements are taken per loop step (U divides n),
// their loads and divisions independent of each other; U = 1 keeps the loops rolled for a
// caller inside the decode kernel, which has few registers to spare.
template <int U = 1, typename Get>
__device__ inline void quantize_group(Get get, int n, int M, uint8_t* codes, int stride, uint32_t* meta, int rot = 0) {
#pragma clang fp contract(off)
  static_assert(U == 1 || U == 2 || U == 4 || U == 8, "elements per step");
  const int mask = n - 1;
  double mn = get(rot & mask), mx = mn;
  if constexpr (U == 1) {
#pragma unroll 1
    for (int k = 1; k < n; ++k) {
      double x = get((k + rot) & mask);
      mn = fmin(mn, x);
      mx = fmax(mx, x);
    }
  } else {
#pragma unroll 1
    for (int k0 = 0; k0 < n; k0 += U) {
      double x[U];
#pragma unroll
      for (int u = 0; u < U; ++u) x[u] = get((k0 + u + rot) & mask);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        mn = fmin(mn, x[u]);
        mx = fmax(mx, x[u]);
      }
    }
  }
  uint32_t zb = f64_to_f16_bits(mn);
  uint32_t sb = f64_to_f16_bits((mx - mn) / (double)M);
  double z = f16_bits_to_f64(zb);
  double s = f16_bits_to_f64(sb);
  // The code is rint of the correctly rounded quotient q = (x - z) / s. The product y = (x - z) *
  // fl(1 / s) is within |q| 2^-51 of q, below 2^-46 for the quotients that matter here (|q| <= 16;
  // larger ones clamp to M either way), so rint(y) = rint(q) unless a rounding tie k + 1/2 lies
  // within 2^-46 of y: there (|y - floor(y) - 1/2| <= 2^-40) the division itself decides.
  // Infinities and NaNs reach the same codes on both routes.
  // The division runs behind a wave-uniform test, only in waves where some lane needs it.
  const double rs = 1.0 / s;
#pragma unroll 1
  for (int k0 = 0; k0 < n; k0 += U) {
    double d[U], y[U];
    bool tie[U];
    bool any_tie = false;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      d[u] = get((k0 + u + rot) & mask) - z;
      y[u] = d[u] * rs;
      tie[u] = fabs(y[u] - floor(y[u]) - 0.5) <= 0x1p-40;
      any_tie |= tie[u];
    }
    if (__any(any_tie)) {
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (tie[u]) y[u] = d[u] / s;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = (k0 + u + rot) & mask;
      int c = 0;
      if (s != 0.0) {   // s = 0: every code is 0 (y is not used)
        double r = rint(y[u]);
        r = fmin(fmax(r, 0.0), (double)M);
        c = (int)r;
      }
      codes[i * stride] = (uint8_t)c;
    }
  }
  *meta = sb | (zb << 16);
}

// Rotation of V group `task` (token task / (D / GS), channels GS (task mod (D / GS)) + ...): the
// groups of consecutive tasks sit GS * 2 bytes apart in the bf16 staging rows and GS bytes apart
// in the code rows, so without it the lanes of a wave hit a few LDS banks at every step; task
// times GS / 32 spreads them over all banks.
template <int GS>
__device__ inline int vgroup_rot(int task) { return task * (GS / 32); }

// Channel stored at K-meta position i: the words of a K column follow the column's
// bit layout (2-bit: byte k, bit pair p; 4-bit: byte k, nibble n).
__device__ inline int kmeta_channel2(int i) { return (i & ~15) + 4 * (i & 3) + ((i >> 2) & 3); }
__device__ inline int kmeta_channel4(int i) { return (i & ~7) + 2 * (i & 3) + ((i >> 2) & 1); }

// Codes and meta of one complete group of GS tokens (values through getk(i, d) / getv(i, d),
// float64): K per channel over the tokens, V per token over each run of GS channels. Work is
// spread over the nthr threads of the calling workgroup (thread tid); the caller synchronizes
// the workgroup after the call.
template <int D, int GS, typename GetK, typename GetV>
__device__ inline void quantize_group_codes(GetK getk, GetV getv, int M, uint8_t (*kc)[D], uint8_t (*vc)[D],
                                            uint32_t* kmeta, uint32_t (*vmeta)[D / GS], int tid, int nthr) {
  for (int d = tid; d < D; d += nthr) quantize_group([&](int i) { return getk(i, d); }, GS, M, &kc[0][d], D, &kmeta[d]);
  for (int task = tid; task < GS * (D / GS); task += nthr) {
    const int i = task / (D / GS), e = task % (D / GS);
    quantize_group([&](int j) { return getv(i, e * GS + j); }, GS, M, &vc[i][e * GS], 1, &vmeta[i][e],
                   vgroup_rot<GS>(task));
  }
}

// Write record `part` (tokens 16 part .. 16 part + 15 and K-meta positions part D / P ..
// (part + 1) D / P - 1, P = GS / 16) of a quantized group to r (one KV head's record).
template <int D, int GS>
__device__ inline void pack_record(uint32_t* r, int kind, int part, const uint8_t (*kc)[D], const uint8_t (*vc)[D],
                                   const uint32_t* kmeta, const uint32_t (*vmeta)[D / GS], int tid, int nthr) {
  constexpr int P = GS / kBlock;
  const int t0 = part * kBlock;
  if (kind == KIND_KIVI4) {
    // K4: D/8 columns x 16 tokens; V4: D channels x 2 words (quads stored transposed).
    for (int idx = tid; idx < (D / 8) * kBlock; idx += nthr) {
      const int w = idx / kBlock, t = idx % kBlock;
      uint32_t word = 0;
      for (int c = 0; c < 8; ++c) word |= (uint32_t)kc[t0 + t][8 * w + c] << (4 * c);
      r[idx] = word;
    }
    for (int idx = tid; idx < D * 2; idx += nthr) {
      const int d = idx / 2, jj = idx % 2;
      uint32_t word = 0;
      for (int tp = 0; tp < 8; ++tp) word |= (uint32_t)vc[t0 + 8 * jj + tp][d] << (8 * (tp % 4) + 4 * (tp / 4));
      r[off_v_kivi(D, GS) / 4 + vword_pos(idx, true, D)] = word;
    }
    for (int c = tid; c < D / P; c += nthr) r[off_kmeta_kivi(D) / 4 + c] = kmeta[kmeta_channel4(part * (D / P) + c)];
    for (int idx = tid; idx < kBlock * (D / GS); idx += nthr)
      r[off_vmeta_kivi(D, GS) / 4 + idx] = vmeta[t0 + idx % kBlock][idx / kBlock];
  } else {
    const bool q4 = kind == KIND_Q4;
    // K planes: D/16 columns x 16 tokens. The lanes of a column read code rows D bytes apart,
    // so each takes its row's four code words in its own rotated order (fewer lanes on one LDS
    // bank at a time) and puts them back in order with selects; kc rows are 16-byte aligned.
    for (int idx = tid; idx < (D / 16) * kBlock; idx += nthr) {
      const int w = idx / kBlock, t = idx % kBlock;
      const uint32_t* row = reinterpret_cast<const uint32_t*>(&kc[t0 + t][16 * w]);
      const int rr = t & 3;
      const uint32_t a0 = row[rr], a1 = row[(rr + 1) & 3], a2 = row[(rr + 2) & 3], a3 = row[(rr + 3) & 3];
      // code word k = a[(k - rr) mod 4]
      const uint32_t cw[4] = {rr == 0 ? a0 : rr == 1 ? a3 : rr == 2 ? a2 : a1,
                              rr == 0 ? a1 : rr == 1 ? a0 : rr == 2 ? a3 : a2,
                              rr == 0 ? a2 : rr == 1 ? a1 : rr == 2 ? a0 : a3,
                              rr == 0 ? a3 : rr == 1 ? a2 : rr == 2 ? a1 : a0};
      uint32_t hi = 0, lo = 0;
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        const uint32_t code = (cw[c >> 2] >> (8 * (c & 3))) & 0xffu;
        if (q4) {
          hi |= (code >> 2) << (2 * c);
          lo |= (code & 3u) << (2 * c);
        } else {
          hi |= code << (2 * c);
        }
      }
      r[idx] = hi;
      if (q4) r[off_klo(D, GS) / 4 + idx] = lo;
    }
    // V planes: one word per channel, token t at bit 8*(t%4) + 2*(t/4).
    for (int d = tid; d < D; d += nthr) {
      uint32_t hi = 0, lo = 0;
      for (int t = 0; t < kBlock; ++t) {
        const uint32_t code = vc[t0 + t][d];
        const int sh = 8 * (t % 4) + 2 * (t / 4);
        if (q4) {
          hi |= (code >> 2) << sh;
          lo |= (code & 3u) << sh;
        } else {
          hi |= code << sh;
        }
      }
      const int wp = vword_pos(d, false, D);   // the planes' quads are stored transposed
      r[off_v_planes(D, GS) / 4 + wp] = hi;
      if (q4) r[off_vlo(D, GS) / 4 + wp] = lo;
    }
    for (int c = tid; c < D / P; c += nthr) r[off_kmeta_planes(D) / 4 + c] = kmeta[kmeta_channel2(part * (D / P) + c)];
    for (int idx = tid; idx < kBlock * (D / GS); idx += nthr)
      r[off_vmeta_planes(D, GS) / 4 + idx] = vmeta[t0 + idx % kBlock][idx / kBlock];
  }
}

}  // namespace lkv
