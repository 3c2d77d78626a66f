// Loop-aware decode attention over the per-(loop, layer) mixed-precision KV cache (gfx950).
//
// Source: "LoopKV: Loop-Aware KV Cache Compression for Serving Looped
// Transformers" (arXiv:2611.04137), Abstract: during decoding each loop reads
// the high 2 bits of every 4-bit value and fetches the low bits only where its
// own attention weights require 4-bit precision; low-attention values are read
// at low precision rather than skipped; a reuse cell reads the final loop's KV;
// KIVI-4 (uniform 4-bit) runs on the same kernel as the baseline.
//
// One workgroup (8 wave64s) owns one row (cell, sequence, head); a whole plan is
// one launch of cells x sequences x heads workgroups. The path is HBM-bound with
// a VALU co-limit, so no MFMA: 2-bit codes are widened with in-place byte masks
// and v_cvt_f32_ubyteN, every per-group / per-token scale is folded into the
// coefficient that multiplies the code, and every wave keeps the loads of its
// next step in flight while it computes the current one.
//
//   K pass   coarse scores s_t = sigma q . (z + s (4 hi + 3/2)) from the high plane
//            (4-bit target); full scores for tau = 0 and KIVI-4; 2-bit scores for a
//            2-bit target; the tail (last len mod 32 tokens) is exact bf16. Scores
//            stay in LDS (4 bytes per token).
//   stats    m = max s, l = sum exp(s - m) over the whole row.
//   select   token t of the quantized prefix is selected when exp(s_t - m)/l >= tau;
//            a ballot per 64 tokens gives one 32-bit mask per 32-token group.
//   refine   only groups with a selected token: read their low K plane and add
//            sigma q . s (lo - 3/2) to the selected scores.
//   V pass   weights w_t = exp(s_t - m') with the final max m'; values
//            z + s (4 hi + lo) for selected tokens (low V plane read only for blocks
//            holding one), z + s (4 hi + 3/2) otherwise, exact on the tail.
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>
#include <math.h>
#include "layout.h"

namespace lkv {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kWaveScratch = 256;   // floats of per-wave LDS scratch

enum : int { MODE_COARSE = 0, MODE_DENSE = 1, MODE_Q2 = 2, MODE_KIVI = 3 };

__device__ inline void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int CTRL>
__device__ inline float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
// Sum over aligned groups of N lanes: quad swaps, then half-row and row mirrors, then shuffles.
template <int N>
__device__ inline float group_sum(float v) {
  if (N >= 2) v += dpp<0xB1>(v);    // quad_perm [1,0,3,2]
  if (N >= 4) v += dpp<0x4E>(v);    // quad_perm [2,3,0,1]
  if (N >= 8) v += dpp<0x141>(v);   // row_half_mirror
  if (N >= 16) v += dpp<0x140>(v);  // row_mirror
  if (N >= 32) v += __shfl_xor(v, 16);
  if (N >= 64) v += __shfl_xor(v, 32);
  return v;
}
__device__ inline float wave_sum(float v) { return group_sum<64>(v); }
__device__ inline float wave_max(float v) {
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

__device__ inline float f16lo(uint32_t w) { return __half2float(__ushort_as_half((unsigned short)(w & 0xffffu))); }
__device__ inline float f16hi(uint32_t w) { return __half2float(__ushort_as_half((unsigned short)(w >> 16))); }
__device__ inline float bf16f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ inline float ubyte(uint32_t x, int k) { return (float)((x >> (8 * k)) & 0xffu); }
// Byte masks the optimizer cannot see through (a scalar move it may hoist and reuse):
// with a visible constant it merges the mask with the byte extraction into 2-bit
// field extracts and loses v_cvt_f32_ubyte1..3 (one extra VALU op per code).
template <uint32_t C>
__device__ inline uint32_t smask() {
  uint32_t m;
  asm("s_mov_b32 %0, %1" : "=s"(m) : "i"(C));
  return m;
}
template <int P>
__device__ inline uint32_t mask2() { return smask<(0x03030303u << (2 * P))>(); }
template <int N>
__device__ inline uint32_t mask4() { return smask<(0x0F0F0F0Fu << (4 * N))>(); }

// Sixteen 2-bit codes of one word. K order: cf[4k + p] for the code at byte k, bits 2p.
template <int P>
__device__ inline float dot4_k(uint32_t x, const float* cf, float acc) {
  const uint32_t m = x & mask2<P>();
#pragma unroll
  for (int k = 0; k < 4; ++k) acc = fmaf(cf[4 * k + P], ubyte(m, k), acc);
  return acc;
}
__device__ inline float dot16_k(uint32_t x, const float* cf, float acc) {
  acc = dot4_k<0>(x, cf, acc);
  acc = dot4_k<1>(x, cf, acc);
  acc = dot4_k<2>(x, cf, acc);
  return dot4_k<3>(x, cf, acc);
}
// V order: cf[4p + k] (token 4p + k of the block).
template <int P>
__device__ inline float dot4_v(uint32_t x, const float* cf, float acc) {
  const uint32_t m = x & mask2<P>();
#pragma unroll
  for (int k = 0; k < 4; ++k) acc = fmaf(cf[4 * P + k], ubyte(m, k), acc);
  return acc;
}
__device__ inline float dot16_v(uint32_t x, const float* cf, float acc) {
  acc = dot4_v<0>(x, cf, acc);
  acc = dot4_v<1>(x, cf, acc);
  acc = dot4_v<2>(x, cf, acc);
  return dot4_v<3>(x, cf, acc);
}
// Eight 4-bit codes of one word. K order (the K-meta position order): cf[4n + k] for
// nibble n of byte k.
template <int N>
__device__ inline float dot4_k4(uint32_t x, const float* cf, float acc) {
  const uint32_t m = x & mask4<N>();
#pragma unroll
  for (int k = 0; k < 4; ++k) acc = fmaf(cf[4 * N + k], ubyte(m, k), acc);
  return acc;
}
__device__ inline float dot8_k4(uint32_t x, const float* cf, float acc) {
  return dot4_k4<1>(x, cf, dot4_k4<0>(x, cf, acc));
}
// V order: cf[4n + k] (token 4n + k of the word's 8 tokens).
template <int N>
__device__ inline float dot4_v4(uint32_t x, const float* cf, float acc) {
  const uint32_t m = x & mask4<N>();
#pragma unroll
  for (int k = 0; k < 4; ++k) acc = fmaf(cf[4 * N + k], ubyte(m, k), acc);
  return acc;
}
__device__ inline float dot8_v4(uint32_t x, const float* cf, float acc) {
  return dot4_v4<1>(x, cf, dot4_v4<0>(x, cf, acc));
}

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
// Streaming loads (the cache bytes are read once per decode).
__device__ inline uint4 ld_stream4(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ inline uint4 ld_stream2(const void* p) {
  const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
  return make_uint4(v.x, v.y, 0u, 0u);
}

__device__ inline int sdot4(uint32_t a, uint32_t b, int c) { return __builtin_amdgcn_sdot4((int)a, (int)b, c, false); }
__device__ inline uint32_t udot4(uint32_t a, uint32_t b, uint32_t c) { return __builtin_amdgcn_udot4(a, b, c, false); }
// Bytes 0..2 of four words, transposed: limb j holds byte j of word k in its byte k.
__device__ inline void transpose3(const uint32_t* u, uint32_t* limb) {
  const uint32_t a = __builtin_amdgcn_perm(u[1], u[0], 0x05010400u);   // u0.b0 u1.b0 u0.b1 u1.b1
  const uint32_t b = __builtin_amdgcn_perm(u[3], u[2], 0x05010400u);   // u2.b0 u3.b0 u2.b1 u3.b1
  const uint32_t c = __builtin_amdgcn_perm(u[1], u[0], 0x07030602u);   // u0.b2 u1.b2 u0.b3 u1.b3
  const uint32_t d = __builtin_amdgcn_perm(u[3], u[2], 0x07030602u);
  limb[0] = __builtin_amdgcn_perm(b, a, 0x05040100u);
  limb[1] = __builtin_amdgcn_perm(b, a, 0x07060302u);
  limb[2] = __builtin_amdgcn_perm(d, c, 0x05040100u);
}
// Bytes 0..1 of four words, transposed.
__device__ inline void transpose2(const uint32_t* u, uint32_t* limb) {
  const uint32_t a = __builtin_amdgcn_perm(u[1], u[0], 0x05010400u);
  const uint32_t b = __builtin_amdgcn_perm(u[3], u[2], 0x05010400u);
  limb[0] = __builtin_amdgcn_perm(b, a, 0x05040100u);
  limb[1] = __builtin_amdgcn_perm(b, a, 0x07060302u);
}
// Binary exponent e with |v| < 2^e for the largest magnitude v of a set (frexp), kept
// above -100 so that 2^(bits - e) stays finite for tiny or zero sets.
__device__ inline int set_exponent(float vmax) {
  const int e = __builtin_amdgcn_frexp_expf(vmax);
  return e < -100 ? -100 : e;
}
// Signed 22-bit fixed point with byte-limb bias: for |v| < 2^21, returns v + 0x808080
// (three biased bytes). The add of 1.5 * 2^23 rounds v to the nearest integer (ties to
// even) inside the fma and leaves it in the low mantissa bits.
__device__ inline uint32_t biased_fixed22(float c, float scl) {
  return __float_as_uint(fmaf(c, scl, 12582912.0f)) - (0x4B400000u - 0x808080u);
}
// Max over aligned groups of N lanes (same lane pattern as group_sum).
template <int N>
__device__ inline float group_max(float v) {
  if (N >= 2) v = fmaxf(v, dpp<0xB1>(v));
  if (N >= 4) v = fmaxf(v, dpp<0x4E>(v));
  if (N >= 8) v = fmaxf(v, dpp<0x141>(v));
  if (N >= 16) v = fmaxf(v, dpp<0x140>(v));
  if (N >= 32) v = fmaxf(v, __shfl_xor(v, 16));
  if (N >= 64) v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}

// Max over aligned groups of N lanes of non-negative floats, compared as unsigned bit
// patterns (same order for values >= 0; fuses into DPP max instructions).
template <int N>
__device__ inline float group_max_nonneg(float x) {
  uint32_t v = __float_as_uint(x);
  if (N >= 2) v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
  if (N >= 4) v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));
  if (N >= 8) v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));
  if (N >= 16) v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));
  if (N >= 32) v = max(v, (uint32_t)__shfl_xor((int)v, 16));
  if (N >= 64) v = max(v, (uint32_t)__shfl_xor((int)v, 32));
  return __uint_as_float(v);
}

// Codes at bit pair p of every byte of two words, each as four bytes: one 64-bit shift
// serves both words (bits pulled in from the upper word land above bit 25 and are
// masked off).
__device__ inline void bitpairs2(uint32_t x0, uint32_t x1, uint32_t* m0, uint32_t* m1) {
  const uint64_t X = ((uint64_t)x1 << 32) | x0;
  m0[0] = x0 & 0x03030303u;
  m1[0] = x1 & 0x03030303u;
#pragma unroll
  for (int p = 1; p < 4; ++p) {
    const uint64_t Y = X >> (2 * p);
    m0[p] = (uint32_t)Y & 0x03030303u;
    m1[p] = (uint32_t)(Y >> 32) & 0x03030303u;
  }
}

__device__ inline uint32_t w4(const uint4& v, int i) { return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w; }

struct Row {
  const uint8_t* pool;     // pool base of the storage cell
  const uint32_t* boff;    // per logical block: record offset in 256-byte units (in LDS)
  const uint16_t* tail;    // tail of (slot, head): [2][32][D] bf16
  int N, n_q, n_groups;
  __device__ inline const uint8_t* rec_ptr(int j) const { return pool + ((uint64_t)boff[j] << 8); }
};

// ----------------------------------------------------------------------------- K pass
// Lane mapping per wave step: GPS groups, each covered by LPG lanes = 2 blocks x 4
// token quads x CPG column pairs (a column is one 32-bit word of UNIT channels). A
// lane reads 4 consecutive tokens of two adjacent columns (two 16-byte loads) and
// keeps 4 partial scores, summed over the CPG column-pair lanes with quad DPP. The
// coefficients of a group are built by its LPG lanes (CPL consecutive K-meta
// positions each) and passed through LDS.
//
// 2-bit planes use integer dot products: the group's coefficients become 23-bit
// fixed point (scale 2^(22-e) from the group maximum) split into three signed byte
// limbs; v_dot4_i32_i8 multiplies the four codes at one bit pair of a word's bytes by
// four limbs, and the limb sums are recombined exactly in one register
// ((l2 << 8) + l1) << 8 + l0. KIVI-4 words (4-bit codes) stay on the fp32 path.
template <int D, int MODE, bool REFINE>
struct KPass {
  static constexpr bool KIVI = MODE == MODE_KIVI;
  static constexpr bool DENSE = MODE == MODE_DENSE && !REFINE;
  static constexpr int UNIT = KIVI ? 8 : 16;
  static constexpr int COLS = D / UNIT;
  static constexpr int CPG = COLS / 2;
  static constexpr int LPG = 8 * CPG;
  static constexpr int GPS = 64 / LPG;
  static constexpr int CPL = UNIT / 4;
  static constexpr int KMETA = KIVI ? off_kmeta_kivi(D) : off_kmeta_planes(D);
  static constexpr int CODE_OFF = REFINE ? off_klo(D) : 0;

  struct Buf {
    uint4 meta, c0, c1, l0, l1;
    bool vm, vc;
  };

  __device__ static inline void lane_role(int lane, int& blk, int& quad, int& cp) {
    const int rl = lane % LPG;
    blk = rl / (4 * CPG);
    quad = (rl / CPG) % 4;
    cp = rl % CPG;
  }

  __device__ static inline void load(const Row& r, const uint32_t* selm, int s, int lane, int w, Buf& b) {
    const int gbase = (s * kWaves + w) * GPS;
    const int idx = lane * CPL;
    const int gm = gbase + idx / D, pos = idx % D;
    b.vm = gm < r.n_groups && (!REFINE || selm[gm] != 0u);
    if (b.vm) {
      const uint8_t* p = r.rec_ptr(2 * gm + (pos >= D / 2)) + KMETA + 4 * (pos % (D / 2));
      b.meta = CPL == 4 ? ld_stream4(p) : ld_stream2(p);
    }
    int blk, quad, cp;
    lane_role(lane, blk, quad, cp);
    const int gc = gbase + lane / LPG;
    b.vc = gc < r.n_groups && (!REFINE || selm[gc] != 0u);
    if (b.vc) {
      const uint8_t* kp = r.rec_ptr(2 * gc + blk) + CODE_OFF + (2 * cp * kBlock + 4 * quad) * 4;
      b.c0 = ld_stream4(kp);                 // column 2cp, tokens 4quad..4quad+3
      b.c1 = ld_stream4(kp + kBlock * 4);    // column 2cp+1
      if (DENSE) {
        b.l0 = ld_stream4(kp + off_klo(D));
        b.l1 = ld_stream4(kp + off_klo(D) + kBlock * 4);
      }
    }
  }

  // Coefficient of the channel at one K-meta position and its share of the constant term.
  __device__ static inline float coef_of(uint32_t mw, float qv, float pre, float& cst) {
    const float sc = f16lo(mw), z = f16hi(mw);
    const float qsv = qv * sc;
    if (REFINE) {
      cst = fmaf(-1.5f, qsv, cst);           // sigma q . s (lo - 3/2)
      return qsv * pre;
    } else if (MODE == MODE_COARSE) {
      cst += qv * fmaf(1.5f, sc, z);         // sigma q . (z + s (4 hi + 3/2))
      return 4.f * qsv * pre;
    } else {
      cst = fmaf(qv, z, cst);                // sigma q . (z + s c), c 2-bit / 4-bit
      return qsv * pre;
    }
  }

  // One limb's contribution of a word's 16 channels: codes m[p] (four channels at bit pair p)
  // times the limb bytes of those channels, accumulated into a.
  __device__ static inline int word_dot(const uint32_t* L, const uint32_t* m, int limb, int a) {
#pragma unroll
    for (int pp = 0; pp < 4; ++pp) a = sdot4(L[3 * pp + limb], m[pp], a);
    return a;
  }

  __device__ static inline void compute(const Row& r, const float* qs, const float* qreg, float* scores,
                                        const uint32_t* selm, float* scratch, int s, int lane, int w, const Buf& b,
                                        float& mloc) {
    const int gbase = (s * kWaves + w) * GPS;
    const int idx = lane * CPL;
    const int gsm = idx / D, pos0 = idx % D;
    const int gsub = lane / LPG;
    int blk, quad, cp;
    lane_role(lane, blk, quad, cp);
    float part[4] = {0.f, 0.f, 0.f, 0.f};
    float cst = 0.f, inv = 1.f;

    if constexpr (KIVI) {
      // positions 8w + 4n + k hold channel 8w + 2k + n; this lane: n fixed, k and k+1
      float* coef = scratch;   // [GPS][D] in position order
      if (b.vm) {
        const int cw = pos0 / 8, r8 = pos0 % 8, n = r8 / 4, k0 = r8 % 4;
        const float pre = n ? 1.f / 16.f : 1.f;
        const float c0 = coef_of(b.meta.x, qs[8 * cw + 2 * k0 + n], pre, cst);
        const float c1 = coef_of(b.meta.y, qs[8 * cw + 2 * (k0 + 1) + n], pre, cst);
        *reinterpret_cast<float2*>(coef + gsm * D + pos0) = make_float2(c0, c1);
      }
      cst = group_sum<LPG>(cst);
      wave_sync_lds();
      if (b.vc) {
        float cf[2 * UNIT];
        const float4* cq = reinterpret_cast<const float4*>(coef + gsub * D + 2 * cp * UNIT);
#pragma unroll
        for (int u = 0; u < UNIT / 2; ++u) {
          const float4 t = cq[u];
          cf[4 * u] = t.x;
          cf[4 * u + 1] = t.y;
          cf[4 * u + 2] = t.z;
          cf[4 * u + 3] = t.w;
        }
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
          part[tt] = dot8_k4(w4(b.c1, tt), cf + UNIT, dot8_k4(w4(b.c0, tt), cf, 0.f));
      }
    } else {
      // positions 16w + 4p + k hold channel 16w + 4k + p; this lane: column w, bit pair p, k = 0..3
      // (sigma q of those channels arrives hoisted in qreg)
      uint32_t* qlimb = reinterpret_cast<uint32_t*>(scratch);   // [GPS][COLS][4 p][3 limbs]
      const int cw = pos0 / 16, p = (pos0 >> 2) & 3;
      float f[4] = {0.f, 0.f, 0.f, 0.f};
      if (b.vm) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t mw = w4(b.meta, k);
          f[k] = qreg[k] * f16lo(mw);                         // sigma q s
          if (REFINE) {
            cst = fmaf(-1.5f, f[k], cst);                     // sigma q s (lo - 3/2)
          } else if (MODE == MODE_COARSE) {
            cst = fmaf(qreg[k], f16hi(mw), cst);              // sigma q (z + s (4 hi + 3/2))
            cst = fmaf(1.5f, f[k], cst);
          } else {
            cst = fmaf(qreg[k], f16hi(mw), cst);              // sigma q (z + s c)
          }
        }
      }
      float fm = fmaxf(fmaxf(fabsf(f[0]), fabsf(f[1])), fmaxf(fabsf(f[2]), fabsf(f[3])));
      fm = group_max_nonneg<LPG>(fm);
      const int ex = set_exponent(fm);
      const float scl = __builtin_amdgcn_ldexpf(1.f, 21 - ex);
      // high-plane-only codes carry weight 4 (code 4 hi): folded into the inverse scale
      inv = __builtin_amdgcn_ldexpf(MODE == MODE_COARSE && !REFINE ? 4.f : 1.f, ex - 21);
      if (b.vm) {
        uint32_t u[4], limb[3];
#pragma unroll
        for (int k = 0; k < 4; ++k) u[k] = biased_fixed22(f[k], scl);
        transpose3(u, limb);
        uint32_t* dst = qlimb + ((gsm * COLS + cw) * 4 + p) * 3;
#pragma unroll
        for (int j = 0; j < 3; ++j) dst[j] = limb[j] ^ 0x80808080u;   // biased byte -> signed digit
      }
      cst = group_sum<LPG>(cst);
      wave_sync_lds();
      if (b.vc) {
        uint32_t L[24];   // limbs of columns 2cp and 2cp+1: [col][p][limb]
        const uint4* lq = reinterpret_cast<const uint4*>(qlimb + (gsub * COLS + 2 * cp) * 12);
#pragma unroll
        for (int u = 0; u < 6; ++u) {
          const uint4 t = lq[u];
          L[4 * u] = t.x;
          L[4 * u + 1] = t.y;
          L[4 * u + 2] = t.z;
          L[4 * u + 3] = t.w;
        }
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          uint32_t m0[4], m1[4];
          bitpairs2(w4(b.c0, tt), w4(b.c1, tt), m0, m1);
          if (DENSE) {   // 4-bit codes 4 hi + lo
            uint32_t n0[4], n1[4];
            bitpairs2(w4(b.l0, tt), w4(b.l1, tt), n0, n1);
#pragma unroll
            for (int pp = 0; pp < 4; ++pp) {
              m0[pp] = (m0[pp] << 2) | n0[pp];
              m1[pp] = (m1[pp] << 2) | n1[pp];
            }
          }
          int a = word_dot(L, m0, 2, 0);
          a = word_dot(L + 12, m1, 2, a);
          a = word_dot(L, m0, 1, a << 8);
          a = word_dot(L + 12, m1, 1, a);
          a = word_dot(L, m0, 0, a << 8);
          a = word_dot(L + 12, m1, 0, a);
          part[tt] = (float)a;
        }
      }
    }
    if constexpr (KIVI) {
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) part[tt] = group_sum<CPG>(part[tt]);
      if (b.vc) {
        const int g = gbase + gsub;
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          if ((tt % CPG) == cp) {
            const int t = g * kGroup + blk * kBlock + quad * 4 + tt;
            const float sc = cst + part[tt];
            scores[t] = sc;
            mloc = fmaxf(mloc, sc);
          }
        }
      }
    } else {
      // The CPG column-pair lanes of a token quad are consecutive: reduce-scatter their
      // four partial scores so that lane cp ends with token cp (CPG = 4) or tokens cp and
      // cp + 2 (CPG = 2).
      const bool odd = cp & 1;
      float k0 = odd ? part[1] : part[0], k1 = odd ? part[3] : part[2];
      const float s0 = odd ? part[0] : part[1], s1 = odd ? part[2] : part[3];
      k0 += dpp<0xB1>(s0);   // quad_perm [1,0,3,2]
      k1 += dpp<0xB1>(s1);
      float mine[2];
      int nmine;
      if (CPG == 4) {
        const bool hi = cp & 2;
        const float keep = hi ? k1 : k0, send = hi ? k0 : k1;
        mine[0] = keep + dpp<0x4E>(send);   // quad_perm [2,3,0,1]
        mine[1] = 0.f;
        nmine = 1;
      } else {
        mine[0] = k0;
        mine[1] = k1;
        nmine = 2;
      }
      if (b.vc) {
        const int g = gbase + gsub;
        const uint32_t gm = REFINE ? selm[g] : 0u;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          if (i < nmine) {
            const int ti = blk * kBlock + quad * 4 + (CPG == 4 ? cp : cp + 2 * i);
            const int t = g * kGroup + ti;
            if (REFINE) {
              if ((gm >> ti) & 1u) {
                const float sc = scores[t] + fmaf(inv, mine[i], cst);
                scores[t] = sc;
                mloc = fmaxf(mloc, sc);
              }
            } else {
              const float sc = fmaf(inv, mine[i], cst);
              scores[t] = sc;
              mloc = fmaxf(mloc, sc);
            }
          }
        }
      }
    }
    wave_sync_lds();
  }

  __device__ static void run(const Row& r, const float* qs, float* scores, const uint32_t* selm, float* scratch,
                             int lane, int w, float& mloc) {
    const int steps = (r.n_groups + kWaves * GPS - 1) / (kWaves * GPS);
    // sigma q of the four channels whose coefficients this lane builds (fixed for the row)
    float qreg[4];
    {
      const int pos0 = (lane * CPL) % D, cw = pos0 / 16, p = (pos0 >> 2) & 3;
#pragma unroll
      for (int k = 0; k < 4; ++k) qreg[k] = KIVI ? 0.f : qs[16 * cw + 4 * k + p];
    }
    // three buffers in rotation: the loads of steps s+1 and s+2 are in flight while step s computes
    Buf b0, b1, b2;
    load(r, selm, 0, lane, w, b0);
    if (1 < steps) load(r, selm, 1, lane, w, b1);
    for (int s = 0; s < steps; s += 3) {
      if (s + 2 < steps) load(r, selm, s + 2, lane, w, b2);
      if (!REFINE || __any(b0.vm)) compute(r, qs, qreg, scores, selm, scratch, s, lane, w, b0, mloc);
      if (s + 1 >= steps) break;
      if (s + 3 < steps) load(r, selm, s + 3, lane, w, b0);
      if (!REFINE || __any(b1.vm)) compute(r, qs, qreg, scores, selm, scratch, s + 1, lane, w, b1, mloc);
      if (s + 2 >= steps) break;
      if (s + 4 < steps) load(r, selm, s + 4, lane, w, b1);
      if (!REFINE || __any(b2.vm)) compute(r, qs, qreg, scores, selm, scratch, s + 2, lane, w, b2, mloc);
    }
  }
};

// ----------------------------------------------------------------------------- V pass
// Lane mapping per wave step: 4 blocks (64 tokens).
//   weights: lane (block jb, bit pair p, channel group e) folds weight, scale and
//            bucket offset of the four tokens 4p..4p+3 of its block and group;
//   values:  lane (block, chunk) reads the V words of D/16 channels (16 tokens per
//            word) and accumulates.
// 2-bit planes use integer dot products: the weights w_t * s_t of a (block, group)
// become 23-bit fixed point split into three unsigned byte limbs, v_dot4_u32_u8
// multiplies them with four tokens' codes of a channel, and each block's exact
// integer sum is scaled back into the fp32 accumulator. A 4-bit target uses the code
// 4*hi + lo, with lo = 0 for tokens whose low bits were not fetched (their bucket
// midpoint sits in the per-token constant term). KIVI-4 stays on the fp32 path.
template <int D, int MODE, bool SPARSE>
struct VPass {
  static constexpr bool KIVI = MODE == MODE_KIVI;
  static constexpr bool DENSE = MODE == MODE_DENSE;
  static constexpr int VCH = D / 16;                // channels per lane
  static constexpr int NE = D / kGroup;             // channel groups
  static constexpr int WPL = KIVI ? 2 * VCH : VCH;  // V words per lane
  static constexpr int NV4 = WPL / 4;               // uint4 loads per lane
  static constexpr int VOFF = KIVI ? off_v_kivi(D) : off_v_planes(D);
  static constexpr int VMETA = KIVI ? off_vmeta_kivi(D) : off_vmeta_planes(D);
  static constexpr int COOP = 16 * NE;              // lanes with a weights role

  struct Buf {
    uint4 meta;
    uint4 c[NV4];
    uint4 l[DENSE ? NV4 : 1];
    bool v, vm;
  };

  __device__ static inline void load(const Row& r, int s, int lane, int w, Buf& b) {
    const int nb = r.n_q / kBlock;
    const int base = (s * kWaves + w) * 4;
    const int jm = base + lane / (4 * NE), p = (lane / NE) % 4, e = lane % NE;
    b.vm = lane < COOP && jm < nb;
    if (b.vm) b.meta = ld_stream4(r.rec_ptr(jm) + VMETA + 4 * (e * kBlock + 4 * p));
    const int j = base + lane / 16;
    b.v = j < nb;
    if (!b.v) return;
    const uint8_t* rb = r.rec_ptr(j);
    const int chunk = lane % 16;
    const uint8_t* vp = rb + VOFF + chunk * WPL * 4;
#pragma unroll
    for (int i = 0; i < NV4; ++i) b.c[i] = ld_stream4(vp + 16 * i);
    if (DENSE) {
      const uint8_t* lp = rb + off_vlo(D) + chunk * WPL * 4;
#pragma unroll
      for (int i = 0; i < NV4; ++i) b.l[i] = ld_stream4(lp + 16 * i);
    }
  }

  __device__ static inline void compute(const Row& r, const float* weights, const uint32_t* selm, float* scratch,
                                        int s, int lane, int w, const Buf& b, float* acc, float& accz) {
    const int base = (s * kWaves + w) * 4;
    const int jbm = lane / (4 * NE), p = (lane / NE) % 4, e = lane % NE;
    float a[4] = {0.f, 0.f, 0.f, 0.f};
    if (b.vm) {
      const int t0 = (base + jbm) * kBlock + 4 * p;
      const float4 w4v = *reinterpret_cast<const float4*>(weights + t0);
      const float wv[4] = {w4v.x, w4v.y, w4v.z, w4v.w};
      uint32_t sel = DENSE ? 0xFu : 0u;
      if (SPARSE) sel = (selm[t0 >> 5] >> (t0 & 31)) & 0xFu;
      // KIVI-4 tokens 4p..4p+3 sit in nibble p % 2 of their word: fold 16^-n here
      const float pre = KIVI && (p & 1) ? (1.f / 16.f) : 1.f;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t mw = w4(b.meta, k);
        const float sc = f16lo(mw), z = f16hi(mw);
        a[k] = wv[k] * sc * pre;
        const bool mid = (MODE == MODE_COARSE) && !((sel >> k) & 1u);
        accz = fmaf(wv[k], mid ? fmaf(1.5f, sc, z) : z, accz);
      }
    }
    const int chunk = lane % 16, jb = lane / 16;
    const int e_lane = (chunk * VCH) / kGroup;
    const int j = base + jb;
    if constexpr (KIVI) {
      float* coefv = scratch;   // [4][NE][16]
      if (b.vm) *reinterpret_cast<float4*>(coefv + (jbm * NE + e) * 16 + 4 * p) = make_float4(a[0], a[1], a[2], a[3]);
      wave_sync_lds();
      if (b.v) {
        float cf[16];
        const float4* cp = reinterpret_cast<const float4*>(coefv + (jb * NE + e_lane) * 16);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float4 tq = cp[u];
          cf[4 * u] = tq.x;
          cf[4 * u + 1] = tq.y;
          cf[4 * u + 2] = tq.z;
          cf[4 * u + 3] = tq.w;
        }
#pragma unroll
        for (int c = 0; c < VCH; ++c) {
#pragma unroll
          for (int jj = 0; jj < 2; ++jj)
            acc[c] = dot8_v4(w4(b.c[(2 * c + jj) / 4], (2 * c + jj) % 4), cf + 8 * jj, acc[c]);
        }
      }
    } else {
      uint32_t* vlimb = reinterpret_cast<uint32_t*>(scratch);   // [4][NE][4 p][2]
      float* vinv = scratch + 4 * NE * 8;                       // [4][NE]
      float am = fmaxf(fmaxf(a[0], a[1]), fmaxf(a[2], a[3]));
      // max over the 4 bit-pair lanes of (block, group): lanes e + NE*p inside a 16-lane row
      // (non-negative: compared as unsigned bit patterns)
      {
        uint32_t v = __float_as_uint(am);
        if (NE == 4) {
          v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xF, 0xF, false));   // row_ror:4
          v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xF, 0xF, false));   // row_ror:8
        } else {
          v = max(v, (uint32_t)__shfl_xor((int)v, NE));
          v = max(v, (uint32_t)__shfl_xor((int)v, 2 * NE));
        }
        am = __uint_as_float(v);
      }
      // unsigned 16-bit fixed point (weights are >= 0), rounded to nearest inside the fma
      // with 2^23 added; the scale 2^(16-e) (1 - 2^-17) keeps the rounded value <= 65535
      const int ex = set_exponent(am);
      const float scl = __builtin_amdgcn_ldexpf(1.f - 0x1p-17f, 16 - ex);
      if (b.vm) {
        uint32_t qb[4], limb[2];
#pragma unroll
        for (int k = 0; k < 4; ++k) qb[k] = __float_as_uint(fmaf(a[k], scl, 8388608.0f)) - 0x4B000000u;
        transpose2(qb, limb);
        uint32_t* dst = vlimb + ((jbm * NE + e) * 4 + p) * 2;
        dst[0] = limb[0];
        dst[1] = limb[1];
        if (p == 0) vinv[jbm * NE + e] = __builtin_amdgcn_ldexpf(1.f + 0x1p-17f, ex - 16);   // 1 / scl
      }
      wave_sync_lds();
      if (b.v) {
        uint32_t L[8];
        const uint4* lp = reinterpret_cast<const uint4*>(vlimb + (jb * NE + e_lane) * 8);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const uint4 t = lp[u];
          L[4 * u] = t.x;
          L[4 * u + 1] = t.y;
          L[4 * u + 2] = t.z;
          L[4 * u + 3] = t.w;
        }
        float binv = vinv[jb * NE + e_lane];
        const float hscale = 4.f * binv;   // high bits only: code 4 hi
        bool need_lo = DENSE;
        uint32_t m32 = 0xffffffffu;
        uint4 lw[NV4];
        if (SPARSE) {
          const uint32_t bm = (selm[j >> 1] >> (16 * (j & 1))) & 0xffffu;
          need_lo = bm != 0u;
          if (need_lo) {
            m32 = 0;
#pragma unroll
            for (int tt = 0; tt < 16; ++tt)
              if ((bm >> tt) & 1u) m32 |= 3u << (8 * (tt & 3) + 2 * (tt >> 2));
            const uint8_t* lq = r.rec_ptr(j) + off_vlo(D) + chunk * VCH * 4;
#pragma unroll
            for (int i = 0; i < NV4; ++i) lw[i] = *reinterpret_cast<const uint4*>(lq + 16 * i);
          }
        }
        if (DENSE) {
#pragma unroll
          for (int i = 0; i < NV4; ++i) lw[i] = b.l[i];
        }
        const bool lo_path = (DENSE || SPARSE) && MODE != MODE_Q2 && need_lo;
        const float cscale = lo_path || MODE == MODE_Q2 ? binv : hscale;
#pragma unroll
        for (int c = 0; c < VCH; c += 2) {
          uint32_t mc[2][4];
          bitpairs2(w4(b.c[c / 4], c % 4), w4(b.c[c / 4], c % 4 + 1), mc[0], mc[1]);
          if (lo_path) {   // 4-bit code 4 hi + lo, lo only for fetched tokens
            uint32_t nc[2][4];
            bitpairs2(w4(lw[c / 4], c % 4) & m32, w4(lw[c / 4], c % 4 + 1) & m32, nc[0], nc[1]);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
              for (int pp = 0; pp < 4; ++pp) mc[i][pp] = (mc[i][pp] << 2) | nc[i][pp];
          }
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            uint32_t a = 0;
#pragma unroll
            for (int pp = 0; pp < 4; ++pp) a = udot4(L[2 * pp + 1], mc[i][pp], a);
            a <<= 8;
#pragma unroll
            for (int pp = 0; pp < 4; ++pp) a = udot4(L[2 * pp], mc[i][pp], a);
            acc[c + i] = fmaf(cscale, (float)a, acc[c + i]);
          }
        }
      }
    }
    wave_sync_lds();
  }

  __device__ static void run(const Row& r, const float* weights, const uint32_t* selm, float* scratch, int lane,
                             int w, float* acc, float& accz) {
    const int nb = r.n_q / kBlock;
    const int steps = (nb + kWaves * 4 - 1) / (kWaves * 4);
    Buf b0, b1, b2;
    load(r, 0, lane, w, b0);
    if (1 < steps) load(r, 1, lane, w, b1);
    for (int s = 0; s < steps; s += 3) {
      if (s + 2 < steps) load(r, s + 2, lane, w, b2);
      compute(r, weights, selm, scratch, s, lane, w, b0, acc, accz);
      if (s + 1 >= steps) break;
      if (s + 3 < steps) load(r, s + 3, lane, w, b0);
      compute(r, weights, selm, scratch, s + 1, lane, w, b1, acc, accz);
      if (s + 2 >= steps) break;
      if (s + 4 < steps) load(r, s + 4, lane, w, b1);
      compute(r, weights, selm, scratch, s + 2, lane, w, b2, acc, accz);
    }
  }
};

struct Smem {
  float* scores;    // [lpad]; after the V pass: [kThreads][VCH] partials, then [kWaves][D] tail partials
  uint32_t* selm;   // [lpad / 32]
  uint32_t* boff;   // [lpad / 16] record offset of each logical block, 256-byte units
  float* qs;        // [D]
  float* wscr;      // [kWaves][kWaveScratch]
  float* misc;      // [64 + kWaves * 4]
};

template <int D, int MODE, bool SPARSE>
__device__ void row_body(const DecodeArgs& a, const Row& r, const Smem& sm, size_t orow) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  float* coef = sm.wscr + w * kWaveScratch;
  float* scores = sm.scores;
  uint32_t* selm = sm.selm;
  float* misc = sm.misc;
  constexpr int NE = D / kGroup;
  constexpr int VCH = D / 16;

  // ---- K pass (coarse / dense / 2-bit / KIVI-4 scores)
  float mloc = -INFINITY;
  KPass<D, MODE, false>::run(r, sm.qs, scores, selm, coef, lane, w, mloc);
  // tail: exact scores
  for (int t = r.n_q + w; t < r.N; t += kWaves) {
    const uint16_t* kt = r.tail + (size_t)(t % kGroup) * D;
    float p = 0.f;
    for (int d = lane; d < D; d += 64) p = fmaf(sm.qs[d], bf16f(kt[d]), p);
    p = wave_sum(p);
    if (lane == 0) {
      scores[t] = p;
      mloc = fmaxf(mloc, p);
    }
  }
  mloc = wave_max(mloc);
  if (lane == 0) misc[w] = mloc;
  __syncthreads();
  float m = misc[0];
  for (int i = 1; i < kWaves; ++i) m = fmaxf(m, misc[i]);
  // ---- row sum of the coarse softmax
  float ls = 0.f;
  for (int t = tid; t < r.N; t += kThreads) ls += __expf(scores[t] - m);
  ls = wave_sum(ls);
  if (lane == 0) misc[8 + w] = ls;
  __syncthreads();
  float l = 0.f;
  for (int i = 0; i < kWaves; ++i) l += misc[8 + i];

  // ---- selection masks (one u32 per 32-token group)
  if (SPARSE) {
    for (int base = 0; base < r.n_q; base += kThreads) {
      const int t = base + tid;
      bool pred = false;
      if (t < r.n_q) pred = __expf(scores[t] - m) / l >= a.tau;
      const unsigned long long bal = __ballot(pred);
      const int g0 = (base + 64 * w) / kGroup;
      if (lane == 0 && g0 < r.n_groups) selm[g0] = (uint32_t)bal;
      if (lane == 0 && g0 + 1 < r.n_groups) selm[g0 + 1] = (uint32_t)(bal >> 32);
    }
  } else {
    const uint32_t fill = (MODE == MODE_DENSE || MODE == MODE_KIVI) ? 0xffffffffu : 0u;
    for (int g = tid; g < r.n_groups; g += kThreads) selm[g] = fill;
  }
  __syncthreads();
  if (a.sel_mask) {
    uint32_t* smo = a.sel_mask + orow * (size_t)a.sel_words;
    for (int g = tid; g < a.sel_words; g += kThreads) smo[g] = g < r.n_groups ? selm[g] : 0u;
  }

  // ---- refinement of the selected scores
  float mfin = m;
  if (SPARSE) {
    float mref = -INFINITY;
    KPass<D, MODE_COARSE, true>::run(r, sm.qs, scores, selm, coef, lane, w, mref);
    mref = wave_max(mref);
    if (lane == 0) misc[16 + w] = mref;
    __syncthreads();
    for (int i = 0; i < kWaves; ++i) mfin = fmaxf(mfin, misc[16 + i]);
  }

  // ---- V pass
  // softmax weights w_t = exp(s_t - m') replace the scores in LDS
  float lsum = 0.f;
  for (int t = tid; t < r.N; t += kThreads) {
    const float wgt = __expf(scores[t] - mfin);
    scores[t] = wgt;
    lsum += wgt;
  }
  __syncthreads();
  const float* weights = scores;
  float acc[VCH];
#pragma unroll
  for (int c = 0; c < VCH; ++c) acc[c] = 0.f;
  float accz = 0.f;   // constant terms of channel group lane % NE
  VPass<D, MODE, SPARSE>::run(r, weights, selm, coef, lane, w, acc, accz);
  // tail values, exact
  float tacc[D / 64];
#pragma unroll
  for (int i = 0; i < D / 64; ++i) tacc[i] = 0.f;
  for (int t = r.n_q + w; t < r.N; t += kWaves) {
    const float wgt = weights[t];
    const uint16_t* vt = r.tail + (size_t)(kGroup + t % kGroup) * D;
#pragma unroll
    for (int i = 0; i < D / 64; ++i) tacc[i] = fmaf(wgt, bf16f(vt[lane + 64 * i]), tacc[i]);
  }
  __syncthreads();   // scores are dead from here on: reuse them for partials
  float* red = scores;                         // [kThreads][VCH]
  float* tred = scores + kThreads * VCH;       // [kWaves][D]
#pragma unroll
  for (int c = 0; c < VCH; ++c) red[tid * VCH + c] = acc[c];
#pragma unroll
  for (int i = 0; i < D / 64; ++i) tred[w * D + lane + 64 * i] = tacc[i];
  lsum = wave_sum(lsum);
  float zs[NE];
#pragma unroll
  for (int e = 0; e < NE; ++e) zs[e] = wave_sum((lane % NE) == e ? accz : 0.f);
  if (lane == 0) {
    misc[24 + w] = lsum;
#pragma unroll
    for (int e = 0; e < NE; ++e) misc[32 + w * 4 + e] = zs[e];
  }
  __syncthreads();
  float L = 0.f;
  for (int i = 0; i < kWaves; ++i) L += misc[24 + i];
  for (int d = tid; d < D; d += kThreads) {
    const int chunk = d / VCH, c = d % VCH;
    float o = 0.f;
    for (int ww = 0; ww < kWaves; ++ww) {
      o += misc[32 + ww * 4 + d / kGroup];
#pragma unroll
      for (int vb = 0; vb < 4; ++vb) o += red[(ww * 64 + vb * 16 + chunk) * VCH + c];
      o += tred[ww * D + d];
    }
    o = o / L;
    if (a.out_bf16) {
      uint32_t u = __float_as_uint(o);
      u += 0x7fffu + ((u >> 16) & 1u);
      reinterpret_cast<uint16_t*>(a.out)[orow * D + d] = (uint16_t)(u >> 16);
    } else {
      reinterpret_cast<float*>(a.out)[orow * D + d] = o;
    }
  }
}

__host__ __device__ inline size_t pad4(size_t n) { return (n + 3) / 4 * 4; }   // keep 16-byte alignment
__host__ __device__ inline size_t lds_lpad(int max_len) { return ((size_t)max_len + 63) / 64 * 64; }
__host__ __device__ inline size_t lds_region_a(int max_len, int D) {
  const size_t need = (size_t)kThreads * (D / 16) + (size_t)kWaves * D;
  const size_t lp = lds_lpad(max_len);
  return pad4(lp > need ? lp : need);
}
__host__ __device__ inline size_t decode_lds_floats(int max_len, int D) {
  const size_t lp = lds_lpad(max_len);
  return lds_region_a(max_len, D) + pad4(lp / 32) + pad4(lp / 16 + 16) + D + (size_t)kWaves * kWaveScratch + 64 +
         kWaves * 4;
}

// One kernel per selection regime of the launch (tau = 0, tau > 1, 0 < tau <= 1, or the
// KIVI-4 layout), so each variant gets its own register allocation; rows of 2-bit cells
// run the 2-bit path inside every planes variant.
enum : int { VAR_KIVI = 0, VAR_DENSE = 1, VAR_COARSE = 2, VAR_SPARSE = 3 };

template <int D, int VAR>
__global__ void __launch_bounds__(kThreads, 4) k_decode(DecodeArgs a) {
  extern __shared__ float smem[];
  const int row = blockIdx.x;
  const int h = row % a.n_heads;
  const int b = (row / a.n_heads) % a.n_seqs;
  const int ci = row / (a.n_heads * a.n_seqs);
  const DecodeCell cell = a.cells[ci];
  const int tid = threadIdx.x;
  const size_t orow = ((size_t)ci * a.n_seqs + b) * a.n_heads + h;
  const int N = a.seq_lens[b];

  const size_t lp = lds_lpad(a.max_len);
  Smem sm;
  sm.scores = smem;
  sm.selm = reinterpret_cast<uint32_t*>(smem + lds_region_a(a.max_len, D));
  sm.boff = sm.selm + pad4(lp / 32);
  sm.qs = reinterpret_cast<float*>(sm.boff + pad4(lp / 16 + 16));
  sm.wscr = sm.qs + D;
  sm.misc = sm.wscr + kWaves * kWaveScratch;

  if (N <= 0 || N > a.max_len) {
    const float v = N == 0 ? 0.f : __builtin_nanf("");
    for (int d = tid; d < D; d += kThreads) {
      if (a.out_bf16) reinterpret_cast<uint16_t*>(a.out)[orow * D + d] = N == 0 ? 0 : 0x7fc0;
      else reinterpret_cast<float*>(a.out)[orow * D + d] = v;
    }
    if (a.sel_mask)
      for (int g = tid; g < a.sel_words; g += kThreads) a.sel_mask[orow * (size_t)a.sel_words + g] = 0u;
    return;
  }

  Row r;
  r.pool = a.ws + cell.pool_off;
  r.boff = sm.boff;
  const int slot = a.seq_slots ? a.seq_slots[b] : b;
  r.tail = reinterpret_cast<const uint16_t*>(a.ws + cell.tail_off) + ((size_t)slot * a.n_heads + h) * tail_elems(D);
  r.N = N;
  r.n_q = (N / kGroup) * kGroup;
  r.n_groups = N / kGroup;

  // block table row and sigma * q into LDS
  const int32_t* bt = a.block_table + (size_t)b * a.bt_stride;
  const int nbq = r.n_q / kBlock;
  const uint32_t rec256 = (uint32_t)(record_bytes(cell.kind, D) / 256);
  for (int j = tid; j < nbq; j += kThreads) sm.boff[j] = ((uint32_t)bt[j] * (uint32_t)a.n_heads + (uint32_t)h) * rec256;
  for (int d = tid; d < D; d += kThreads) {
    const size_t qi = orow * D + d;
    const float qv = a.q_bf16 ? bf16f(reinterpret_cast<const uint16_t*>(a.q)[qi]) : reinterpret_cast<const float*>(a.q)[qi];
    sm.qs[d] = a.sm_scale * qv;
  }
  __syncthreads();

  if constexpr (VAR == VAR_KIVI) {
    row_body<D, MODE_KIVI, false>(a, r, sm, orow);
  } else {
    if (cell.kind == KIND_Q2) row_body<D, MODE_Q2, false>(a, r, sm, orow);
    else if (VAR == VAR_DENSE) row_body<D, MODE_DENSE, false>(a, r, sm, orow);
    else if (VAR == VAR_COARSE) row_body<D, MODE_COARSE, false>(a, r, sm, orow);
    else row_body<D, MODE_COARSE, true>(a, r, sm, orow);
  }
}

size_t decode_lds_bytes(int max_len, int head_dim) { return decode_lds_floats(max_len, head_dim) * 4; }

template <int D, int VAR>
static void launch_variant(const DecodeArgs& a, size_t rows, size_t lds, hipStream_t stream) {
  static bool attr_set = false;
  if (!attr_set) {
    (void)hipFuncSetAttribute((const void*)k_decode<D, VAR>, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    attr_set = true;
  }
  hipLaunchKernelGGL((k_decode<D, VAR>), dim3((unsigned)rows), dim3(kThreads), lds, stream, a);
}

template <int D>
static void launch_d(const DecodeArgs& a, size_t rows, size_t lds, hipStream_t stream) {
  if (a.cells[0].kind == KIND_KIVI4) launch_variant<D, VAR_KIVI>(a, rows, lds, stream);
  else if (a.tau <= 0.f) launch_variant<D, VAR_DENSE>(a, rows, lds, stream);
  else if (a.tau > 1.f) launch_variant<D, VAR_COARSE>(a, rows, lds, stream);
  else launch_variant<D, VAR_SPARSE>(a, rows, lds, stream);
}

hipError_t launch_decode(const DecodeArgs& a, int head_dim, hipStream_t stream) {
  const size_t rows = (size_t)a.n_cells * a.n_seqs * a.n_heads;
  if (rows == 0) return hipSuccess;
  const size_t lds = decode_lds_bytes(a.max_len, head_dim);
  if (head_dim == 128) launch_d<128>(a, rows, lds, stream);
  else launch_d<64>(a, rows, lds, stream);
  return hipGetLastError();
}

}  // namespace lkv
