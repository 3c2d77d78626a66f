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

// Sixteen 2-bit codes of one word. K order: cf[4k + p] for the code at byte k, bits 2p.
__device__ inline float dot16_k(uint32_t x, const float* cf, float acc) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t m = x & (0x03030303u << (2 * p));
#pragma unroll
    for (int k = 0; k < 4; ++k) acc = fmaf(cf[4 * k + p], ubyte(m, k), acc);
  }
  return acc;
}
// V order: cf[4p + k] (token 4p + k of the block).
__device__ inline float dot16_v(uint32_t x, const float* cf, float acc) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t m = x & (0x03030303u << (2 * p));
#pragma unroll
    for (int k = 0; k < 4; ++k) acc = fmaf(cf[4 * p + k], ubyte(m, k), acc);
  }
  return acc;
}
// Eight 4-bit codes of one word. K order: cf[2k + n] for the nibble n of byte k.
__device__ inline float dot8_k4(uint32_t x, const float* cf, float acc) {
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const uint32_t m = x & (0x0F0F0F0Fu << (4 * n));
#pragma unroll
    for (int k = 0; k < 4; ++k) acc = fmaf(cf[2 * k + n], ubyte(m, k), acc);
  }
  return acc;
}
// V order: cf[4n + k] (token 4n + k of the word's 8 tokens).
__device__ inline float dot8_v4(uint32_t x, const float* cf, float acc) {
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const uint32_t m = x & (0x0F0F0F0Fu << (4 * n));
#pragma unroll
    for (int k = 0; k < 4; ++k) acc = fmaf(cf[4 * n + k], ubyte(m, k), acc);
  }
  return acc;
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

__device__ inline uint32_t w4(const uint4& v, int i) { return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w; }

struct Row {
  const uint8_t* pool;     // pool base of the storage cell
  const int32_t* btl;      // block table row of the sequence (in LDS)
  const uint16_t* tail;    // tail of (slot, head): [2][32][D] bf16
  int H, h, rec, N, n_q, n_groups;
  __device__ inline const uint8_t* rec_ptr(int j) const {
    return pool + ((size_t)btl[j] * H + h) * (size_t)rec;
  }
};

// ----------------------------------------------------------------------------- K pass
// Lane mapping per wave step: GPS groups, each covered by LPG = 4*COLS lanes
// (2 blocks x 2 token octets x COLS columns of UNIT channels). A lane reads the 8
// words of its column for 8 consecutive tokens and keeps 8 partial scores, which
// are summed over the COLS column lanes with DPP. Coefficients of a group are
// built by the LPG lanes of the group (CPL channels each) and passed through LDS.
template <int D, int MODE, bool REFINE>
struct KPass {
  static constexpr bool KIVI = MODE == MODE_KIVI;
  static constexpr bool DENSE = MODE == MODE_DENSE && !REFINE;
  static constexpr int UNIT = KIVI ? 8 : 16;
  static constexpr int COLS = D / UNIT;
  static constexpr int LPG = 4 * COLS;
  static constexpr int GPS = 64 / LPG;
  static constexpr int CPL = UNIT / 4;
  static constexpr int KMETA = KIVI ? off_kmeta_kivi(D) : off_kmeta_planes(D);
  static constexpr int CODE_OFF = REFINE ? off_klo(D) : 0;

  struct Buf {
    uint4 meta, c0, c1, l0, l1;
    bool vm, vc;
  };

  __device__ static inline void load(const Row& r, const uint32_t* selm, int s, int lane, int w, Buf& b) {
    const int gbase = (s * kWaves + w) * GPS;
    const int idx = lane * CPL;
    const int gm = gbase + idx / D, ch = idx % D;
    b.vm = gm < r.n_groups && (!REFINE || selm[gm] != 0u);
    if (b.vm) {
      const uint8_t* p = r.rec_ptr(2 * gm + (ch >= D / 2)) + KMETA + 4 * (ch % (D / 2));
      b.meta = CPL == 4 ? ld_stream4(p) : ld_stream2(p);
    }
    const int rl = lane % LPG;
    const int blk = rl / (2 * COLS), oct = (rl / COLS) & 1, col = rl % COLS;
    const int gc = gbase + lane / LPG;
    b.vc = gc < r.n_groups && (!REFINE || selm[gc] != 0u);
    if (b.vc) {
      const uint8_t* rb = r.rec_ptr(2 * gc + blk);
      const uint8_t* kp = rb + CODE_OFF + (col * kBlock + oct * 8) * 4;
      b.c0 = ld_stream4(kp);
      b.c1 = ld_stream4(kp + 16);
      if (DENSE) {
        const uint8_t* lp = rb + off_klo(D) + (col * kBlock + oct * 8) * 4;
        b.l0 = ld_stream4(lp);
        b.l1 = ld_stream4(lp + 16);
      }
    }
  }

  __device__ static inline void compute(const Row& r, const float* qs, float* scores, const uint32_t* selm,
                                        float* coef, int s, int lane, int w, const Buf& b, float& mloc) {
    const int gbase = (s * kWaves + w) * GPS;
    const int idx = lane * CPL;
    const int gsm = idx / D, ch0 = idx % D;
    // coefficients of CPL consecutive channels; stored [column][byte k][bit pair p]
    float cst = 0.f;
    if (b.vm) {
      float cv[CPL];
#pragma unroll
      for (int rr = 0; rr < CPL; ++rr) {
        const uint32_t mw = w4(b.meta, rr);
        const int ch = ch0 + rr;
        const float sc = f16lo(mw), z = f16hi(mw), qv = qs[ch];
        const float qsv = qv * sc;
        const float pre = KIVI ? (rr ? 1.f / 16.f : 1.f)
                               : (rr == 0 ? 1.f : rr == 1 ? 0.25f : rr == 2 ? 0.0625f : 0.015625f);
        if (REFINE) {
          cv[rr] = qsv * pre;
          cst = fmaf(-1.5f, qsv, cst);
        } else if (MODE == MODE_COARSE || MODE == MODE_DENSE) {
          cv[rr] = 4.f * qsv * pre;
          cst += (MODE == MODE_COARSE) ? qv * fmaf(1.5f, sc, z) : qv * z;
        } else {
          cv[rr] = qsv * pre;
          cst = fmaf(qv, z, cst);
        }
      }
      float* dst = coef + gsm * D + ch0;   // CPL consecutive floats
      if (CPL == 4) *reinterpret_cast<float4*>(dst) = make_float4(cv[0], cv[1], cv[2], cv[3]);
      else *reinterpret_cast<float2*>(dst) = make_float2(cv[0], cv[CPL - 1]);
    }
    cst = group_sum<LPG>(cst);
    wave_sync_lds();

    const int gsub = lane / LPG;
    const int rl = lane % LPG;
    const int blk = rl / (2 * COLS), oct = (rl / COLS) & 1, col = rl % COLS;
    float part[8], partl[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) part[j] = partl[j] = 0.f;
    if (b.vc) {
      float cf[UNIT];
      const float4* cp = reinterpret_cast<const float4*>(coef + gsub * D + col * UNIT);
#pragma unroll
      for (int u = 0; u < UNIT / 4; ++u) {
        const float4 t = cp[u];
        cf[4 * u] = t.x;
        cf[4 * u + 1] = t.y;
        cf[4 * u + 2] = t.z;
        cf[4 * u + 3] = t.w;
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t x = j < 4 ? w4(b.c0, j) : w4(b.c1, j - 4);
        part[j] = KIVI ? dot8_k4(x, cf, 0.f) : dot16_k(x, cf, 0.f);
        if (DENSE) partl[j] = dot16_k(j < 4 ? w4(b.l0, j) : w4(b.l1, j - 4), cf, 0.f);
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (DENSE) part[j] = fmaf(0.25f, partl[j], part[j]);
      part[j] = group_sum<COLS>(part[j]);
    }
    if (b.vc) {
      const int g = gbase + gsub;
      const uint32_t gm = REFINE ? selm[g] : 0u;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if ((j % COLS) == col) {
          const int tt = blk * kBlock + oct * 8 + j;
          const int t = g * kGroup + tt;
          if (REFINE) {
            if ((gm >> tt) & 1u) {
              const float sc = scores[t] + cst + part[j];
              scores[t] = sc;
              mloc = fmaxf(mloc, sc);
            }
          } else {
            const float sc = cst + part[j];
            scores[t] = sc;
            mloc = fmaxf(mloc, sc);
          }
        }
      }
    }
    wave_sync_lds();
  }

  __device__ static void run(const Row& r, const float* qs, float* scores, const uint32_t* selm, float* coef,
                             int lane, int w, float& mloc) {
    const int steps = (r.n_groups + kWaves * GPS - 1) / (kWaves * GPS);
    Buf cur, nxt;
    load(r, selm, 0, lane, w, cur);
    for (int s = 0; s < steps; ++s) {
      if (s + 1 < steps) load(r, selm, s + 1, lane, w, nxt);
      if (!REFINE || __any(cur.vm))
        compute(r, qs, scores, selm, coef, s, lane, w, cur, mloc);
      cur = nxt;
    }
  }
};

// ----------------------------------------------------------------------------- V pass
// Lane mapping per wave step: 4 blocks (64 tokens). Lane t of the step first folds
// weight, scale and bucket offset of its token into LDS coefficients (one per
// 32-channel group); then lane (block, chunk) reads the V words of its D/16
// channels (16 tokens per word) and accumulates.
template <int D, int MODE, bool SPARSE>
struct VPass {
  static constexpr bool KIVI = MODE == MODE_KIVI;
  static constexpr int VCH = D / 16;            // channels per lane
  static constexpr int NE = D / kGroup;         // channel groups
  static constexpr int WPL = KIVI ? 2 * VCH : VCH;  // V words per lane
  static constexpr int NV4 = WPL / 4;           // uint4 loads per lane
  static constexpr int VOFF = KIVI ? off_v_kivi(D) : off_v_planes(D);
  static constexpr int VMETA = KIVI ? off_vmeta_kivi(D) : off_vmeta_planes(D);
  static constexpr bool DENSE = MODE == MODE_DENSE;

  struct Buf {
    uint4 meta;
    uint4 c[NV4];
    uint4 l[DENSE ? NV4 : 1];
    bool v;
  };

  __device__ static inline void load(const Row& r, int s, int lane, int w, Buf& b) {
    const int nb = r.n_q / kBlock;
    const int j = (s * kWaves + w) * 4 + lane / 16;
    b.v = j < nb;
    if (!b.v) return;
    const uint8_t* rb = r.rec_ptr(j);
    const int t16 = lane % 16, chunk = lane % 16;
    const uint8_t* mp = rb + VMETA + 4 * NE * t16;
    b.meta = NE == 4 ? ld_stream4(mp) : ld_stream2(mp);
    const uint8_t* vp = rb + VOFF + chunk * WPL * 4;
#pragma unroll
    for (int i = 0; i < NV4; ++i) b.c[i] = ld_stream4(vp + 16 * i);
    if (DENSE) {
      const uint8_t* lp = rb + off_vlo(D) + chunk * WPL * 4;
#pragma unroll
      for (int i = 0; i < NV4; ++i) b.l[i] = ld_stream4(lp + 16 * i);
    }
  }

  __device__ static inline void compute(const Row& r, const float* scores, const uint32_t* selm, float* coefv,
                                        int s, int lane, int w, float mfin, const Buf& b, float* acc,
                                        float* accl, float* accz, float& lsum) {
    const int jb = lane / 16, t16 = lane % 16;
    const int j = (s * kWaves + w) * 4 + jb;
    if (b.v) {
      const int t = j * kBlock + t16;
      const float wgt = __expf(scores[t] - mfin);
      bool sel = DENSE;
      if (SPARSE) sel = (selm[t >> 5] >> (t & 31)) & 1u;
      float pre;
      if (KIVI) pre = ((t16 & 7) >> 2) ? (1.f / 16.f) : 1.f;
      else {
        const int p = t16 >> 2;
        pre = p == 0 ? 1.f : p == 1 ? 0.25f : p == 2 ? 0.0625f : 0.015625f;
      }
      const float mult = (MODE == MODE_Q2 || KIVI) ? 1.f : 4.f;
#pragma unroll
      for (int e = 0; e < NE; ++e) {
        const uint32_t mw = w4(b.meta, e);
        const float sc = f16lo(mw), z = f16hi(mw);
        const float ws = wgt * sc;
        coefv[(jb * NE + e) * 16 + t16] = mult * ws * pre;
        const bool mid = (MODE == MODE_COARSE) && !sel;
        accz[e] = fmaf(wgt, mid ? fmaf(1.5f, sc, z) : z, accz[e]);
      }
      lsum += wgt;
    }
    wave_sync_lds();
    if (b.v) {
      const int chunk = lane % 16;
      const int e_lane = (chunk * VCH) / kGroup;
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
      if (KIVI) {
#pragma unroll
        for (int c = 0; c < VCH; ++c) {
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) acc[c] = dot8_v4(w4(b.c[(2 * c + jj) / 4], (2 * c + jj) % 4), cf + 8 * jj, acc[c]);
        }
      } else {
#pragma unroll
        for (int c = 0; c < VCH; ++c) acc[c] = dot16_v(w4(b.c[c / 4], c % 4), cf, acc[c]);
        if (DENSE) {
#pragma unroll
          for (int c = 0; c < VCH; ++c) accl[c] = dot16_v(w4(b.l[c / 4], c % 4), cf, accl[c]);
        }
        if (SPARSE) {
          const uint32_t bm = (selm[j >> 1] >> (16 * (j & 1))) & 0xffffu;
          if (bm) {
            uint32_t m32 = 0;
#pragma unroll
            for (int tt = 0; tt < 16; ++tt)
              if ((bm >> tt) & 1u) m32 |= 3u << (8 * (tt & 3) + 2 * (tt >> 2));
            const uint4* lp = reinterpret_cast<const uint4*>(r.rec_ptr(j) + off_vlo(D) + chunk * VCH * 4);
            uint4 lw[NV4];
#pragma unroll
            for (int i = 0; i < NV4; ++i) lw[i] = lp[i];
#pragma unroll
            for (int c = 0; c < VCH; ++c) accl[c] = dot16_v(w4(lw[c / 4], c % 4) & m32, cf, accl[c]);
          }
        }
      }
    }
    wave_sync_lds();
  }

  __device__ static void run(const Row& r, const float* scores, const uint32_t* selm, float* coefv, int lane,
                             int w, float mfin, float* acc, float* accl, float* accz, float& lsum) {
    const int nb = r.n_q / kBlock;
    const int steps = (nb + kWaves * 4 - 1) / (kWaves * 4);
    Buf cur, nxt;
    load(r, 0, lane, w, cur);
    for (int s = 0; s < steps; ++s) {
      if (s + 1 < steps) load(r, s + 1, lane, w, nxt);
      compute(r, scores, selm, coefv, s, lane, w, mfin, cur, acc, accl, accz, lsum);
      cur = nxt;
    }
  }
};

struct Smem {
  float* scores;    // [lpad]; after the V pass: [kThreads][VCH] partials, then [kWaves][D] tail partials
  uint32_t* selm;   // [lpad / 32]
  int32_t* btl;     // [lpad / 16]
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
  float acc[VCH], accl[VCH], accz[NE];
#pragma unroll
  for (int c = 0; c < VCH; ++c) acc[c] = accl[c] = 0.f;
#pragma unroll
  for (int e = 0; e < NE; ++e) accz[e] = 0.f;
  float lsum = 0.f;
  VPass<D, MODE, SPARSE>::run(r, scores, selm, coef, lane, w, mfin, acc, accl, accz, lsum);
  // tail values, exact
  float tacc[D / 64];
#pragma unroll
  for (int i = 0; i < D / 64; ++i) tacc[i] = 0.f;
  for (int t = r.n_q + w; t < r.N; t += kWaves) {
    const float wgt = __expf(scores[t] - mfin);
    const uint16_t* vt = r.tail + (size_t)(kGroup + t % kGroup) * D;
#pragma unroll
    for (int i = 0; i < D / 64; ++i) tacc[i] = fmaf(wgt, bf16f(vt[lane + 64 * i]), tacc[i]);
    if (lane == 0) lsum += wgt;
  }
  __syncthreads();   // scores are dead from here on: reuse them for partials
  float* red = scores;                         // [kThreads][VCH]
  float* tred = scores + kThreads * VCH;       // [kWaves][D]
#pragma unroll
  for (int c = 0; c < VCH; ++c) red[tid * VCH + c] = fmaf(0.25f, accl[c], acc[c]);
#pragma unroll
  for (int i = 0; i < D / 64; ++i) tred[w * D + lane + 64 * i] = tacc[i];
  lsum = wave_sum(lsum);
#pragma unroll
  for (int e = 0; e < NE; ++e) accz[e] = wave_sum(accz[e]);
  if (lane == 0) {
    misc[24 + w] = lsum;
#pragma unroll
    for (int e = 0; e < NE; ++e) misc[32 + w * 4 + e] = accz[e];
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

__host__ __device__ inline size_t lds_lpad(int max_len) { return ((size_t)max_len + 63) / 64 * 64; }
__host__ __device__ inline size_t lds_region_a(int max_len, int D) {
  const size_t need = (size_t)kThreads * (D / 16) + (size_t)kWaves * D;
  const size_t lp = lds_lpad(max_len);
  return lp > need ? lp : need;
}
__host__ __device__ inline size_t decode_lds_floats(int max_len, int D) {
  const size_t lp = lds_lpad(max_len);
  return lds_region_a(max_len, D) + lp / 32 + lp / 16 + 16 + D + (size_t)kWaves * kWaveScratch + 64 + kWaves * 4;
}

template <int D>
__global__ void __launch_bounds__(kThreads) k_decode(DecodeArgs a) {
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
  sm.btl = reinterpret_cast<int32_t*>(sm.selm + lp / 32);
  sm.qs = reinterpret_cast<float*>(sm.btl + lp / 16 + 16);
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
  r.btl = sm.btl;
  const int slot = a.seq_slots ? a.seq_slots[b] : b;
  r.tail = reinterpret_cast<const uint16_t*>(a.ws + cell.tail_off) + ((size_t)slot * a.n_heads + h) * tail_elems(D);
  r.H = a.n_heads;
  r.h = h;
  r.rec = record_bytes(cell.kind, D);
  r.N = N;
  r.n_q = (N / kGroup) * kGroup;
  r.n_groups = N / kGroup;

  // block table row and sigma * q into LDS
  const int32_t* bt = a.block_table + (size_t)b * a.bt_stride;
  const int nbq = r.n_q / kBlock;
  for (int j = tid; j < nbq; j += kThreads) sm.btl[j] = bt[j];
  for (int d = tid; d < D; d += kThreads) {
    const size_t qi = orow * D + d;
    const float qv = a.q_bf16 ? bf16f(reinterpret_cast<const uint16_t*>(a.q)[qi]) : reinterpret_cast<const float*>(a.q)[qi];
    sm.qs[d] = a.sm_scale * qv;
  }
  __syncthreads();

  if (cell.kind == KIND_KIVI4) {
    row_body<D, MODE_KIVI, false>(a, r, sm, orow);
  } else if (cell.kind == KIND_Q2) {
    row_body<D, MODE_Q2, false>(a, r, sm, orow);
  } else if (a.tau <= 0.f) {
    row_body<D, MODE_DENSE, false>(a, r, sm, orow);
  } else if (a.tau > 1.f) {
    row_body<D, MODE_COARSE, false>(a, r, sm, orow);
  } else {
    row_body<D, MODE_COARSE, true>(a, r, sm, orow);
  }
}

size_t decode_lds_bytes(int max_len, int head_dim) { return decode_lds_floats(max_len, head_dim) * 4; }

hipError_t launch_decode(const DecodeArgs& a, int head_dim, hipStream_t stream) {
  const size_t rows = (size_t)a.n_cells * a.n_seqs * a.n_heads;
  if (rows == 0) return hipSuccess;
  const size_t lds = decode_lds_bytes(a.max_len, head_dim);
  static bool attr_set[2] = {false, false};
  if (head_dim == 128) {
    if (!attr_set[1]) {
      (void)hipFuncSetAttribute((const void*)k_decode<128>, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
      attr_set[1] = true;
    }
    hipLaunchKernelGGL(k_decode<128>, dim3((unsigned)rows), dim3(kThreads), lds, stream, a);
  } else {
    if (!attr_set[0]) {
      (void)hipFuncSetAttribute((const void*)k_decode<64>, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
      attr_set[0] = true;
    }
    hipLaunchKernelGGL(k_decode<64>, dim3((unsigned)rows), dim3(kThreads), lds, stream, a);
  }
  return hipGetLastError();
}

}  // namespace lkv
