// Loop-aware decode attention over the per-(loop, layer) mixed-precision KV cache (gfx950).
//
// Source: "LoopKV: Loop-Aware KV Cache Compression for Serving Looped
// Transformers" (arXiv:2611.04137), Abstract: during decoding each loop reads
// the high 2 bits of every 4-bit value and fetches the low bits only where its
// own attention weights require 4-bit precision; low-attention values are read
// at low precision rather than skipped; a reuse cell reads the final loop's KV;
// KIVI-4 (uniform 4-bit) runs on the same kernel as the baseline.
//
// One workgroup (4 wave64s) owns one row (cell, sequence, head). The path is
// HBM-bound with a VALU co-limit, so no MFMA: 2-bit codes are widened with
// in-place byte masks and v_cvt_f32_ubyteN, and every per-group / per-token
// scale is folded into the coefficient that multiplies the code.
//
//   K pass   coarse scores s_t = sigma q . (z + s (4 hi + 3/2)) from the high plane
//            (4-bit target), full scores for tau = 0 and KIVI-4, 2-bit scores for a
//            2-bit target; the tail (last len mod 32 tokens) is exact bf16. Scores
//            stay in LDS (4 bytes per token).
//   stats    m = max s, l = sum exp(s - m) over the whole row.
//   select   token t of the quantized prefix is selected when exp(s_t - m)/l >= tau;
//            a ballot per 64 tokens gives one 32-bit mask per 32-token group.
//   refine   only groups with a selected token: gather their low K plane and add
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

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kWaveScratch = 512;   // floats of per-wave LDS scratch

enum : int { MODE_COARSE = 0, MODE_DENSE = 1, MODE_Q2 = 2, MODE_KIVI = 3 };

__device__ inline void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ inline float wave_sum(float v) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}
__device__ inline float wave_max(float v) {
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

__device__ inline float f16lo(uint32_t w) { return __half2float(__ushort_as_half((unsigned short)(w & 0xffffu))); }
__device__ inline float f16hi(uint32_t w) { return __half2float(__ushort_as_half((unsigned short)(w >> 16))); }
__device__ inline float bf16f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ inline float ubyte(uint32_t x, int k) { return (float)((x >> (8 * k)) & 0xffu); }

// Sixteen 2-bit codes of one word; cf[4p + k] multiplies the code at byte k, bits 2p.
__device__ inline float dot16_2bit(uint32_t x, const float* cf, float acc) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t m = x & (0x03030303u << (2 * p));
#pragma unroll
    for (int k = 0; k < 4; ++k) acc = fmaf(cf[4 * p + k], ubyte(m, k), acc);
  }
  return acc;
}
// Eight 4-bit codes of one word; cf[4n + k] multiplies the code at byte k, nibble n.
__device__ inline float dot8_4bit(uint32_t x, const float* cf, float acc) {
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const uint32_t m = x & (0x0F0F0F0Fu << (4 * n));
#pragma unroll
    for (int k = 0; k < 4; ++k) acc = fmaf(cf[4 * n + k], ubyte(m, k), acc);
  }
  return acc;
}

struct Row {
  const uint8_t* pool;     // pool base of the storage cell
  const int32_t* bt;       // block table row of the sequence
  const uint16_t* tail;    // tail of (slot, head): [2][32][D] bf16
  int H, h, rec, N, n_q, n_groups;
  __device__ inline const uint8_t* rec_ptr(int j) const {
    return pool + ((size_t)bt[j] * H + h) * (size_t)rec;
  }
};

// ----------------------------------------------------------------------------- K pass
// Lane mapping per wave step: GPS groups, each covered by LPG = 4*COLS lanes
// (2 blocks x 2 token octets x COLS columns of UNIT channels). A lane reads 8
// consecutive words of its column (8 tokens) and keeps 8 partial scores, which
// are summed over the COLS column lanes with xor shuffles.
template <int D, int MODE, bool REFINE>
__device__ void k_pass(const Row& r, const float* qs, float* scores, const uint32_t* selm,
                       float* wscr, int lane, int w, float& mloc) {
  constexpr bool KIVI = MODE == MODE_KIVI;
  constexpr int UNIT = KIVI ? 8 : 16;
  constexpr int COLS = D / UNIT;
  constexpr int LPG = 4 * COLS;
  constexpr int GPS = 64 / LPG;
  constexpr int CPL = UNIT / 4;
  constexpr int KMETA = KIVI ? off_kmeta_kivi(D) : off_kmeta_planes(D);
  const int gsub = lane / LPG;
  const int rl = lane % LPG;
  const int blk = rl / (2 * COLS), oct = (rl / COLS) & 1, col = rl % COLS;
  float* coef = wscr;             // [GPS][D]
  float* coefl = wscr + GPS * D;  // [GPS][D]

  for (int it = 0;; ++it) {
    const int gbase = (it * kWaves + w) * GPS;
    if (gbase >= r.n_groups) break;
    if (REFINE) {
      bool any = false;
#pragma unroll
      for (int gs = 0; gs < GPS; ++gs) any |= (gbase + gs < r.n_groups) && selm[gbase + gs] != 0u;
      if (!any) continue;
    }
    // Per-(group, channel) coefficients, each lane CPL channels of one group.
    float cst = 0.f;
#pragma unroll
    for (int rr = 0; rr < CPL; ++rr) {
      const int idx = lane * CPL + rr;
      const int gs = idx / D, ch = idx % D;
      const int g = gbase + gs;
      if (g < r.n_groups) {
        const uint32_t mw = *reinterpret_cast<const uint32_t*>(
            r.rec_ptr(2 * g + (ch >= D / 2)) + KMETA + 4 * (ch % (D / 2)));
        const float s = f16lo(mw), z = f16hi(mw), qv = qs[ch];
        int pos;
        float pre;
        if (KIVI) {
          const int n = ch & 1;
          pos = (ch / 8) * 8 + n * 4 + ((ch >> 1) & 3);
          pre = n ? (1.f / 16.f) : 1.f;
        } else {
          const int p = ch & 3;
          pos = (ch / 16) * 16 + p * 4 + ((ch >> 2) & 3);
          pre = p == 0 ? 1.f : p == 1 ? 0.25f : p == 2 ? 0.0625f : 0.015625f;
        }
        const float qsv = qv * s;
        if (REFINE) {
          coefl[gs * D + pos] = qsv * pre;
          cst = fmaf(-1.5f, qsv, cst);
        } else if (MODE == MODE_COARSE) {
          coef[gs * D + pos] = 4.f * qsv * pre;
          cst += qv * fmaf(1.5f, s, z);
        } else if (MODE == MODE_DENSE) {
          coef[gs * D + pos] = 4.f * qsv * pre;
          coefl[gs * D + pos] = qsv * pre;
          cst = fmaf(qv, z, cst);
        } else {
          coef[gs * D + pos] = qsv * pre;
          cst = fmaf(qv, z, cst);
        }
      }
    }
#pragma unroll
    for (int off = 1; off < LPG; off <<= 1) cst += __shfl_xor(cst, off);
    wave_sync_lds();

    const int g = gbase + gsub;
    const bool active = g < r.n_groups && (!REFINE || selm[g] != 0u);
    if (active) {
      const uint8_t* rb = r.rec_ptr(2 * g + blk);
      const int woff = (col * kBlock + oct * 8) * 4;
      float part[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) part[j] = 0.f;
      if (!REFINE) {
        const uint4* kp = reinterpret_cast<const uint4*>(rb + woff);
        const uint4 x0 = kp[0], x1 = kp[1];
        const uint32_t xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
        float cf[UNIT];
#pragma unroll
        for (int u = 0; u < UNIT; ++u) cf[u] = coef[gsub * D + col * UNIT + u];
#pragma unroll
        for (int j = 0; j < 8; ++j) part[j] = KIVI ? dot8_4bit(xs[j], cf, 0.f) : dot16_2bit(xs[j], cf, 0.f);
      }
      if (REFINE || MODE == MODE_DENSE) {
        const uint4* lp = reinterpret_cast<const uint4*>(rb + off_klo(D) + woff);
        const uint4 y0 = lp[0], y1 = lp[1];
        const uint32_t ys[8] = {y0.x, y0.y, y0.z, y0.w, y1.x, y1.y, y1.z, y1.w};
        float cl[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) cl[u] = coefl[gsub * D + col * 16 + u];
#pragma unroll
        for (int j = 0; j < 8; ++j) part[j] = dot16_2bit(ys[j], cl, part[j]);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
#pragma unroll
        for (int off = 1; off < COLS; off <<= 1) part[j] += __shfl_xor(part[j], off);
      }
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
}

// ----------------------------------------------------------------------------- V pass
// Lane mapping per wave step: BPS blocks, each covered by LPB lanes of VCH
// channels. First every lane folds weight, scale and bucket offset of a few
// (token, channel group) pairs into LDS coefficients; then each lane reads the
// V words of its channels (16 tokens per word) and accumulates.
template <int D, int MODE, bool SPARSE>
__device__ void v_pass(const Row& r, const float* scores, const uint32_t* selm, float* wscr,
                       int lane, int w, float mfin, float* acc, float& accz, float& lsum) {
  constexpr bool KIVI = MODE == MODE_KIVI;
  constexpr int VCH = KIVI ? 4 : 8;
  constexpr int LPB = D / VCH;
  constexpr int BPS = 64 / LPB;
  constexpr int NE = D / kGroup;
  constexpr int ITEMS = kBlock * BPS * NE / 64;
  constexpr int VOFF = KIVI ? off_v_kivi(D) : off_v_planes(D);
  constexpr int VMETA = KIVI ? off_vmeta_kivi(D) : off_vmeta_planes(D);
  const int vblk = lane / LPB, chunk = lane % LPB;
  const int e_lane = (chunk * VCH) / kGroup;
  float* coefv = wscr;                    // [BPS][NE][16]
  float* coefvl = wscr + BPS * NE * 16;   // [BPS][NE][16]
  const int nb = r.n_q / kBlock;

  for (int it = 0;; ++it) {
    const int jbase = (it * kWaves + w) * BPS;
    if (jbase >= nb) break;
#pragma unroll
    for (int q = 0; q < ITEMS; ++q) {
      const int idx = lane + 64 * q;
      const int e = idx % NE, tt = idx / NE;
      const int jb = tt / kBlock, t16 = tt % kBlock;
      const int j = jbase + jb;
      float ahi = 0.f, alo = 0.f;
      if (j < nb) {
        const int t = j * kBlock + t16;
        const float wgt = __expf(scores[t] - mfin);
        const uint32_t mw = *reinterpret_cast<const uint32_t*>(r.rec_ptr(j) + VMETA + 4 * (t16 * NE + e));
        const float s = f16lo(mw), z = f16hi(mw);
        const float ws = wgt * s;
        if (KIVI) {
          ahi = ws * (((t16 & 7) >> 2) ? (1.f / 16.f) : 1.f);
          accz = fmaf(wgt, z, accz);
        } else {
          const int p = t16 >> 2;
          const float pre = p == 0 ? 1.f : p == 1 ? 0.25f : p == 2 ? 0.0625f : 0.015625f;
          if (MODE == MODE_Q2) {
            ahi = ws * pre;
            accz = fmaf(wgt, z, accz);
          } else {
            ahi = 4.f * ws * pre;
            bool sel = MODE == MODE_DENSE;
            if (SPARSE) sel = (selm[t >> 5] >> (t & 31)) & 1u;
            if (sel) {
              alo = ws * pre;
              accz = fmaf(wgt, z, accz);
            } else {
              accz = fmaf(wgt, fmaf(1.5f, s, z), accz);
            }
          }
        }
        if (e == 0) lsum += wgt;
      }
      coefv[(jb * NE + e) * 16 + t16] = ahi;
      coefvl[(jb * NE + e) * 16 + t16] = alo;
    }
    wave_sync_lds();

    const int j = jbase + vblk;
    if (j < nb) {
      const uint8_t* rb = r.rec_ptr(j);
      float cf[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) cf[u] = coefv[(vblk * NE + e_lane) * 16 + u];
      if (KIVI) {
        const uint4* vp = reinterpret_cast<const uint4*>(rb + VOFF + chunk * VCH * 8);
        const uint4 x0 = vp[0], x1 = vp[1];
        const uint32_t xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
        for (int c = 0; c < VCH; ++c) {
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) acc[c] = dot8_4bit(xs[2 * c + jj], cf + 8 * jj, acc[c]);
        }
      } else {
        const uint4* vp = reinterpret_cast<const uint4*>(rb + VOFF + chunk * VCH * 4);
        const uint4 x0 = vp[0], x1 = vp[1];
        const uint32_t xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
        for (int c = 0; c < VCH; ++c) acc[c] = dot16_2bit(xs[c], cf, acc[c]);
        bool need_lo = MODE == MODE_DENSE;
        if (SPARSE) need_lo = ((selm[j >> 1] >> (16 * (j & 1))) & 0xffffu) != 0u;
        if (MODE != MODE_Q2 && need_lo) {
          float cl[16];
#pragma unroll
          for (int u = 0; u < 16; ++u) cl[u] = coefvl[(vblk * NE + e_lane) * 16 + u];
          const uint4* lp = reinterpret_cast<const uint4*>(rb + off_vlo(D) + chunk * VCH * 4);
          const uint4 y0 = lp[0], y1 = lp[1];
          const uint32_t ys[8] = {y0.x, y0.y, y0.z, y0.w, y1.x, y1.y, y1.z, y1.w};
#pragma unroll
          for (int c = 0; c < VCH; ++c) acc[c] = dot16_2bit(ys[c], cl, acc[c]);
        }
      }
    }
    wave_sync_lds();
  }
}

// KIVI-4 V words use the 4-bit coefficient order (token t' of 16, scaled by 16^-n).
// dot8_4bit consumes cf[4n + k] for the word's tokens 8jj + 4n + k, which is cf + 8jj.

template <int D, int MODE, bool SPARSE>
__device__ void row_body(const DecodeArgs& a, const Row& r, float* scores, uint32_t* selm, float* qs,
                         float* wscr_all, float* tred, float* misc, size_t orow, int ci, int b, int h) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  float* wscr = wscr_all + w * kWaveScratch;
  constexpr int NE = D / kGroup;
  constexpr int VCH = (MODE == MODE_KIVI) ? 4 : 8;
  constexpr int LPB = D / VCH;

  // ---- K pass (coarse / dense / 2-bit / KIVI-4 scores)
  float mloc = -INFINITY;
  k_pass<D, MODE, false>(r, qs, scores, selm, wscr, lane, w, mloc);
  // tail: exact scores
  for (int t = r.n_q + w; t < r.N; t += kWaves) {
    const uint16_t* kt = r.tail + (size_t)(t % kGroup) * D;
    float p = 0.f;
    for (int d = lane; d < D; d += 64) p = fmaf(qs[d], bf16f(kt[d]), p);
    p = wave_sum(p);
    if (lane == 0) {
      scores[t] = p;
      mloc = fmaxf(mloc, p);
    }
  }
  mloc = wave_max(mloc);
  if (lane == 0) misc[w] = mloc;
  __syncthreads();
  const float m = fmaxf(fmaxf(misc[0], misc[1]), fmaxf(misc[2], misc[3]));
  // ---- row sum of the coarse softmax
  float ls = 0.f;
  for (int t = tid; t < r.N; t += kThreads) ls += __expf(scores[t] - m);
  ls = wave_sum(ls);
  if (lane == 0) misc[4 + w] = ls;
  __syncthreads();
  const float l = (misc[4] + misc[5]) + (misc[6] + misc[7]);

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
    uint32_t* sm = a.sel_mask + orow * (size_t)a.sel_words;
    for (int g = tid; g < a.sel_words; g += kThreads) sm[g] = g < r.n_groups ? selm[g] : 0u;
  }

  // ---- refinement of the selected scores
  float mfin = m;
  if (SPARSE) {
    float mref = -INFINITY;
    k_pass<D, MODE_COARSE, true>(r, qs, scores, selm, wscr, lane, w, mref);
    mref = wave_max(mref);
    if (lane == 0) misc[8 + w] = mref;
    __syncthreads();
    mfin = fmaxf(m, fmaxf(fmaxf(misc[8], misc[9]), fmaxf(misc[10], misc[11])));
  }

  // ---- V pass
  float acc[VCH];
#pragma unroll
  for (int c = 0; c < VCH; ++c) acc[c] = 0.f;
  float accz = 0.f, lsum = 0.f;
  v_pass<D, MODE, SPARSE>(r, scores, selm, wscr, lane, w, mfin, acc, accz, lsum);
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
  __syncthreads();   // all waves are done with their scratch
  float* red = wscr_all;   // [kWaves * 64][VCH]
#pragma unroll
  for (int c = 0; c < VCH; ++c) red[tid * VCH + c] = acc[c];
#pragma unroll
  for (int i = 0; i < D / 64; ++i) tred[w * D + lane + 64 * i] = tacc[i];
  float* zred = misc + 16;   // [kThreads]
  zred[tid] = accz;
  lsum = wave_sum(lsum);
  if (lane == 0) misc[12 + w] = lsum;
  __syncthreads();
  if (tid < NE) {
    float zs = 0.f;
    for (int i = tid; i < kThreads; i += NE) zs += zred[i];
    misc[16 + kThreads + tid] = zs;
  }
  __syncthreads();
  const float L = (misc[12] + misc[13]) + (misc[14] + misc[15]);
  for (int d = tid; d < D; d += kThreads) {
    const int chunk = d / VCH, c = d % VCH;
    float o = misc[16 + kThreads + d / kGroup];
    for (int ww = 0; ww < kWaves; ++ww) {
      for (int vb = 0; vb < 64 / LPB; ++vb) o += red[(ww * 64 + vb * LPB + chunk) * VCH + c];
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

__host__ __device__ inline size_t decode_lds_floats(int max_len, int D) {
  const size_t lpad = ((size_t)max_len + 63) / 64 * 64;
  return lpad + lpad / 32 + D + (size_t)kWaves * kWaveScratch + (size_t)kWaves * D + 16 + kThreads + 16;
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

  const size_t lpad = ((size_t)a.max_len + 63) / 64 * 64;
  float* scores = smem;
  uint32_t* selm = reinterpret_cast<uint32_t*>(smem + lpad);
  float* qs = smem + lpad + lpad / 32;
  float* wscr = qs + D;
  float* tred = wscr + kWaves * kWaveScratch;
  float* misc = tred + kWaves * D;

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
  r.bt = a.block_table + (size_t)b * a.bt_stride;
  const int slot = a.seq_slots ? a.seq_slots[b] : b;
  r.tail = reinterpret_cast<const uint16_t*>(a.ws + cell.tail_off) + ((size_t)slot * a.n_heads + h) * tail_elems(D);
  r.H = a.n_heads;
  r.h = h;
  r.rec = record_bytes(cell.kind, D);
  r.N = N;
  r.n_q = (N / kGroup) * kGroup;
  r.n_groups = N / kGroup;

  // sigma * q in LDS
  for (int d = tid; d < D; d += kThreads) {
    const size_t qi = orow * D + d;
    const float qv = a.q_bf16 ? bf16f(reinterpret_cast<const uint16_t*>(a.q)[qi]) : reinterpret_cast<const float*>(a.q)[qi];
    qs[d] = a.sm_scale * qv;
  }
  __syncthreads();

  if (cell.kind == KIND_KIVI4) {
    row_body<D, MODE_KIVI, false>(a, r, scores, selm, qs, wscr, tred, misc, orow, ci, b, h);
  } else if (cell.kind == KIND_Q2) {
    row_body<D, MODE_Q2, false>(a, r, scores, selm, qs, wscr, tred, misc, orow, ci, b, h);
  } else if (a.tau <= 0.f) {
    row_body<D, MODE_DENSE, false>(a, r, scores, selm, qs, wscr, tred, misc, orow, ci, b, h);
  } else if (a.tau > 1.f) {
    row_body<D, MODE_COARSE, false>(a, r, scores, selm, qs, wscr, tred, misc, orow, ci, b, h);
  } else {
    row_body<D, MODE_COARSE, true>(a, r, scores, selm, qs, wscr, tred, misc, orow, ci, b, h);
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
      hipFuncSetAttribute((const void*)k_decode<128>, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
      attr_set[1] = true;
    }
    hipLaunchKernelGGL(k_decode<128>, dim3((unsigned)rows), dim3(kThreads), lds, stream, a);
  } else {
    if (!attr_set[0]) {
      hipFuncSetAttribute((const void*)k_decode<64>, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
      attr_set[0] = true;
    }
    hipLaunchKernelGGL(k_decode<64>, dim3((unsigned)rows), dim3(kThreads), lds, stream, a);
  }
  return hipGetLastError();
}

}  // namespace lkv
