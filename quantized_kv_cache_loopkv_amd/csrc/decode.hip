// Loop-aware decode attention over the per-(loop, layer) mixed-precision KV cache (gfx950).
//
// Source: "LoopKV: Loop-Aware KV Cache Compression for Serving Looped
// Transformers" (arXiv:2611.04137), Abstract (sentences on decoding, on skipping,
// on the three storage choices and the serving sentence): a loop scores every key
// from the upper half of its 4-bit code and loads the lower half only for tokens
// whose weight in that loop is large enough to need the full code; tokens of small
// weight still count, read coarsely; a reuse cell reads the final loop's cache; the
// uniform 4-bit KIVI-4 layout goes through the same kernel as the baseline.
//
// One workgroup (8 wave64s) owns one row (cell, sequence, head); a whole plan is
// one launch of cells x sequences x heads workgroups. The path is HBM-bound with a
// VALU co-limit: codes are widened with byte masks and multiplied by fixed-point
// coefficients in exact integer arithmetic; the key scores' dot products run on the
// matrix cores (v_mfma_i32_16x16x64_i8, most rows of A zero: it takes integer work off the
// VALU, not a GEMM), the value sums on v_dot4.
//
// Single streaming pass (split-K online softmax): each wave walks its share of the
// row in steps of 32, 64 or 128 tokens. A step reads, for every 16-token block it covers,
// the K and V parts of the record that every token needs (one contiguous span of the
// record), and computes
//   K   scores s_t = sigma q . (z + s c) from the codes it read (4-bit target: high
//       plane, c = 4 hi + 3/2; 2-bit target: c; tau = 0 or KIVI-4: the 4-bit code);
//       the scores stay in LDS;
//   max the wave's running maximum m; on a new maximum its accumulators are rescaled;
//   V   weights w_t = exp(s_t - m) times the codes, accumulated per channel.
// The last (len mod GS) tokens are exact bf16 and join the same online softmax.
//
// Quantization groups GS of 32 (the default) or 64 tokens / channels are a template
// parameter; the kernel works in 32-token units either way (selection words, gathers,
// step geometry), and a unit of a 64-group reads its group's meta: K meta from the
// group's four records (a quarter each), V meta word e / 2 for 32-channel slice e.
//
// Selection (0 < tau <= 1, 4-bit target): after the pass the row's coarse maximum M
// and sum L are known; token t of the quantized prefix is selected when
// exp(s_t - M) / L >= tau. The 32-token units holding a selected token are gathered (a
// ballot over the per-unit masks); their low K plane refines the selected scores, and the
// selected tokens' contributions are corrected in place:
//   w' (z + s (4 hi + lo)) - w (z + s (4 hi + 3/2)),  w, w' = exp(coarse, refined - m).
// Token weights enter the value sums as 16-bit fixed point against the largest weight of
// their 16-token block, so a selected token that dominated its block and then loses most of
// its weight leaves its neighbours' rounding (up to 2^-16 of its coarse weight each) in the
// sum; relative to the output that error grows with removed / kept weight. Past 8 the row's
// V is recomputed from the final scores.
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>
#include <math.h>
#include "loopkv.h"
#include "layout.h"
#include "quantize.h"

namespace lkv {

#ifndef LKV_WAVES
#define LKV_WAVES 8
#endif
constexpr int kWaves = LKV_WAVES;           // waves per workgroup (one row)
constexpr int kThreads = 64 * kWaves;
constexpr int kWavesPerSimd = kWaves / 2;   // two workgroups per CU (LDS-bound)
// Words of per-wave LDS scratch: 256, or 272 for head dim 64, whose 128-token steps keep 128
// weights below the value limbs. (At 16K tokens a workgroup's LDS sits just under half of
// the CU's 160 KB, so two workgroups share a CU; the larger scratch would break that.)
__host__ __device__ constexpr int wave_scratch(int D) { return D == 64 ? 272 : 256; }

enum : int { MODE_COARSE = 0, MODE_DENSE = 1, MODE_Q2 = 2, MODE_KIVI = 3 };

// ----------------------------------------------------------------------------- helpers
__device__ inline void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// DPP lane moves. Every pattern used here (quad permutes, row mirrors, row rotates) reads a
// valid lane, so the old value is never kept: mov_dpp leaves it undefined and the move
// fuses into the consuming ALU op without initializing a destination first.
template <int CTRL>
__device__ inline float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}
template <int CTRL>
__device__ inline uint32_t dpp_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true);
}
// Cross-row exchanges without LDS (gfx950 permlane swaps): with both operands equal,
// permlane16_swap returns rows (0,0,2,2) and (1,1,3,3); permlane32_swap returns rows
// (0,1,0,1) and (2,3,2,3). Combining the pair reduces over row pairs / wave halves, with
// the same operand order in every lane.
__device__ inline float add_rows2(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ inline float add_halves(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ inline uint32_t max_rows2(uint32_t v) {
  const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return max((uint32_t)r[0], (uint32_t)r[1]);
}
__device__ inline uint32_t max_halves(uint32_t v) {
  const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return max((uint32_t)r[0], (uint32_t)r[1]);
}

// Sum over aligned groups of N lanes: quad swaps, half-row and row mirrors, then row pairs
// and wave halves. Every lane of a group ends with the same value.
template <int N>
__device__ inline float group_sum(float v) {
  if (N >= 2) v += dpp<0xB1>(v);    // quad_perm [1,0,3,2]
  if (N >= 4) v += dpp<0x4E>(v);    // quad_perm [2,3,0,1]
  if (N >= 8) v += dpp<0x141>(v);   // row_half_mirror
  if (N >= 16) v += dpp<0x140>(v);  // row_mirror
  if (N >= 32) v = add_rows2(v);
  if (N >= 64) v = add_halves(v);
  return v;
}
__device__ inline float wave_sum(float v) { return group_sum<64>(v); }
__device__ inline float uniform(float v) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v)));
}

// Max over aligned groups of N lanes of non-negative floats, compared as unsigned bit
// patterns (same order for values >= 0; fuses into DPP max instructions).
template <int N>
__device__ inline float group_max_nonneg(float x) {
  uint32_t v = __float_as_uint(x);
  if (N >= 2) v = max(v, dpp_u<0xB1>(v));
  if (N >= 4) v = max(v, dpp_u<0x4E>(v));
  if (N >= 8) v = max(v, dpp_u<0x141>(v));
  if (N >= 16) v = max(v, dpp_u<0x140>(v));
  if (N >= 32) v = max_rows2(v);
  if (N >= 64) v = max_halves(v);
  return __uint_as_float(v);
}
// Wave-uniform max of floats of any sign: order-preserving unsigned keys, row maxima by
// DPP, then the four row maxima read into scalars.
__device__ inline float wave_max(float x) {
  const uint32_t u = __float_as_uint(x);
  uint32_t k = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  k = max(k, dpp_u<0xB1>(k));
  k = max(k, dpp_u<0x4E>(k));
  k = max(k, dpp_u<0x141>(k));
  k = max(k, dpp_u<0x140>(k));
  const uint32_t m01 = max((uint32_t)__builtin_amdgcn_readlane((int)k, 0), (uint32_t)__builtin_amdgcn_readlane((int)k, 16));
  const uint32_t m23 = max((uint32_t)__builtin_amdgcn_readlane((int)k, 32), (uint32_t)__builtin_amdgcn_readlane((int)k, 48));
  const uint32_t m = max(m01, m23);
  return __uint_as_float((m & 0x80000000u) ? (m & 0x7fffffffu) : ~m);
}

__device__ inline float f16lo(uint32_t w) { return __half2float(__ushort_as_half((unsigned short)(w & 0xffffu))); }
__device__ inline float f16hi(uint32_t w) { return __half2float(__ushort_as_half((unsigned short)(w >> 16))); }
// a * (f16 in the low half of w), rounded once (v_fma_mix; the compiler otherwise converts
// and multiplies in two instructions).
__device__ inline float mul_f16lo(float a, uint32_t w) {
  float r;
  asm("v_fma_mix_f32 %0, %1, %2, 0 op_sel_hi:[0,1,0]" : "=v"(r) : "v"(a), "v"(w));
  return r;
}
__device__ inline float bf16f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// TC consecutive bf16 values of a tail row, read with one 2-, 4- or 8-byte load.
template <int TC>
struct TailRow {
  uint32_t w[(TC + 1) / 2];
  __device__ inline void load(const uint16_t* p) {
    if constexpr (TC == 1) w[0] = *p;
    else if constexpr (TC == 2) w[0] = *reinterpret_cast<const uint32_t*>(p);
    else {
      const uint2 v = *reinterpret_cast<const uint2*>(p);
      w[0] = v.x;
      w[1] = v.y;
    }
  }
  __device__ inline float f(int i) const {
    const uint32_t x = w[i / 2];
    return __uint_as_float(i % 2 ? (x & 0xffff0000u) : (x << 16));
  }
};
__device__ inline uint32_t w4(const uint4& v, int i) { return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w; }

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
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
__device__ inline uint4 ld_stream1(const void* p) {
  return make_uint4(__builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p)), 0u, 0u, 0u);
}
template <int N>
__device__ inline uint4 ld_words(const void* p) {
  return N == 4 ? ld_stream4(p) : N == 2 ? ld_stream2(p) : ld_stream1(p);
}

template <int N>
__device__ inline uint4 ld_words_lds(const float* p) {
  if constexpr (N == 4) {
    const float4 v = *reinterpret_cast<const float4*>(p);
    return make_uint4(__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z), __float_as_uint(v.w));
  } else if constexpr (N == 2) {
    const float2 v = *reinterpret_cast<const float2*>(p);
    return make_uint4(__float_as_uint(v.x), __float_as_uint(v.y), 0u, 0u);
  } else {
    return make_uint4(__float_as_uint(p[0]), 0u, 0u, 0u);
  }
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
// Signed 22-bit fixed point split into three signed byte digits: for |v| < 2^21 returns
// w = v + 0x8080 (two's complement), so v = (b0 - 128) + 256 (b1 - 128) + 65536 b2 with b2
// the signed top byte of w; bytes 0 and 1 become signed digits by flipping their top bit.
// The add of 1.5 * 2^23 rounds v to the nearest integer (ties to even) inside the fma and
// leaves it in the low mantissa bits.
__device__ inline uint32_t biased_fixed22(float c, float scl) {
  return __float_as_uint(fmaf(c, scl, 12582912.0f)) - (0x4B400000u - 0x8080u);
}
// Unsigned 16-bit fixed point of a >= 0 with scale scl (a * scl <= 65535.5), rounded to
// nearest inside the fma with 2^23 added: bytes 0 and 1 of the returned bit pattern are the
// value (the exponent bits above are never read).
__device__ inline uint32_t fixed16_lo(float a, float scl) {
  return __float_as_uint(fmaf(a, scl, 8388608.0f));
}

// BIG: the pool may exceed 4 GiB. Otherwise a record's byte offset fits 32 bits and a load
// takes the uniform pool base plus a 32-bit lane offset (the scalar-base form, no 64-bit
// address arithmetic); with BIG each lane forms a 64-bit address.
template <bool BIG>
struct RowT {
  const uint8_t* pool;     // pool base of the storage cell
  const uint32_t* boff;    // per logical block: record offset in 256-byte units (in LDS)
  const uint16_t* tail;    // tail of (slot, head): [2][32][D] bf16
  int N, n_q, n_groups;
  // Byte `off` of logical block j's record.
  __device__ inline const uint8_t* at(int j, uint32_t off) const {
    if constexpr (BIG) return pool + (((size_t)boff[j] << 8) + off);
    else return pool + ((boff[j] << 8) + off);
  }
  __device__ inline const uint8_t* rec_ptr(int j) const { return at(j, 0u); }
};

// Per-wave state of the online softmax. acc: this lane's V channels; accz: constant
// (zero-point / bucket-midpoint) terms of channel group lane % NE on the weight lanes;
// lsum: weights of the tokens this lane owns (tail tokens: lane 0); m: the reference.
template <int VCH>
struct Acc {
  float acc[VCH];
  float accz, lsum, m;
  __device__ inline void zero() {
#pragma unroll
    for (int c = 0; c < VCH; ++c) acc[c] = 0.f;
    accz = lsum = 0.f;
    m = -INFINITY;
  }
  // Move the reference up to mnew (wave-uniform, mnew > m); returns the factor applied.
  __device__ inline float raise(float mnew) {
    const float f = __expf(m - mnew);
#pragma unroll
    for (int c = 0; c < VCH; ++c) acc[c] *= f;
    accz *= f;
    lsum *= f;
    m = mnew;
    return f;
  }
};

// ----------------------------------------------------------------------------- step geometry
// A step covers TPS tokens: 64, or 32 for 4-bit codes at D = 128 and for D = 256, so that
// every lane reads 32 bytes of K codes and 32 bytes of V codes. WIDE: the streaming pass of
// 2-bit codes at D = 64 takes 128-token steps (four units), so a lane still reads 32 bytes of
// each and the per-step work that does not scale with D is spread over twice the tokens;
// the corrections, the exact pass and the merge keep the 64-token geometry (WIDE false).
template <int D, int MODE, int GS, bool WIDE = true>
struct Geo {
  static constexpr bool KIVI = MODE == MODE_KIVI;
  static constexpr bool DENSE = MODE == MODE_DENSE;
  static constexpr bool W128 = WIDE && D == 64 && !KIVI && !DENSE;
  static constexpr int TPS = W128 ? 128 : (D == 256 || ((KIVI || DENSE) && D == 128)) ? 32 : 64;
  static constexpr int GPS = TPS / kUnit;       // 32-token units per step
  static constexpr int GU = GS / kUnit;         // units per quantization group (1 or 2)
  static constexpr int GP = GS / kBlock;        // records per quantization group (2 or 4)
  static constexpr int BPS = TPS / kBlock;      // blocks per step
  // K: a group is covered by LPG lanes = 2 blocks x 4 token quads x CPG column lanes;
  // a column is one 32-bit word of UNIT channels, NC columns per lane.
  static constexpr int UNIT = KIVI ? 8 : 16;
  static constexpr int COLS = D / UNIT;
  static constexpr int LPG = 64 / GPS;
  static constexpr int CPG = LPG / 8;
  static constexpr int NC = COLS / CPG;
  static constexpr int CPL = GPS * D / 64;      // K-meta positions per lane
  static constexpr int SPC = KIVI ? 2 : 4;      // limb sets (4 channels each) per column
  static constexpr int KMETA = KIVI ? off_kmeta_kivi(D) : off_kmeta_planes(D);
  // V: LPB lanes per block, VCH channels per lane; weight lanes (block, bit pair, group).
  static constexpr int LPB = 64 / BPS;
  static constexpr int VCH = D / LPB;
  static constexpr int NE = D / kUnit;           // 32-channel V slices per token (GU share a meta word)
  static constexpr int COOP = BPS * 4 * NE;
  static constexpr int VW = KIVI ? 2 * VCH : VCH;   // code words per lane (high plane or KIVI-4)
  static constexpr int NV4 = VW / 4;
  static constexpr int NQ = KIVI ? D / 2 : D / 4;    // 16-byte quads of a V plane
  static constexpr int VR = vquad_r(KIVI, D);        // their stored transposition (layout.h)
  static_assert(KIVI ? NV4 == VR : (NV4 == 1 || NV4 == VR), "value lanes read whole transposed quads");
  static constexpr int VOFF = KIVI ? off_v_kivi(D, GS) : off_v_planes(D, GS);
  static constexpr int VMETA = KIVI ? off_vmeta_kivi(D, GS) : off_vmeta_planes(D, GS);
  // Token t_loc of a step is owned by lane t_loc and a weight lane's four tokens are its own
  // quad: the weights reach the weight lanes by quad broadcasts (D = 128, 2-bit codes).
  static constexpr bool QUAD_W = CPG == 4 && LPG == 32 && NE == 4;
  // per-wave scratch (words): K limbs at 0; step weights at 0 once the K limbs are
  // consumed; V limbs and their inverse scales from max(64, TPS).
  static constexpr int S_W = 0, S_VL = TPS > 64 ? TPS : 64, S_VI = S_VL + BPS * NE * 8;
  static_assert(NC >= 1 && VW % 4 == 0 && COOP <= 64, "geometry");
  static_assert(GPS * (D / 4) * 3 <= wave_scratch(D) && S_VI + BPS * NE <= wave_scratch(D) && TPS <= S_VL, "scratch");
};

// ----------------------------------------------------------------------------- K step
// Coefficients: the lanes of a group build the fixed-point coefficients of its D channels
// (CPL consecutive K-meta positions each; four consecutive positions form one limb set:
// the four channels a code word holds at one bit pair or nibble). They become 22-bit fixed
// point (scale 2^(21-e) from the group maximum) in three signed byte limbs; v_dot4_i32_i8
// multiplies four codes by four limbs and the limb sums recombine exactly in one register,
// ((l2 << 8) + l1) << 8 + l0. REFINE reads the low plane of a 4-bit cell with coefficients
// sigma q s and the constant -3/2 sigma q . s (from the bucket midpoint to lo).
template <int D, int MODE, bool REFINE, int GS>
struct KStep {
  using G = Geo<D, MODE, GS, !REFINE>;
  static constexpr int CODE_OFF = REFINE ? off_klo(D, GS) : 0;
  // Matrix-core path (2-bit codes, 64-token steps of two units): v_mfma_i32_16x16x64_i8 with
  // the codes as B (column j of tile T = token 4j + T of the step; lane group cg = one code
  // column of 16 channels, its four bit-pair words) and the coefficient limbs as A (rows
  // 0..2: limbs 0..2 of the step's first unit, rows 4..6: of its second, other rows zero).
  // Each token's three limb sums come out exact in 32-bit integers and combine exactly.
  // (also the corrections' low-plane refinement, REFINE: the same 2-bit geometry)
  static constexpr bool MF = !G::KIVI && !G::DENSE && G::TPS == 64 && G::GPS == 2 && (D == 64 || D == 128);
  static constexpr int NCH = D / 64;   // 64-channel chunks (MFMA depth)
  static_assert(!MF || NCH == G::NC, "one 16-byte code load per chunk");
  // The same on 128-token steps of four units (D = 64, one chunk): column j of tile T is
  // token 8j + T (a lane loads eight consecutive tokens of its column), A row 4u + r holds
  // limb r of unit u, and the valid outputs of column j are those of lane group j / 4.
  static constexpr bool MF128 = !REFINE && G::W128;
  static_assert(!MF128 || (G::GPS == 4 && G::COLS == 4 && G::NC == 2 && G::CPL == 4), "wide key geometry");
  // And on 32-token steps of one unit (D = 256, both planes at D = 128 and the KIVI-4 layout:
  // 4-bit codes, one byte each): column j of tile T is token 2j + T (a lane loads two
  // consecutive tokens of each of its columns), A rows 0..2 hold the unit's limbs, and lanes
  // 0..15 receive the 32 tokens' sums. A lane group covers 16 channels: one 2-bit column
  // (four bit-pair words) or two KIVI-4 columns (two nibble words each).
  static constexpr bool MF32 = G::TPS == 32 && (D == 256 || (D == 128 && (G::DENSE || G::KIVI)));
  static_assert(!MF32 || (G::GPS == 1 && G::COLS == 8 * G::NC && NCH == (G::KIVI ? 1 : 2) * G::NC), "32-token key geometry");

  struct Buf {
    uint4 meta, c[G::NC], l[G::DENSE ? G::NC : 1];
  };

  __device__ static inline void role(int lane, int& gsub, int& blk, int& quad, int& cp) {
    const int rl = lane % G::LPG;
    gsub = lane / G::LPG;
    blk = rl / (4 * G::CPG);
    quad = (rl / G::CPG) % 4;
    cp = rl % G::CPG;
  }

  // groups: the group read by each of the step's GPS slots (an empty slot repeats a valid
  // group of the step, so every load is in bounds and the kernel needs no per-lane branch).
  template <class RW>
  __device__ static inline void load(const RW& r, const int* groups, int lane, Buf& b) {
    int gsub, blk, quad, cp;
    role(lane, gsub, blk, quad, cp);
    const int g = groups[gsub];
    const int pos0 = (lane % G::LPG) * G::CPL;
    // K meta of the unit's group: its D / GP positions per record over the group's GP records
    if constexpr (G::GU == 1)
      b.meta = ld_words<G::CPL>(r.at(2 * g + (pos0 >= D / 2), G::KMETA + 4 * (pos0 % (D / 2))));
    else
      b.meta = ld_words<G::CPL>(r.at(G::GP * (g / G::GU) + pos0 / (D / G::GP), G::KMETA + 4 * (pos0 % (D / G::GP))));
    if constexpr (MF32 && G::KIVI) {
      // lane (token pair j, column group cg): tokens 2j, 2j + 1 of columns 8C + 2cg and
      // 8C + 2cg + 1 (record j / 8); b.c[C] = {first column: t, t + 1; second: t, t + 1}
      const int j = lane % 16, cg = lane / 16;
      const uint8_t* kq = r.at(2 * groups[0] + j / 8, CODE_OFF + (2 * cg * kBlock + 2 * (j % 8)) * 4);
#pragma unroll
      for (int c = 0; c < G::NC; ++c) {
        const uint4 a0 = ld_stream2(kq + 8 * c * kBlock * 4), a1 = ld_stream2(kq + (8 * c + 1) * kBlock * 4);
        b.c[c] = make_uint4(a0.x, a0.y, a1.x, a1.y);
      }
      return;
    }
    if constexpr (MF32) {
      // lane (token pair j, column group cg): tokens 2j, 2j + 1 of columns 4C + cg (record
      // j / 8); per chunk the 16 lanes of a record cover its four columns (256 bytes)
      const int j = lane % 16, cg = lane / 16;
      const uint8_t* kq = r.at(2 * groups[0] + j / 8, CODE_OFF + (cg * kBlock + 2 * (j % 8)) * 4);
#pragma unroll
      for (int c = 0; c < G::NC; ++c) {   // chunk 2c: words 0, 1; chunk 2c + 1: words 2, 3
        const uint4 a0 = ld_stream2(kq + (2 * c) * 4 * kBlock * 4), a1 = ld_stream2(kq + (2 * c + 1) * 4 * kBlock * 4);
        b.c[c] = make_uint4(a0.x, a0.y, a1.x, a1.y);
        if constexpr (G::DENSE) {
          const uint4 b0 = ld_stream2(kq + off_klo(D, GS) + (2 * c) * 4 * kBlock * 4);
          const uint4 b1 = ld_stream2(kq + off_klo(D, GS) + (2 * c + 1) * 4 * kBlock * 4);
          b.l[c] = make_uint4(b0.x, b0.y, b1.x, b1.y);
        }
      }
      return;
    }
    if constexpr (MF128) {
      // lane (token octet j, column cg): tokens 8j .. 8j + 7 of column cg (unit j / 4); the
      // eight lanes of two octets cover the record's four columns (256 contiguous bytes)
      const int j = lane % 16, cg = lane / 16;
      const uint8_t* kq = r.at(2 * groups[j / 4] + (j % 4) / 2, CODE_OFF + (cg * kBlock + 8 * (j % 2)) * 4);
      b.c[0] = ld_stream4(kq);
      b.c[1] = ld_stream4(kq + 16);
      return;
    }
    if constexpr (MF) {
      // lane (token quad j, column group cg): tokens 4j .. 4j + 3 of column 4C + cg; the 16
      // lanes of a quad-of-quads cover four whole consecutive columns of a record
      const int j = lane % 16, cg = lane / 16;
      const uint8_t* kq = r.at(2 * groups[j / 8] + (j % 8) / 4, CODE_OFF + (cg * kBlock + 4 * (j % 4)) * 4);
#pragma unroll
      for (int i = 0; i < NCH; ++i) b.c[i] = ld_stream4(kq + i * 4 * kBlock * 4);
      return;
    }
    // lane cp reads columns cp, cp + CPG, ...: each load instruction covers CPG whole
    // consecutive columns (CPG x 64 contiguous bytes) of each of its records
    const uint8_t* kp = r.at(2 * g + blk, CODE_OFF + (cp * kBlock + 4 * quad) * 4);
#pragma unroll
    for (int i = 0; i < G::NC; ++i) b.c[i] = ld_stream4(kp + i * G::CPG * kBlock * 4);
    if (G::DENSE) {
#pragma unroll
      for (int i = 0; i < G::NC; ++i) b.l[i] = ld_stream4(kp + off_klo(D, GS) + i * G::CPG * kBlock * 4);
    }
  }

  // sigma q in K-meta position order (2-bit: position 16w + 4p + k holds channel 16w + 4k + p;
  // 4-bit: 8w + 4n + k holds 8w + 2k + n), written once per row so that a lane reads the q
  // of its positions with one LDS load per step instead of holding them in registers.
  __device__ static inline void fill_qperm(const float* qs, float* qperm) {
    for (int pos = threadIdx.x; pos < D; pos += kThreads) {
      const int ch = G::KIVI ? 8 * (pos / 8) + 2 * (pos % 4) + (pos / 4) % 2
                             : 16 * (pos / 16) + 4 * (pos % 4) + (pos / 4) % 4;
      qperm[pos] = qs[ch];
    }
  }

  // Masked words of one code word (and its low-plane word for DENSE): the four codes of
  // one limb set each, one code per byte. 2-bit planes: bit pairs 1 and 3 are taken in place
  // (4 c, no shift) and their coefficients stay at scale 1 while those of pairs 0 and 2 are
  // made 4x, so every product carries the same factor 4 (five operations per word).
  __device__ static inline void masked(uint32_t x, uint32_t y, uint32_t* m) {
    if constexpr (G::KIVI) {
      m[0] = x & 0x0F0F0F0Fu;
      m[1] = (x >> 4) & 0x0F0F0F0Fu;
    } else if constexpr (!G::DENSE) {
      const uint32_t x4 = x >> 4;
      m[0] = x & 0x03030303u;
      m[1] = x & 0x0C0C0C0Cu;
      m[2] = x4 & 0x03030303u;
      m[3] = x4 & 0x0C0C0C0Cu;
    } else {
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        m[p] = (x >> (2 * p)) & 0x03030303u;
        if (G::DENSE) m[p] = (m[p] << 2) | ((y >> (2 * p)) & 0x03030303u);
      }
    }
  }

  // The step's scores. Every token t_loc of the step has one owner lane (own), which
  // receives sigma q . k_t (REFINE: the correction to it).
  // MF128: every lane owns two tokens, t_loc and t_loc + 64 (the second score in *second).
  __device__ static inline float compute(const float* qperm, uint32_t* klimb, int lane, const Buf& b, bool& own,
                                         int& t_loc, float* second = nullptr) {
    int gsub, blk, quad, cp;
    role(lane, gsub, blk, quad, cp);
    const int pos0 = (lane % G::LPG) * G::CPL;
    float qreg[G::CPL];
    {
      const uint4 qv = ld_words_lds<G::CPL>(qperm + pos0);
#pragma unroll
      for (int k = 0; k < G::CPL; ++k) qreg[k] = __uint_as_float(w4(qv, k));
    }
    float f[G::CPL];
    float cst = 0.f;
#pragma unroll
    for (int k = 0; k < G::CPL; ++k) {
      const uint32_t mw = w4(b.meta, k);
      f[k] = mul_f16lo(qreg[k], mw);                       // sigma q s
      if (REFINE) {
        cst = fmaf(-1.5f, f[k], cst);                     // sigma q s (lo - 3/2)
      } else if (MODE == MODE_COARSE) {
        cst = fmaf(qreg[k], f16hi(mw), cst);              // sigma q (z + s (4 hi + 3/2))
        cst = fmaf(1.5f, f[k], cst);
      } else {
        cst = fmaf(qreg[k], f16hi(mw), cst);              // sigma q (z + s c)
      }
    }
    float fm = fabsf(f[0]);
#pragma unroll
    for (int k = 1; k < G::CPL; ++k) fm = fmaxf(fm, fabsf(f[k]));
    // group max of |f| and group sum of the constant, interleaved
    {
      uint32_t v = __float_as_uint(fm);
      v = max(v, dpp_u<0xB1>(v));
      cst += dpp<0xB1>(cst);
      v = max(v, dpp_u<0x4E>(v));
      cst += dpp<0x4E>(cst);
      v = max(v, dpp_u<0x141>(v));
      cst += dpp<0x141>(cst);
      v = max(v, dpp_u<0x140>(v));
      cst += dpp<0x140>(cst);
      if (G::LPG >= 32) {
        v = max_rows2(v);
        cst = add_rows2(cst);
      }
      if (G::LPG == 64) {
        v = max_halves(v);
        cst = add_halves(cst);
      }
      fm = __uint_as_float(v);
    }
    static_assert(G::LPG >= (MF128 ? 16 : 32), "group lanes");
    const int ex = set_exponent(fm);
    // 2-bit planes (see masked): positions of bit pairs 0 and 2 get 4x coefficients (below
    // 2^22), those of pairs 1 and 3 scale 1 (below 2^20), every product then holds 4 v c;
    // a lane's positions share one bit pair. Other layouts: below 2^21, factor 1.
    constexpr bool X4 = !G::KIVI && !G::DENSE;
    const bool even_pair = ((pos0 % 16) / 4) % 2 == 0;
    const float scl = __builtin_amdgcn_ldexpf(X4 && even_pair ? 4.f : 1.f, (X4 ? 20 : 21) - ex);
    // high-plane-only codes carry weight 4 (code 4 hi): folded into the inverse scale
    const float inv = __builtin_amdgcn_ldexpf(MODE == MODE_COARSE && !REFINE ? 4.f : 1.f, ex - (X4 ? 22 : 21));
    uint32_t mine[G::CPL];
#pragma unroll
    for (int k = 0; k < G::CPL; ++k) mine[k] = biased_fixed22(f[k], scl);
    // the four values of this lane's limb set (held by 4 / CPL consecutive lanes)
    uint32_t u[4];
    if constexpr (G::CPL == 4) {
#pragma unroll
      for (int k = 0; k < 4; ++k) u[k] = mine[k];
    } else if constexpr (G::CPL == 2) {
      const uint32_t o0 = dpp_u<0xB1>(mine[0]), o1 = dpp_u<0xB1>(mine[1]);
      const bool odd = lane & 1;
      u[0] = odd ? o0 : mine[0];
      u[1] = odd ? o1 : mine[1];
      u[2] = odd ? mine[0] : o0;
      u[3] = odd ? mine[1] : o1;
    } else {
      u[0] = dpp_u<0x00>(mine[0]);   // quad_perm [0,0,0,0]
      u[1] = dpp_u<0x55>(mine[0]);   // quad_perm [1,1,1,1]
      u[2] = dpp_u<0xAA>(mine[0]);
      u[3] = dpp_u<0xFF>(mine[0]);
    }
    if ((lane % (4 / G::CPL)) == 0) {
      uint32_t limb[3];
      transpose3(u, limb);
      if constexpr (MF || MF128 || MF32) {
        // [unit][column][limb][bit pair or nibble]: an A row reads its column's limb words at once
        const int st = pos0 / 4;   // limb set: column st / SPC, bit pair (or nibble) st % SPC
        uint32_t* dst = klimb + (gsub * G::COLS + st / G::SPC) * (3 * G::SPC) + st % G::SPC;
        dst[0] = limb[0] ^ 0x80808080u;   // biased byte -> signed digit
        dst[G::SPC] = limb[1] ^ 0x80808080u;
        dst[2 * G::SPC] = limb[2];
      } else {
        uint32_t* dst = klimb + (gsub * (D / 4) + pos0 / 4) * 3;
#pragma unroll
        for (int j = 0; j < 2; ++j) dst[j] = limb[j] ^ 0x80808080u;   // biased byte -> signed digit
        dst[2] = limb[2];
      }
    }
    wave_sync_lds();
    if constexpr (MF32) {
      const int m = lane % 16, cg = lane / 16;
      i32x4_t acc[2] = {i32x4_t{0, 0, 0, 0}, i32x4_t{0, 0, 0, 0}};
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        i32x4_t A;
        if constexpr (G::KIVI) {   // columns 8c + 2cg and 8c + 2cg + 1: two nibble words each
          const uint2 t0 = *reinterpret_cast<const uint2*>(klimb + (8 * c + 2 * cg) * 6 + (m < 3 ? m : 0) * 2);
          const uint2 t1 = *reinterpret_cast<const uint2*>(klimb + (8 * c + 2 * cg + 1) * 6 + (m < 3 ? m : 0) * 2);
          A = m < 3 ? i32x4_t{(int)t0.x, (int)t0.y, (int)t1.x, (int)t1.y} : i32x4_t{0, 0, 0, 0};
        } else {
          const uint4 t = *reinterpret_cast<const uint4*>(klimb + (4 * c + cg) * 12 + (m < 3 ? m : 0) * 4);
          A = m < 3 ? i32x4_t{(int)t.x, (int)t.y, (int)t.z, (int)t.w} : i32x4_t{0, 0, 0, 0};
        }
#pragma unroll
        for (int T = 0; T < 2; ++T) {
          uint32_t mw[4];
          if constexpr (G::KIVI) {
            masked(w4(b.c[c], T), 0u, mw);
            masked(w4(b.c[c], 2 + T), 0u, mw + 2);
          } else {
            masked(w4(b.c[c / 2], 2 * (c % 2) + T), G::DENSE ? w4(b.l[c / 2], 2 * (c % 2) + T) : 0u, mw);
          }
          const i32x4_t bv = {(int)mw[0], (int)mw[1], (int)mw[2], (int)mw[3]};
          acc[T] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, bv, acc[T], 0, 0, 0);
        }
      }
      wave_sync_lds();   // every lane's A words are read before the scores reuse them
      float* tr = reinterpret_cast<float*>(klimb);
      if (lane < 16) {
        float2 sc;
        const uint32_t v0 = (uint32_t)acc[0][0] + ((uint32_t)acc[0][1] << 8) + ((uint32_t)acc[0][2] << 16);
        const uint32_t v1 = (uint32_t)acc[1][0] + ((uint32_t)acc[1][1] << 8) + ((uint32_t)acc[1][2] << 16);
        sc.x = fmaf(inv, (float)(int)v0, cst);
        sc.y = fmaf(inv, (float)(int)v1, cst);
        *reinterpret_cast<float2*>(tr + 2 * lane) = sc;
      }
      wave_sync_lds();
      own = lane < 32;
      t_loc = lane % 32;
      return tr[lane % 32];
    }
    if constexpr (MF128) {
      const int m = lane % 16, cg = lane / 16;
      const uint4 t = *reinterpret_cast<const uint4*>(klimb + ((m / 4) * G::COLS + cg) * 12 + (m & 3) % 3 * 4);
      const i32x4_t A = (m & 3) < 3 ? i32x4_t{(int)t.x, (int)t.y, (int)t.z, (int)t.w} : i32x4_t{0, 0, 0, 0};
      wave_sync_lds();   // every lane's A words are read before the scores reuse them
      float* tr = reinterpret_cast<float*>(klimb);
      const int j = lane % 16;
      const bool mine = j / 4 == cg;   // lane group q holds rows 4q .. 4q + 3: unit q's limbs,
                                       // whose scale and constant this lane built
#pragma unroll
      for (int T = 0; T < 8; ++T) {
        uint32_t mw[4];
        masked(w4(b.c[T / 4], T % 4), 0u, mw);
        const i32x4_t bv = {(int)mw[0], (int)mw[1], (int)mw[2], (int)mw[3]};
        const i32x4_t acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, bv, i32x4_t{0, 0, 0, 0}, 0, 0, 0);
        const uint32_t v = (uint32_t)acc[0] + ((uint32_t)acc[1] << 8) + ((uint32_t)acc[2] << 16);
        if (mine) tr[8 * j + T] = fmaf(inv, (float)(int)v, cst);
      }
      wave_sync_lds();
      own = true;
      t_loc = lane;
      *second = tr[64 + lane];
      return tr[lane];
    }
    if constexpr (MF) {
      const int m = lane % 16, cg = lane / 16;
      const bool arow = m < 8 && (m & 3) < 3;
      i32x4_t A[NCH];
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const uint4 t = *reinterpret_cast<const uint4*>(klimb + ((m / 4) % 2 * G::COLS + 4 * c + cg) * 12 + (m & 3) % 3 * 4);
        A[c] = arow ? i32x4_t{(int)t.x, (int)t.y, (int)t.z, (int)t.w} : i32x4_t{0, 0, 0, 0};
      }
      // the two units' inverse scales and constants (uniform over each unit's 32 lanes)
      const float inv0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(inv), 0));
      const float inv1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(inv), 32));
      const float cst0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cst), 0));
      const float cst1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cst), 32));
      float sc[4];
#pragma unroll
      for (int T = 0; T < 4; ++T) {
        i32x4_t acc = {0, 0, 0, 0};
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
          uint32_t mw[4];
          masked(w4(b.c[c], T), 0u, mw);
          const i32x4_t bv = {(int)mw[0], (int)mw[1], (int)mw[2], (int)mw[3]};
          acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[c], bv, acc, 0, 0, 0);
        }
        // lanes 0..7: rows 0..3 (unit 0) of columns 0..7; lanes 24..31: rows 4..7 (unit 1)
        // of columns 8..15; the limb sums recombine exactly (mod 2^32, the true sum fits)
        const uint32_t v = (uint32_t)acc[0] + ((uint32_t)acc[1] << 8) + ((uint32_t)acc[2] << 16);
        sc[T] = fmaf(lane >= 16 ? inv1 : inv0, (float)(int)v, lane >= 16 ? cst1 : cst0);
      }
      // to one token per lane: token 4j + T of column j sits in lane j (j < 8) or 16 + j
      wave_sync_lds();   // every lane's A words are read before the scores reuse them
      float* tr = reinterpret_cast<float*>(klimb);
      if (lane < 8 || (lane >= 24 && lane < 32))
        *reinterpret_cast<float4*>(tr + 4 * (lane % 16)) = make_float4(sc[0], sc[1], sc[2], sc[3]);
      wave_sync_lds();
      own = true;
      t_loc = lane;
      return tr[lane];
    }
    // Limbs of this lane's NC columns (SPC sets x 3 words each); the four tokens' chains run
    // interleaved, limb 2 first, one column at a time, each recombined exactly.
    constexpr int NCC = 1;   // columns per chain
    constexpr int CW = NCC * G::SPC * 3;
    int acc4[4] = {0, 0, 0, 0};
#pragma unroll
    for (int i0 = 0; i0 < G::NC; i0 += NCC) {
      uint32_t L[CW];
      const uint32_t* src = klimb + (gsub * (D / 4) + (cp + i0 * G::CPG) * G::SPC) * 3;   // column cp + i0 CPG
      if constexpr (CW % 4 == 0) {
#pragma unroll
        for (int u4 = 0; u4 < CW / 4; ++u4) {
          const uint4 t = reinterpret_cast<const uint4*>(src)[u4];
          L[4 * u4] = t.x;
          L[4 * u4 + 1] = t.y;
          L[4 * u4 + 2] = t.z;
          L[4 * u4 + 3] = t.w;
        }
      } else {
#pragma unroll
        for (int u2 = 0; u2 < CW / 2; ++u2) {
          const uint2 t = reinterpret_cast<const uint2*>(src)[u2];
          L[2 * u2] = t.x;
          L[2 * u2 + 1] = t.y;
        }
      }
      uint32_t m[4][NCC][G::SPC];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int i = 0; i < NCC; ++i)
          masked(w4(b.c[i0 + i], tt), G::DENSE ? w4(b.l[i0 + i], tt) : 0u, m[tt][i]);
      int a[4] = {0, 0, 0, 0};
#pragma unroll
      for (int j = 2; j >= 0; --j) {
        if (j < 2) {
#pragma unroll
          for (int tt = 0; tt < 4; ++tt) a[tt] <<= 8;
        }
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
          for (int i = 0; i < NCC; ++i)
#pragma unroll
            for (int s = 0; s < G::SPC; ++s) a[tt] = sdot4(L[(i * G::SPC + s) * 3 + j], m[tt][i][s], a[tt]);
      }
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) acc4[tt] = i0 == 0 ? a[tt] : acc4[tt] + a[tt];
    }
    float part[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) part[tt] = (float)acc4[tt];
    // Reduce-scatter over the CPG column lanes of a token quad (consecutive lanes): the lane
    // with in-quad index q ends with token q (CPG = 8: pairs i, 7 - i first; lanes 0..3 own).
    if (G::CPG == 8) {
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) part[tt] += dpp<0x141>(part[tt]);   // row_half_mirror
    }
    const bool odd = cp & 1, hi = cp & 2;
    float k0 = odd ? part[1] : part[0], k1 = odd ? part[3] : part[2];
    const float s0 = odd ? part[0] : part[1], s1 = odd ? part[2] : part[3];
    k0 += dpp<0xB1>(s0);   // quad_perm [1,0,3,2]
    k1 += dpp<0xB1>(s1);
    const float keep = hi ? k1 : k0, send = hi ? k0 : k1;
    const float sum = keep + dpp<0x4E>(send);   // quad_perm [2,3,0,1]
    own = G::CPG == 4 || cp < 4;
    t_loc = gsub * kUnit + blk * kBlock + quad * 4 + (cp & 3);
    return fmaf(inv, sum, cst);
  }
};

// ----------------------------------------------------------------------------- V step
// Weight lanes (block jbm, bit pair p, channel group e) fold weight and scale of the four
// tokens 4p..4p+3 of their block and group into 16-bit fixed point (scale from the max over
// the block and group) in two unsigned byte limbs; value lanes (block, chunk of VCH
// channels) multiply them with four tokens' codes of a channel with v_dot4_u32_u8 and
// scale each block's exact integer sum into the fp32 accumulator. Constant terms (w z, plus
// w s 3/2 for a high-plane-only read) go to accz on the weight lanes.
template <int D, int MODE, int GS>
struct VStep {
  using G = Geo<D, MODE, GS>;

  struct Buf {
    uint4 meta, c[G::NV4], l[G::DENSE ? G::NV4 : 1];
  };

  // Blocks past the row's end repeat the step's first block (in bounds; their weights are 0).
  template <class RW>
  __device__ static inline void load(const RW& r, int jbase, int nb, int lane, Buf& b) {
    int jm = jbase + lane / (4 * G::NE);
    const int p = (lane / G::NE) % 4, e = lane % G::NE;
    jm = jm < nb ? jm : jbase;
    if (lane < G::COOP) b.meta = ld_stream4(r.at(jm, G::VMETA + 4 * ((e / G::GU) * kBlock + 4 * p)));
    int j = jbase + lane / G::LPB;
    j = j < nb ? j : jbase;
    const int chunk = lane % G::LPB;
    // the lane's NV4 logical quads chunk NV4 + i, stored transposed (see vquad_pos)
#pragma unroll
    for (int i = 0; i < G::NV4; ++i) b.c[i] = ld_stream4(r.at(j, G::VOFF + 16 * vquad_pos(chunk * G::NV4 + i, G::NQ, G::VR)));
    if (G::DENSE) {
#pragma unroll
      for (int i = 0; i < G::NV4; ++i)
        b.l[i] = ld_stream4(r.at(j, off_vlo(D, GS) + 16 * vquad_pos(chunk * G::NV4 + i, G::NQ, G::VR)));
    }
  }

  // wgt: this lane's own token weight (QUAD_W) or the step's weights in LDS (wts).
  template <class A>
  __device__ static inline void compute(float wgt, const float* wts, float* scratch, int lane, const Buf& b, A& st) {
    const int jbm = lane / (4 * G::NE), p = (lane / G::NE) % 4, e = lane % G::NE;
    uint32_t* vlimb = reinterpret_cast<uint32_t*>(scratch + G::S_VL);   // [BPS][NE][4 p][2]
    float* vinv = scratch + G::S_VI;                                     // [BPS][NE]
    float a[4] = {0.f, 0.f, 0.f, 0.f};
    const bool coop = lane < G::COOP;
    if (coop) {
      float wv[4];
      if constexpr (G::QUAD_W) {
        wv[0] = dpp<0x00>(wgt);   // quad_perm [0,0,0,0]
        wv[1] = dpp<0x55>(wgt);
        wv[2] = dpp<0xAA>(wgt);
        wv[3] = dpp<0xFF>(wgt);
      } else {
        const float4 w4v = *reinterpret_cast<const float4*>(wts + jbm * kBlock + 4 * p);
        wv[0] = w4v.x;
        wv[1] = w4v.y;
        wv[2] = w4v.z;
        wv[3] = w4v.w;
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t mw = w4(b.meta, k);
        a[k] = mul_f16lo(wv[k], mw);
        st.accz = fmaf(wv[k], f16hi(mw), st.accz);
        if (MODE == MODE_COARSE) st.accz = fmaf(1.5f, a[k], st.accz);   // bucket midpoint
      }
    }
    float am;
    {   // max over the 4 tokens and the 4 bit-pair lanes of (block, group) (non-negative:
        // unsigned compare of the bit patterns)
      uint32_t v = max(max(__float_as_uint(a[0]), __float_as_uint(a[1])), max(__float_as_uint(a[2]), __float_as_uint(a[3])));
      if (G::NE == 4) {   // lanes e + 4p of a 16-lane row
        v = max(v, dpp_u<0x124>(v));   // row_ror:4
        v = max(v, dpp_u<0x128>(v));   // row_ror:8
      } else {
        v = max(v, (uint32_t)__shfl_xor((int)v, G::NE));
        v = max(v, (uint32_t)__shfl_xor((int)v, 2 * G::NE));
      }
      am = __uint_as_float(v);
    }
    // scale 2^(16-e) (1 - 2^-17) keeps the rounded value <= 65535
    const int ex = set_exponent(am);
    const float scl = __builtin_amdgcn_ldexpf(1.f - 0x1p-17f, 16 - ex);
    if (coop) {
      uint32_t qb[4], limb[2];
#pragma unroll
      for (int k = 0; k < 4; ++k) qb[k] = fixed16_lo(a[k], scl);
      transpose2(qb, limb);
      uint32_t* dst = vlimb + ((jbm * G::NE + e) * 4 + p) * 2;
      dst[0] = limb[0];
      dst[1] = limb[1];
      if (p == 0) vinv[jbm * G::NE + e] = __builtin_amdgcn_ldexpf(1.f + 0x1p-17f, ex - 16);   // 1 / scl
    }
    wave_sync_lds();
    const int jb = lane / G::LPB, chunk = lane % G::LPB;
    const int e_lane = chunk * G::VCH / kUnit;
    uint32_t L[8];
    const uint4* lp = reinterpret_cast<const uint4*>(vlimb + (jb * G::NE + e_lane) * 8);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const uint4 t = lp[u];
      L[4 * u] = t.x;
      L[4 * u + 1] = t.y;
      L[4 * u + 2] = t.z;
      L[4 * u + 3] = t.w;
    }
    const float binv = vinv[jb * G::NE + e_lane];
    const float cscale = MODE == MODE_COARSE ? 4.f * binv : binv;   // high plane only: code 4 hi
    // two channels at a time, their chains interleaved
#pragma unroll
    for (int c = 0; c < G::VCH; c += 2) {
      uint32_t m[2][4];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        if constexpr (G::KIVI) {   // word (d, j): token 8j + 4n + k at nibble n of byte k
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            const int wi = 2 * (c + i) + jj;
            const uint32_t x = w4(b.c[wi / 4], wi % 4);
            m[i][2 * jj] = x & 0x0F0F0F0Fu;
            m[i][2 * jj + 1] = (x >> 4) & 0x0F0F0F0Fu;
          }
        } else {   // word d: token 4p + k at bits 8k + 2p
          const uint32_t x = w4(b.c[(c + i) / 4], (c + i) % 4);
#pragma unroll
          for (int pp = 0; pp < 4; ++pp) {
            m[i][pp] = (x >> (2 * pp)) & 0x03030303u;
            if (G::DENSE) m[i][pp] = (m[i][pp] << 2) | ((w4(b.l[(c + i) / 4], (c + i) % 4) >> (2 * pp)) & 0x03030303u);
          }
        }
      }
      uint32_t s0 = 0, s1 = 0;
#pragma unroll
      for (int pp = 0; pp < 4; ++pp) {
        s0 = udot4(L[2 * pp + 1], m[0][pp], s0);
        s1 = udot4(L[2 * pp + 1], m[1][pp], s1);
      }
      s0 <<= 8;
      s1 <<= 8;
#pragma unroll
      for (int pp = 0; pp < 4; ++pp) {
        s0 = udot4(L[2 * pp], m[0][pp], s0);
        s1 = udot4(L[2 * pp], m[1][pp], s1);
      }
      st.acc[c] = fmaf(cscale, (float)s0, st.acc[c]);
      st.acc[c + 1] = fmaf(cscale, (float)s1, st.acc[c + 1]);
    }
  }
};

// ----------------------------------------------------------------------------- exact V pass
// Recomputes a 4-bit row's V sum from final weights held in LDS (selected tokens at 4
// bits, the rest at the bucket midpoint) in the value-lane layout of the coarse step
// (4 blocks per 64 lanes, D/16 channels per lane), constants included. Runs only when a
// correction would cancel most of the row's weight.
template <int D, int GS, class RW>
__device__ void exact_v_pass(const RW& r, const float* weights, const uint32_t* selm, int lane, int w,
                             float* acc) {
  using GC = Geo<D, MODE_COARSE, GS, false>;
  constexpr int VCH = GC::VCH;
  const int nb = r.n_q / kBlock;
  const int jb = lane / GC::LPB, chunk = lane % GC::LPB, e = chunk * VCH / kUnit / GC::GU;   // meta group
  for (int j = w * GC::BPS + jb; j < nb; j += GC::BPS * kWaves) {
    const uint8_t* rb = r.rec_ptr(j);
    uint32_t hw[VCH], lw[VCH];
#pragma unroll
    for (int c = 0; c < VCH; ++c) {
      const int wp = vword_pos(chunk * VCH + c, false, D);
      hw[c] = reinterpret_cast<const uint32_t*>(rb + off_v_planes(D, GS))[wp];
      lw[c] = reinterpret_cast<const uint32_t*>(rb + off_vlo(D, GS))[wp];
    }
    const uint32_t bm = (selm[j >> 1] >> (16 * (j & 1))) & 0xffffu;
    for (int tt = 0; tt < kBlock; ++tt) {
      const float wt = weights[j * kBlock + tt];
      const uint32_t mw = reinterpret_cast<const uint32_t*>(rb + off_vmeta_planes(D, GS))[e * kBlock + tt];
      const float s = f16lo(mw), z = f16hi(mw);
      const bool sel = (bm >> tt) & 1u;
      const int sh = 8 * (tt % 4) + 2 * (tt / 4);
#pragma unroll
      for (int c = 0; c < VCH; ++c) {
        const float code = 4.f * (float)((hw[c] >> sh) & 3u) + (sel ? (float)((lw[c] >> sh) & 3u) : 1.5f);
        acc[c] = fmaf(wt, fmaf(s, code, z), acc[c]);
      }
    }
  }
}

// Bit m of an 8-bit value to bit 4m (m = 0..7).
__device__ inline uint32_t spread4(uint32_t x) {
  x = (x | (x << 12)) & 0x000F000Fu;
  x = (x | (x << 6)) & 0x03030303u;
  return (x | (x << 3)) & 0x11111111u;
}

// ----------------------------------------------------------------------------- LDS sizes
__host__ __device__ inline size_t pad4(size_t n) { return (n + 3) / 4 * 4; }   // keep 16-byte alignment
__host__ __device__ inline size_t lds_lpad(int max_len) { return ((size_t)max_len + 63) / 64 * 64; }
__host__ __device__ inline size_t lds_region_a(int max_len, int D) {
  const size_t need = (size_t)kWaves * D;   // the merge's wave vectors
  const size_t lp = lds_lpad(max_len);
  return pad4(lp > need ? lp : need);
}
__host__ __device__ inline size_t decode_lds_floats(int max_len, int D) {
  const size_t lp = lds_lpad(max_len);
  return lds_region_a(max_len, D) + pad4(lp / 32) + pad4(lp / 16 + 16) + 2 * D + (size_t)kWaves * wave_scratch(D) + 96;
}
// A finishing launch also stages the row's n_split partial value vectors in LDS, right after
// the row's regions (the exchange words are last), when they fit in the 160 KB.
__host__ __device__ inline bool finish_parts_in_lds(int max_len, int D, int n_split) {
  return decode_lds_floats(max_len, D) + (size_t)n_split * D <= (size_t)160 * 1024 / 4;
}
__host__ __device__ inline size_t finish_lds_floats(int max_len, int D, int n_split) {
  return decode_lds_floats(max_len, D) + (finish_parts_in_lds(max_len, D, n_split) ? (size_t)n_split * D : 0);
}

struct Smem {
  float* scores;    // [lpad]; at the end: [kWaves][D] the waves' value vectors
  uint32_t* selm;   // [lpad / 32]
  uint32_t* boff;   // [lpad / 16] record offset of each logical block, 256-byte units
  float* qs;        // [D]
  float* qperm;     // [D] sigma q in K-meta position order
  float* wscr;      // [kWaves][wave_scratch(D)]
  float* misc;      // [96]: per wave m, l, removed weight (0..23); the partials' factors (32..95)
};

// ----------------------------------------------------------------------------- row body
// Phases: PH_ROW runs a whole row in one workgroup. A split decode runs PH_PART on each of
// n_split workgroups of a row (a range of its chunks; the last one also takes the tail) and
// writes a partial (m, l, o) plus, when the row selects, its coarse scores; PH_FINISH then
// merges the partials of the row, selects, corrects the selected tokens and writes the row.
enum : int { PH_ROW = 0, PH_PART = 1, PH_FINISH = 2 };

// Chunk range [cb, ce) of split `split` over a row of n_chunks chunks: equal shares rounded
// up to a multiple of the waves of a workgroup, so every wave gets the same step count, taken
// from the row's end: the last split always holds the last chunks (with the tail), so in a
// serving step the workgroup that appends the step's token is the only one reading the group
// that token completes; splits left without chunks are the first ones.
__device__ inline void split_range(int n_chunks, int n_split, int split, int& cb, int& ce) {
  const int per = ((n_chunks + n_split - 1) / n_split + kWaves - 1) / kWaves * kWaves;
  ce = max(0, n_chunks - (n_split - 1 - split) * per);
  cb = max(0, ce - per);
}

// The in-launch append of a serving step (DecodeArgs::app_k): the token of (sequence b, KV
// head kh) at position L0 = app_lens[b]. It stays in the tail (slot L0 mod GS) unless it
// completes group g = L0 / GS; then the group's GS tokens (GS - 1 from the tail, the new one)
// are quantized and its GS / 16 records written through the block table, exactly as the
// append kernels do (same quantizer, same packer). Unmapped pages and invalid sequences are
// skipped as there. The caller synchronizes the workgroup afterwards.
template <int D, int GS>
__device__ void fused_append(const DecodeArgs& a, const DecodeCell& cell, int b, int kh, unsigned char* lds) {
  const int tid = threadIdx.x;
  const int L0 = a.app_lens[b];
  const int slot = a.seq_slots ? a.seq_slots[b] : b;
  if (L0 < 0 || (uint32_t)slot >= (uint32_t)a.max_seqs) return;   // uniform: nothing written
  uint16_t* tail = reinterpret_cast<uint16_t*>(const_cast<uint8_t*>(a.ws) + cell.tail_off) +
                   ((size_t)slot * a.n_kv_heads + kh) * tail_elems(D, GS);
  const size_t e0 = ((size_t)b * a.n_kv_heads + kh) * D;
  auto new_bits = [&](const void* src, int d) -> uint16_t {
    return a.app_bf16 ? reinterpret_cast<const uint16_t*>(src)[e0 + d]
                      : f32_to_bf16_rne(reinterpret_cast<const float*>(src)[e0 + d]);
  };
  const int pos = L0 % GS;
  if (pos != GS - 1) {   // the token stays in the tail
    for (int d = tid; d < D; d += kThreads) {
      tail[(size_t)pos * D + d] = new_bits(a.app_k, d);
      tail[(size_t)(GS + pos) * D + d] = new_bits(a.app_v, d);
    }
    return;
  }
  auto kx = reinterpret_cast<uint16_t(*)[D]>(lds);                        // [GS][D]
  auto vx = reinterpret_cast<uint16_t(*)[D]>(lds + 2 * GS * D);
  auto kc = reinterpret_cast<uint8_t(*)[D]>(lds + 4 * GS * D);
  auto vc = reinterpret_cast<uint8_t(*)[D]>(lds + 5 * GS * D);
  uint32_t* kmeta = reinterpret_cast<uint32_t*>(lds + 6 * GS * D);
  auto vmeta = reinterpret_cast<uint32_t(*)[D / GS]>(lds + 6 * GS * D + 4 * D);
  for (int idx = tid; idx < GS * D; idx += kThreads) {
    const int i = idx / D, d = idx % D;
    const bool old = i < GS - 1;   // positions g GS .. L0 - 1 sit in tail slots 0 .. GS - 2
    kx[i][d] = old ? tail[(size_t)i * D + d] : new_bits(a.app_k, d);
    vx[i][d] = old ? tail[(size_t)(GS + i) * D + d] : new_bits(a.app_v, d);
  }
  __syncthreads();
  const int M = cell.kind == KIND_Q2 ? 3 : 15;
  quantize_group_codes<D, GS>([&](int i, int d) { return (double)bf16_bits_to_f32(kx[i][d]); },
                              [&](int i, int d) { return (double)bf16_bits_to_f32(vx[i][d]); }, M, kc, vc, kmeta,
                              vmeta, tid, kThreads);
  __syncthreads();
  const int g = L0 / GS;
  const int rec = record_bytes(cell.kind, D, GS);
  const int32_t* bt = a.block_table + (size_t)b * a.bt_stride;
  for (int part = 0; part < GS / kBlock; ++part) {
    const int j = (GS / kBlock) * g + part;
    if ((j >> a.bt_shift) >= a.bt_stride || (uint32_t)bt[j >> a.bt_shift] >= (uint32_t)a.num_pages) continue;
    uint32_t* r = reinterpret_cast<uint32_t*>(const_cast<uint8_t*>(a.ws) + cell.pool_off +
                                              ((size_t)record_slot(bt, j, a.bt_shift) * a.n_kv_heads + kh) * rec);
    pack_record<D, GS>(r, cell.kind, part, kc, vc, kmeta, vmeta, tid, kThreads);
  }
}

// SKIP (with SPARSE, PH_ROW): the token-skipping ablation. The same coarse pass and
// selection, but the values are not streamed and the unselected quantized tokens leave the
// attention: the softmax runs over the selected tokens (at 4 bits) and the tail only.
// What a finishing launch reads of its row's partials, requested at the launch's start: lane
// i of every wave holds partial i's (m, l) (n_split <= 64); the partials' value vectors are
// staged in LDS after the row's regions when they fit (pre), else the merge loads them.
struct FinishIn {
  const float* parts = nullptr;
  float* pre = nullptr;
  float m = -INFINITY, l = 0.f;
};

template <int D, int GS, int MODE, bool SPARSE, int PH, bool SKIP = false, class RW>
__device__ __forceinline__ void row_body(const DecodeArgs& a, const RW& r, const Smem& sm, size_t orow, int split,
                                         const FinishIn& fin) {
  using G = Geo<D, MODE, GS>;
  using GN = Geo<D, MODE, GS, false>;   // value-lane layout after the pass (corrections, merge)
  using KS = KStep<D, MODE, false, GS>;
  using VS = VStep<D, MODE, GS>;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  float* scr = sm.wscr + w * wave_scratch(D);
  uint32_t* klimb = reinterpret_cast<uint32_t*>(scr);
  // coarse scores: LDS, except the partial launches of a split row, which leave them in the
  // row's scratch line for the finishing launch to copy back into LDS
  float* scores = (SPARSE && PH == PH_PART) ? a.part_scores + orow * (size_t)a.split_row_stride : sm.scores;
  uint32_t* selm = sm.selm;
  float* misc = sm.misc;
  constexpr int NE = G::NE;
  constexpr int VCH = G::VCH;

  Acc<VCH> st;
  st.zero();
  KS::fill_qperm(sm.qs, sm.qperm);
  const float* parts = fin.parts;
  const float part_m = fin.m, part_l = fin.l;
  float* pre_parts = fin.pre;
  // The row's coarse (M, L) from the partials: with tau L > 1 no token is selected (see the
  // selection below) and the score line is not needed.
  bool stage_scores = SPARSE && PH == PH_FINISH;
  if constexpr (SPARSE && PH == PH_FINISH) {
    const float Mf = wave_max(part_m);
    stage_scores = !(a.tau * wave_sum(part_m > -INFINITY ? part_l * __expf(part_m - Mf) : 0.f) > 1.f);
  }
  if (stage_scores) {
    // the row's coarse scores (tail included) from its scratch line into LDS: eight
    // independent 16-byte loads per thread in flight at once
    const float4* g4 = reinterpret_cast<const float4*>(a.part_scores + orow * (size_t)a.split_row_stride);
    float4* l4 = reinterpret_cast<float4*>(scores);
    const int n4 = (r.N + 3) / 4;   // within the line: its stride is a multiple of 64 floats
    for (int base = tid; base < n4; base += 8 * kThreads) {
      // eight named registers (an array here can end up in scratch memory); N >= 1
      const float4 v0 = g4[min(base + 0 * kThreads, n4 - 1)], v1 = g4[min(base + 1 * kThreads, n4 - 1)];
      const float4 v2 = g4[min(base + 2 * kThreads, n4 - 1)], v3 = g4[min(base + 3 * kThreads, n4 - 1)];
      const float4 v4 = g4[min(base + 4 * kThreads, n4 - 1)], v5 = g4[min(base + 5 * kThreads, n4 - 1)];
      const float4 v6 = g4[min(base + 6 * kThreads, n4 - 1)], v7 = g4[min(base + 7 * kThreads, n4 - 1)];
      if (base + 0 * kThreads < n4) l4[base + 0 * kThreads] = v0;
      if (base + 1 * kThreads < n4) l4[base + 1 * kThreads] = v1;
      if (base + 2 * kThreads < n4) l4[base + 2 * kThreads] = v2;
      if (base + 3 * kThreads < n4) l4[base + 3 * kThreads] = v3;
      if (base + 4 * kThreads < n4) l4[base + 4 * kThreads] = v4;
      if (base + 5 * kThreads < n4) l4[base + 5 * kThreads] = v5;
      if (base + 6 * kThreads < n4) l4[base + 6 * kThreads] = v6;
      if (base + 7 * kThreads < n4) l4[base + 7 * kThreads] = v7;
    }
  }
  __syncthreads();

  // ---- single streaming pass: K scores, online softmax, V accumulation; wave w takes the
  // steps (chunks of TPS tokens) w, w + 8, ...; the loads of the next step are in flight
  // while a step computes
  const int nb = r.n_q / kBlock;
  int cb = 0, n_chunks = (r.n_q + G::TPS - 1) / G::TPS;   // this workgroup's chunks: [cb, n_chunks)
  if constexpr (PH == PH_PART) split_range(n_chunks, a.n_split, split, cb, n_chunks);
  if constexpr (PH == PH_FINISH) n_chunks = 0;
  const int steps = (n_chunks - cb + kWaves - 1) / kWaves;
  typename KS::Buf kb0, kb1;
  typename VS::Buf vb0, vb1;
  // K loads of step s + 1 are issued as step s starts, its V loads once step s's K part is
  // done: each load has about one step of lead while at most three buffers are live.
  auto issue_k = [&](int s, typename KS::Buf& kb) {
    const int c = cb + s * kWaves + w;
    if (c >= n_chunks) return;   // no chunk for this wave (uniform)
    int groups[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int g = c * G::GPS + i;
      groups[i] = (i < G::GPS && g < r.n_groups) ? g : c * G::GPS;
    }
    KS::load(r, groups, lane, kb);
  };
  auto issue_v = [&](int s, typename VS::Buf& vb) {
    if constexpr (SKIP) return;
    const int c = cb + s * kWaves + w;
    if (c >= n_chunks) return;
    VS::load(r, c * G::BPS, nb, lane, vb);
  };
  auto step_k = [&](int s, const typename KS::Buf& kb) -> float {
    const int c = cb + s * kWaves + w;
    if (c >= n_chunks) return 0.f;
    bool own;
    int t_loc;
    if constexpr (G::TPS == 128) {   // two tokens per lane: lane and lane + 64
      float sc1;
      const float sc0 = KS::compute(sm.qperm, klimb, lane, kb, own, t_loc, &sc1);
      const bool v0 = c * G::GPS + lane / kUnit < r.n_groups, v1 = c * G::GPS + (64 + lane) / kUnit < r.n_groups;
      const float s0 = v0 ? sc0 : -INFINITY, s1 = v1 ? sc1 : -INFINITY;
      if (v0) scores[c * G::TPS + lane] = s0;
      if (v1) scores[c * G::TPS + 64 + lane] = s1;
      const float smax = fmaxf(s0, s1);
      if (__any(smax > st.m)) st.raise(wave_max(smax));
      const float w0 = v0 ? __expf(s0 - st.m) : 0.f, w1 = v1 ? __expf(s1 - st.m) : 0.f;
      st.lsum += w0 + w1;
      wave_sync_lds();   // the transposed scores are read before the weights overwrite them
      scr[G::S_W + lane] = w0;
      scr[G::S_W + 64 + lane] = w1;
      wave_sync_lds();
      return 0.f;
    } else {
      const float sc0 = KS::compute(sm.qperm, klimb, lane, kb, own, t_loc);
      const bool valid = own && c * G::GPS + t_loc / kUnit < r.n_groups;
      const float sc = valid ? sc0 : -INFINITY;
      if (valid) scores[c * G::TPS + t_loc] = sc;
      if (__any(sc > st.m)) st.raise(wave_max(sc));   // a new running maximum (rare once warm)
      const float wgt = valid ? __expf(sc - st.m) : 0.f;
      st.lsum += wgt;
      if constexpr (!G::QUAD_W) {
        wave_sync_lds();   // the K limbs are read before the weights overwrite them
        if (own) scr[G::S_W + t_loc] = wgt;
      }
      wave_sync_lds();
      return wgt;
    }
  };
  auto step_v = [&](int s, const typename VS::Buf& vb, float wgt) {
    if constexpr (SKIP) return;
    const int c = cb + s * kWaves + w;
    if (c >= n_chunks) return;
    VS::compute(wgt, scr + G::S_W, scr, lane, vb, st);
    wave_sync_lds();
  };
  if (steps > 0) {
    issue_k(0, kb0);
    issue_v(0, vb0);
  }
  // Waves w and w + 4 share a SIMD, where the older wave wins issue ties; left alone, waves
  // 4..7 finish their steps well after waves 0..3 and the merge waits for them. The two take
  // turns at the higher priority instead: one step each per loop round.
  const bool hi_half = w >= 4;
  for (int s = 0; s < steps; s += 2) {
    if (hi_half) __builtin_amdgcn_s_setprio(1);
    else __builtin_amdgcn_s_setprio(0);
    if (s + 1 < steps) issue_k(s + 1, kb1);
    float wgt = step_k(s, kb0);
    if (s + 1 < steps) issue_v(s + 1, vb1);
    step_v(s, vb0, wgt);
    if (s + 1 >= steps) break;
    if (hi_half) __builtin_amdgcn_s_setprio(0);
    else __builtin_amdgcn_s_setprio(1);
    if (s + 2 < steps) issue_k(s + 2, kb0);
    wgt = step_k(s + 1, kb1);
    if (s + 2 < steps) issue_v(s + 2, vb0);
    step_v(s + 1, vb1, wgt);
  }
  __builtin_amdgcn_s_setprio(0);
  if constexpr (G::W128 && !SKIP) {
    // 128-token steps leave lane (block jb = lane / 8, chunk) with channels 8 chunk .. of
    // block jb: sum the eight blocks (lane bits 3, 4, 5) and hand the channel totals to the
    // 64-token value-lane layout the rest of the row uses (lanes 0..15, 4 channels each)
    float x[VCH];
#pragma unroll
    for (int c = 0; c < VCH; ++c) x[c] = add_halves(add_rows2(st.acc[c] + dpp<0x128>(st.acc[c])));   // row_ror:8
    wave_sync_lds();
    if (lane < 8) {
#pragma unroll
      for (int c = 0; c < VCH; ++c) scr[VCH * lane + c] = x[c];
    }
    wave_sync_lds();
#pragma unroll
    for (int c = 0; c < VCH; ++c) st.acc[c] = lane < 16 && c < GN::VCH ? scr[GN::VCH * lane + c % GN::VCH] : 0.f;
    wave_sync_lds();
  }
  // ---- tail (exact bf16): tokens n_q + w, n_q + w + 8, ...; a lane holds the TC contiguous
  // channels lane TC .. lane TC + TC - 1 (tacc), read with one load per row. A wave requests the
  // K and V rows of TB of its tail tokens at once, then works through them, so the tail costs
  // one memory round trip per TB tokens instead of one per token.
  constexpr int TC = D / 64;
  constexpr int TB = 2;
  float tacc[TC];
#pragma unroll
  for (int i = 0; i < TC; ++i) tacc[i] = 0.f;
  const bool has_tail = PH == PH_ROW || (PH == PH_PART && split == a.n_split - 1);
  float tl = 0.f;   // SKIP: the tail's weight (lane 0)
  for (int t0 = r.n_q + w; has_tail && t0 < r.N; t0 += TB * kWaves) {
    TailRow<TC> kr[TB], vr[TB];
#pragma unroll
    for (int k = 0; k < TB; ++k) {
      const int t = t0 + k * kWaves;
      if (t < r.N) {
        kr[k].load(r.tail + (size_t)(t % GS) * D + lane * TC);
        vr[k].load(r.tail + (size_t)(GS + t % GS) * D + lane * TC);
      }
    }
#pragma unroll
    for (int k = 0; k < TB; ++k) {
      const int t = t0 + k * kWaves;
      if (t >= r.N) break;   // uniform over the wave
      float p = 0.f;
#pragma unroll
      for (int i = 0; i < TC; ++i) p = fmaf(sm.qs[lane * TC + i], kr[k].f(i), p);
      p = uniform(wave_sum(p));
      if (lane == 0) scores[t] = p;
      if (p > st.m) {
        const float f = st.raise(p);
#pragma unroll
        for (int i = 0; i < TC; ++i) tacc[i] *= f;
        if constexpr (SKIP) tl *= f;
      }
      const float wgt = __expf(p - st.m);
      if (lane == 0) st.lsum += wgt;
      if constexpr (SKIP)
        if (lane == 0) tl += wgt;
#pragma unroll
      for (int i = 0; i < TC; ++i) tacc[i] = fmaf(wgt, vr[k].f(i), tacc[i]);
    }
  }

  // ---- selection (4-bit target, 0 < tau <= 1) and corrections
  bool use_parts = true;   // PH_FINISH: the partials hold the row's streamed part
  if constexpr (SPARSE && PH != PH_PART) {
    float M = -INFINITY, L = 0.f;   // the row's coarse maximum and weight
    if constexpr (PH == PH_FINISH) {
      M = wave_max(part_m);   // the scores reached LDS at the row's start
      L = wave_sum(part_m > -INFINITY ? part_l * __expf(part_m - M) : 0.f);
    } else {
      const float lw = wave_sum(st.lsum);
      if (lane == 0) {
        misc[w] = st.m;
        misc[8 + w] = lw;
      }
      __syncthreads();
      M = misc[0];
      for (int i = 1; i < kWaves; ++i) M = fmaxf(M, misc[i]);
      for (int i = 0; i < kWaves; ++i)
        if (misc[i] > -INFINITY) L += misc[8 + i] * __expf(misc[i] - M);
    }
    if (st.m > -INFINITY) {
      const float f = st.raise(M);
#pragma unroll
      for (int i = 0; i < TC; ++i) tacc[i] *= f;
      if constexpr (SKIP) tl *= f;
    }
    st.m = M;   // every wave now shares the reference M
    if constexpr (SKIP) st.lsum = tl;   // the quantized tokens' coarse weights served the selection only
    float removed = 0.f;   // coarse weight taken out by the corrections
    // exp(s - M) / L >= tau  <=>  s >= M + ln(tau L): one compare per token. With tau L > 1 the
    // threshold lies above the maximum M, so no token is selected: the row skips the scan and
    // the gather (the same outcome as running them).
    const float thr = M + logf(a.tau * L);
    const bool none = a.tau * L > 1.f;   // the same in every wave
    const int n_units = none ? 0 : r.n_groups;
    if (!none) {
      // Selection words: wave w scans 256 tokens per round, lane l the four tokens 4l .. 4l + 3
      // with one LDS read; ballot k holds bit k of every lane's four, and the word of unit u
      // (lanes 8u .. 8u + 7, token 4m + k of the unit at bit 4m + k) interleaves byte u of
      // the four ballots.
      for (int base = 256 * w; base < r.n_q; base += 256 * kWaves) {
        const int t0 = base + 4 * lane;   // n_q is a multiple of 32: all four or none valid
        bool p0 = false, p1 = false, p2 = false, p3 = false;
        if (t0 < r.n_q) {
          const float4 v = *reinterpret_cast<const float4*>(scores + t0);
          p0 = v.x >= thr;
          p1 = v.y >= thr;
          p2 = v.z >= thr;
          p3 = v.w >= thr;
        }
        const unsigned long long b0 = __ballot(p0), b1 = __ballot(p1), b2 = __ballot(p2), b3 = __ballot(p3);
        const int g = base / kUnit + lane;
        if (lane < 8 && g < r.n_groups) {
          const int sh = 8 * lane;
          selm[g] = spread4((uint32_t)(b0 >> sh) & 0xffu) | (spread4((uint32_t)(b1 >> sh) & 0xffu) << 1) |
                    (spread4((uint32_t)(b2 >> sh) & 0xffu) << 2) | (spread4((uint32_t)(b3 >> sh) & 0xffu) << 3);
        }
      }
      __syncthreads();
    }
    if (a.sel_mask) {
      uint32_t* smo = a.sel_mask + orow * (size_t)a.sel_words;
      for (int g = tid; g < a.sel_words; g += kThreads) smo[g] = g < n_units ? selm[g] : 0u;
    }
    // Gather: the selected units are dealt round-robin over the waves in unit order (the
    // unit of rank k goes to wave k mod 8), and a wave corrects its units as many at a time as
    // a coarse step holds (two; one at D = 256), so the dependent loads of the corrections
    // spread over all waves however the selected units cluster.
    using KR = KStep<D, MODE_COARSE, true, GS>;
    using GC = Geo<D, MODE_COARSE, GS, false>;
    float* wfix = scr;   // [2][64]: refined and coarse weights of the step's selected tokens
    int rank0 = 0;       // selected units in the spans before this one (the same in every wave)
    for (int g64 = 0; g64 < n_units; g64 += 64) {
      const int gi = g64 + lane;
      const unsigned long long all = __ballot(gi < r.n_groups && selm[gi < r.n_groups ? gi : 0] != 0u);
      unsigned long long pend = 0;   // this wave's share of the span
      {
        unsigned long long rest = all;
        for (int k = rank0; rest; ++k) {
          const unsigned long long bit = rest & (~rest + 1ull);
          rest &= rest - 1;
          if (k % kWaves == w) pend |= bit;
        }
      }
      rank0 += __builtin_popcountll(all);
      while (pend) {
        int groups[2] = {-1, -1};
        groups[0] = g64 + __builtin_ctzll(pend);
        pend &= pend - 1;
        if constexpr (GC::GPS == 2) {
          groups[1] = pend ? g64 + __builtin_ctzll(pend) : -1;
          if (pend) pend &= pend - 1;
        }
        typename KR::Buf kb;
        const int lg[2] = {groups[0], groups[1] >= 0 ? groups[1] : groups[0]};
        KR::load(r, lg, lane, kb);
        // the V words the corrections need are loaded together with the K low plane (one
        // memory round trip): value-lane layout of the step, blocks holding a selected token
        const int jb = lane / GC::LPB, chunk = lane % GC::LPB;
        const int gv = groups[jb / 2];
        const uint32_t bm = gv >= 0 ? (selm[gv] >> (16 * (jb % 2))) & 0xffffu : 0u;
        const int ev = chunk * GC::VCH / kUnit / GC::GU;   // meta group of the lane's channels
        uint4 hw4[GC::VCH / 4], lw4[GC::VCH / 4], mv4[4];
        if (bm) {
          const uint8_t* rb = r.rec_ptr(2 * gv + jb % 2);
#pragma unroll
          for (int i = 0; i < GC::VCH / 4; ++i) {
            const int qp = 16 * vquad_pos(chunk * GC::NV4 + i, GC::NQ, GC::VR);
            hw4[i] = *reinterpret_cast<const uint4*>(rb + off_v_planes(D, GS) + qp);
            lw4[i] = *reinterpret_cast<const uint4*>(rb + off_vlo(D, GS) + qp);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i)
            mv4[i] = *reinterpret_cast<const uint4*>(rb + off_vmeta_planes(D, GS) + 4 * (ev * kBlock + 4 * i));
        }
        bool own;
        int t_loc;
        const float delta = KR::compute(sm.qperm, klimb, lane, kb, own, t_loc);
        const int ti = t_loc % kUnit;
        const int g = groups[t_loc / kUnit];
        const bool sel = own && g >= 0 && ((selm[g < 0 ? 0 : g] >> ti) & 1u);
        const int t = g * kUnit + ti;
        const float s_hat = sel ? scores[t] : 0.f;
        const float s_ref = s_hat + delta;
        if (sel) scores[t] = s_ref;
        const float sref = sel ? s_ref : -INFINITY;
        if (__any(sref > st.m)) {
          const float f = st.raise(wave_max(sref));
          removed *= f;
#pragma unroll
          for (int i = 0; i < TC; ++i) tacc[i] *= f;
        }
        const float wf = sel ? __expf(s_ref - st.m) : 0.f;
        const float wc = (sel && !SKIP) ? __expf(s_hat - st.m) : 0.f;   // SKIP: nothing to take out
        st.lsum += wf - wc;
        removed += wc;
        wave_sync_lds();
        if (own) {
          wfix[t_loc] = wf;
          wfix[64 + t_loc] = wc;
        }
        wave_sync_lds();
        // corrections of the selected tokens' values
        if (bm) {
          for (int tt = 0; tt < kBlock; ++tt) {
            if (!((bm >> tt) & 1u)) continue;
            const uint32_t mw = w4(mv4[tt / 4], tt % 4);
            const float s = f16lo(mw), z = f16hi(mw);
            const float f1 = wfix[jb * kBlock + tt], f0 = wfix[64 + jb * kBlock + tt];
            // w' (z + s (4 hi + lo)) - w (z + s (4 hi + 3/2)) = A hi + B lo + C
            const float A = 4.f * s * (f1 - f0), B = s * f1, C = (f1 - f0) * z - 1.5f * s * f0;
            const int sh = 8 * (tt % 4) + 2 * (tt / 4);
#pragma unroll
            for (int c = 0; c < GC::VCH; ++c) {
              const uint32_t hwc = w4(hw4[c / 4], c % 4), lwc = w4(lw4[c / 4], c % 4);
              st.acc[c] += fmaf(A, (float)((hwc >> sh) & 3u), fmaf(B, (float)((lwc >> sh) & 3u), C));
            }
          }
        }
        wave_sync_lds();
      }
    }
    // Cancellation check over the row (nothing removed when nothing was selected).
    if (!none) {
      const float lw2 = wave_sum(st.lsum), rw = wave_sum(removed);
      __syncthreads();
      if (lane == 0) {
        misc[w] = st.m;
        misc[8 + w] = lw2;
        misc[16 + w] = rw;
      }
      __syncthreads();
      float Ms = misc[0];
      for (int i = 1; i < kWaves; ++i) Ms = fmaxf(Ms, misc[i]);
      float Lp = 0.f, Rm = 0.f;
      for (int i = 0; i < kWaves; ++i) {
        const float f = __expf(misc[i] - Ms);
        Lp += misc[8 + i] * f;
        Rm += misc[16 + i] * f;
      }
      if (PH == PH_FINISH) Lp += L * __expf(M - Ms);   // the streamed part's coarse weight
      if (Rm > 8.f * Lp) {   // recompute the row's V from the final scores
        use_parts = false;
        __syncthreads();
        float ls = 0.f;
        for (int t = tid; t < r.N; t += kThreads) {
          const float wgt = __expf(scores[t] - Ms);
          scores[t] = wgt;
          ls += wgt;
        }
        __syncthreads();
        st.zero();
        st.m = Ms;
        st.lsum = ls;
        exact_v_pass<D, GS>(r, scores, selm, lane, w, st.acc);
#pragma unroll
        for (int i = 0; i < TC; ++i) tacc[i] = 0.f;
        for (int t = r.n_q + w; t < r.N; t += kWaves) {
          const uint16_t* vt = r.tail + (size_t)(GS + t % GS) * D;
#pragma unroll
          for (int i = 0; i < TC; ++i) tacc[i] = fmaf(scores[t], bf16f(vt[lane * TC + i]), tacc[i]);
        }
      }
    }
  } else if constexpr (PH != PH_PART) {
    if (a.sel_mask) {
      const uint32_t fill = (MODE == MODE_DENSE || MODE == MODE_KIVI) ? 0xffffffffu : 0u;
      uint32_t* smo = a.sel_mask + orow * (size_t)a.sel_words;
      for (int g = tid; g < a.sel_words; g += kThreads) smo[g] = g < r.n_groups ? fill : 0u;
    }
  }

  // ---- merge the waves (the exact pass writes in the value-lane layout of the coarse
  // step, which is this mode's layout whenever it runs). Each wave folds its value lanes over
  // the step's blocks with cross-row swaps, adds its constant terms and its tail channels,
  // scales by exp(m_w - M) and leaves one D-vector in LDS; four lanes per channel then add
  // the waves (and, finishing a split row, the partials) in a fixed order.
  const float lsum = wave_sum(st.lsum);
  // constant terms of each 32-channel slice e: the lanes l = e (mod NE) summed by row
  // rotates and cross-row swaps; lane e then holds slice e's
  float zl = lane < G::COOP ? st.accz : 0.f;
  static_assert(NE == 2 || NE == 4 || NE == 8, "slices per row");
  zl += dpp<0x128>(zl);                           // row_ror:8
  if constexpr (NE <= 4) zl += dpp<0x124>(zl);    // row_ror:4
  if constexpr (NE <= 2) zl += dpp<0x122>(zl);    // row_ror:2
  zl = add_halves(add_rows2(zl));
  float zs[NE];
#pragma unroll
  for (int e = 0; e < NE; ++e) zs[e] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(zl), e));
  __syncthreads();   // scores are dead from here on: reuse them for the wave vectors
  if (lane == 0) {
    misc[w] = st.m;
    misc[8 + w] = lsum;
  }
  __syncthreads();
  float M = misc[0];
  for (int i = 1; i < kWaves; ++i) M = fmaxf(M, misc[i]);
  // PH_FINISH: the row's partials join the merge, unless the exact pass replaced them
  const bool with_parts = PH == PH_FINISH && use_parts;
  if (with_parts) M = fmaxf(M, wave_max(part_m));
  const float part_f = with_parts && part_m > -INFINITY ? __expf(part_m - M) : 0.f;   // lane i: partial i
  const float fw = st.m > -INFINITY ? __expf(st.m - M) : 0.f;
  float* wv = sm.scores;   // [kWaves][D]
  float* pf = misc + 32;   // [n_split] the partials' factors (n_split <= 64)
  {
    constexpr int VN = GN::VCH;
    float v[VN];
#pragma unroll
    for (int c = 0; c < VN; ++c) {
      float x = st.acc[c];
      if constexpr (GN::BPS == 4) x = add_halves(add_rows2(x));   // lanes chunk + 16 vb
      else x = add_halves(x);                                     // lanes chunk + 32 vb
      v[c] = x;
    }
    const int chunk = lane % GN::LPB;
    if (lane < GN::LPB) {
#pragma unroll
      for (int c = 0; c < VN; ++c) {
        const int e = (chunk * VN + c) / kUnit;   // the channel's 32-channel slice
        float z = zs[0];
#pragma unroll
        for (int k = 1; k < NE; ++k) z = e == k ? zs[k] : z;
        wv[w * D + chunk * VN + c] = (v[c] + z) * fw;
      }
    }
  }
  wave_sync_lds();   // the wave's value lanes wrote its vector; its tail lanes add theirs
#pragma unroll
  for (int i = 0; i < TC; ++i) wv[w * D + lane * TC + i] += tacc[i] * fw;
  if (with_parts && w == 0 && lane < a.n_split) pf[lane] = part_f;
  __syncthreads();
  float Lt = 0.f;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) Lt += misc[8 + i] * (misc[i] > -INFINITY ? __expf(misc[i] - M) : 0.f);
  if (with_parts) Lt += wave_sum(part_l * part_f);
  const int j = tid & 3;
  for (int d = tid >> 2; d < D; d += kThreads / 4) {   // four lanes per channel (quad-uniform)
    float o = wv[j * D + d] + wv[(j + 4) * D + d];
    if (with_parts) {
      for (int i = j; i < a.n_split; i += 4) {
        const float pv = pre_parts ? pre_parts[i * D + d] : parts[(size_t)i * (2 + D) + 2 + d];
        o = fmaf(pv, pf[i], o);
      }
    }
    o += dpp<0xB1>(o);   // quad_perm [1,0,3,2]
    o += dpp<0x4E>(o);   // quad_perm [2,3,0,1]
    if (j != 0) continue;
    if constexpr (PH == PH_PART) {   // unnormalized, relative to M
      float* pp = a.part + (orow * (size_t)a.n_split + split) * (2 + D);
      if (d == 0) {
        pp[0] = M;
        pp[1] = Lt;
      }
      pp[2 + d] = o;
      continue;
    }
    if constexpr (SKIP) o = Lt > 0.f ? o / Lt : 0.f;   // nothing kept: 0
    else o = o / Lt;
    if (a.out_bf16) {
      uint32_t u = __float_as_uint(o);
      u += 0x7fffu + ((u >> 16) & 1u);
      reinterpret_cast<uint16_t*>(a.out)[orow * D + d] = (uint16_t)(u >> 16);
    } else {
      reinterpret_cast<float*>(a.out)[orow * D + d] = o;
    }
  }
}

// One kernel per selection regime of the launch (tau = 0, tau > 1, 0 < tau <= 1, or the
// KIVI-4 layout), so each variant gets its own register allocation; rows of 2-bit cells
// run the 2-bit path inside every planes variant.
enum : int { VAR_KIVI = 0, VAR_DENSE = 1, VAR_COARSE = 2, VAR_SPARSE = 3, VAR_SKIP = 4 };

// Head dim 256 with both planes (tau = 0) or the KIVI-4 layout needs ~156 VGPRs: those kernels
// run one workgroup per CU rather than spill (about a third faster than spilling at two).
template <int D, int VAR>
constexpr int decode_waves_per_simd() {
  return (D == 256 && (VAR == VAR_DENSE || VAR == VAR_KIVI)) ? 2 : kWavesPerSimd;
}

// Finishing launch of a split row that selects nothing (every row of a launch whose target
// is not 4-bit, or with tau L > 1): the output is the partials' merge alone, read by four
// lanes per channel in the same order as the general merge (whose wave vectors are zero
// here), so the result is the same bit for bit. The partials' factors reach the lanes by
// lane shuffles; no workgroup barrier is needed past the staging of the value vectors.
template <int D>
__device__ void finish_from_partials(const DecodeArgs& a, const FinishIn& fin, size_t orow, int n_groups,
                                     uint32_t fill) {
  const int tid = threadIdx.x;
  if (fin.pre) __syncthreads();   // the staged value vectors
  const float M = wave_max(fin.m);   // lanes >= n_split hold -inf
  const float f = fin.m > -INFINITY ? __expf(fin.m - M) : 0.f;
  const float Lt = wave_sum(fin.l * f);
  const int j = tid & 3;
  for (int d = tid >> 2; d < D; d += kThreads / 4) {   // quad-uniform
    float o = 0.f;
    for (int i = j; i < a.n_split; i += 4) {
      const float pv = fin.pre ? fin.pre[i * D + d] : fin.parts[(size_t)i * (2 + D) + 2 + d];
      o = fmaf(pv, __shfl(f, i), o);
    }
    o += dpp<0xB1>(o);   // quad_perm [1,0,3,2]
    o += dpp<0x4E>(o);   // quad_perm [2,3,0,1]
    if (j != 0) continue;
    o = o / Lt;
    if (a.out_bf16) {
      uint32_t u = __float_as_uint(o);
      u += 0x7fffu + ((u >> 16) & 1u);
      reinterpret_cast<uint16_t*>(a.out)[orow * D + d] = (uint16_t)(u >> 16);
    } else {
      reinterpret_cast<float*>(a.out)[orow * D + d] = o;
    }
  }
  if (a.sel_mask) {
    uint32_t* smo = a.sel_mask + orow * (size_t)a.sel_words;
    for (int g = tid; g < a.sel_words; g += kThreads) smo[g] = g < n_groups ? fill : 0u;
  }
}

template <int D, int GS, int VAR, int PH, bool BIG>
__global__ void __launch_bounds__(kThreads, (decode_waves_per_simd<D, VAR>())) k_decode(DecodeArgs a) {
  extern __shared__ float smem[];
  // Rows are (cell, sequence, query head). PH_PART: workgroup (row, split), the splits of a
  // row adjacent. PH_ROW with grouped queries (G query heads per KV head): workgroups are
  // dispatched round-robin over the 8 XCDs, so the G rows of one KV head take the block
  // indices 8 apart (same XCD, same L2, dispatched together) and stream the same records.
  const int G = a.n_heads / a.n_kv_heads;
  int row;
  if (PH == PH_ROW && G > 1) {
    const int span = 8 * G, q = blockIdx.x / span, rem = blockIdx.x % span;
    const int gi = 8 * q + rem % 8;   // (cell, sequence, KV head)
    if (gi >= a.n_cells * a.n_seqs * a.n_kv_heads) return;   // grid padding
    row = (gi / a.n_kv_heads) * a.n_heads + (gi % a.n_kv_heads) * G + rem / 8;
  } else {
    row = PH == PH_PART ? blockIdx.x / a.n_split : blockIdx.x;
  }
  const int split = PH == PH_PART ? blockIdx.x % a.n_split : 0;
  const int h = row % a.n_heads;
  const int kh = h / G;   // the KV head this query head reads
  const int b = (row / a.n_heads) % a.n_seqs;
  const int ci = row / (a.n_heads * a.n_seqs);
  const DecodeCell cell = a.cells[ci];
  const int tid = threadIdx.x;
  const size_t orow = ((size_t)ci * a.n_seqs + b) * a.n_heads + h;
  if (a.app_k && (PH == PH_ROW || (PH == PH_PART && split == a.n_split - 1))) {
    static_assert(fused_append_lds_bytes(D, GS) <= 160 * 1024, "in-launch append LDS");
    fused_append<D, GS>(a, cell, b, kh, reinterpret_cast<unsigned char*>(smem));
    __syncthreads();   // the appended token and records are written before the row reads them
  }
  const size_t lp = lds_lpad(a.max_len);
  Smem sm;
  sm.scores = smem;
  sm.selm = reinterpret_cast<uint32_t*>(smem + lds_region_a(a.max_len, D));
  sm.boff = sm.selm + pad4(lp / 32);
  sm.qs = reinterpret_cast<float*>(sm.boff + pad4(lp / 16 + 16));
  sm.qperm = sm.qs + D;
  sm.wscr = sm.qperm + D;
  sm.misc = sm.wscr + kWaves * wave_scratch(D);

  // PH_FINISH: the row's partials depend on nothing the prologue reads, so they are
  // requested first and their latency overlaps the prologue's
  FinishIn fin;
  if constexpr (PH == PH_FINISH) {
    fin.parts = a.part + orow * (size_t)a.n_split * (2 + D);
    const int lane = tid & 63;
    if (lane < a.n_split) {
      fin.m = fin.parts[(size_t)lane * (2 + D)];
      fin.l = fin.parts[(size_t)lane * (2 + D) + 1];
    }
    if (finish_parts_in_lds(a.max_len, D, a.n_split)) {
      fin.pre = sm.misc + 96;
      for (int idx = tid; idx < a.n_split * D; idx += kThreads)
        fin.pre[idx] = fin.parts[(size_t)(idx / D) * (2 + D) + 2 + idx % D];
    }
  }
  // PH_ROW / PH_PART: the row's block-table entries (every block a row of max_len tokens can
  // have quantized) are requested together with its length, so the first record loads wait
  // for one memory round trip less; the entries past the row are never used.
  constexpr int kBtPer = (LOOPKV_MAX_LEN / kBlock + kThreads - 1) / kThreads;
  int32_t btv[kBtPer];
  if constexpr (PH != PH_FINISH) {
    const int32_t* bt0 = a.block_table + (size_t)b * a.bt_stride;
    const int nb_max = a.max_len / kBlock;   // bt_stride pages cover max_len tokens
#pragma unroll
    for (int k = 0; k < kBtPer; ++k) {
      const int j = tid + k * kThreads;
      btv[k] = j < nb_max ? bt0[j >> a.bt_shift] : 0;
    }
  }
  const int N = a.seq_lens[b];

  // rows that read nothing: empty (output 0) or invalid (NaN; length above max_len, or a
  // page of the quantized prefix outside the pool)
  auto empty_row = [&](bool zero) {
    if (PH == PH_PART) return;   // the finishing launch writes the row
    const float v = zero ? 0.f : __builtin_nanf("");
    for (int d = tid; d < D; d += kThreads) {
      if (a.out_bf16) reinterpret_cast<uint16_t*>(a.out)[orow * D + d] = zero ? 0 : 0x7fc0;
      else reinterpret_cast<float*>(a.out)[orow * D + d] = v;
    }
    if (a.sel_mask)
      for (int g = tid; g < a.sel_words; g += kThreads) a.sel_mask[orow * (size_t)a.sel_words + g] = 0u;
  };
  if (N <= 0 || N > a.max_len) {
    empty_row(N == 0);
    return;
  }

  RowT<BIG> r;
  r.pool = a.ws + cell.pool_off;
  r.boff = sm.boff;
  const int slot = a.seq_slots ? a.seq_slots[b] : b;
  if ((uint32_t)slot >= (uint32_t)a.max_seqs) {   // no tail of this row exists
    empty_row(false);
    return;
  }
  r.tail = reinterpret_cast<const uint16_t*>(a.ws + cell.tail_off) + ((size_t)slot * a.n_kv_heads + kh) * tail_elems(D, GS);
  r.N = N;
  r.n_q = (N / GS) * GS;
  r.n_groups = r.n_q / kUnit;   // 32-token units of the quantized prefix

  if constexpr (PH == PH_FINISH) {
    // A row whose prefix maps a page outside the pool has NaN partials (its partial launch
    // checked the pages and read no record).
    const int lane = tid & 63;
    if (__any(lane < a.n_split && fin.m != fin.m)) {
      empty_row(false);
      return;
    }
    // Rows that select nothing need neither the block table nor the query: the partials
    // are the row.
    bool selects = false;
    if constexpr (VAR == VAR_SPARSE || VAR == VAR_SKIP) {
      selects = VAR == VAR_SKIP || cell.kind != KIND_Q2;
      if (VAR == VAR_SPARSE && selects) {
        const float Mf = wave_max(fin.m);
        selects = !(a.tau * wave_sum(fin.m > -INFINITY ? fin.l * __expf(fin.m - Mf) : 0.f) > 1.f);
      }
    }
    if (!selects) {
      const bool full = VAR == VAR_KIVI || (VAR == VAR_DENSE && cell.kind != KIND_Q2);   // every token at 4 bits
      finish_from_partials<D>(a, fin, orow, r.n_groups, full ? 0xffffffffu : 0u);
      return;
    }
  }

  // block table row and sigma * q into LDS
  const int32_t* bt = a.block_table + (size_t)b * a.bt_stride;
  const int nbq = r.n_q / kBlock;
  const uint32_t rec256 = (uint32_t)(record_bytes(cell.kind, D, GS) / 256);
  int bad_page = 0;
  if constexpr (PH != PH_FINISH) {
#pragma unroll
    for (int k = 0; k < kBtPer; ++k) {
      const int j = tid + k * kThreads;
      if (j < nbq) {
        bad_page |= (uint32_t)btv[k] >= (uint32_t)a.num_pages;   // -1 (unmapped) included
        const uint32_t slot_j = ((uint32_t)btv[k] << a.bt_shift) + (uint32_t)(j & ((1 << a.bt_shift) - 1));
        sm.boff[j] = (slot_j * (uint32_t)a.n_kv_heads + (uint32_t)kh) * rec256;
      }
    }
  } else {
    for (int j = tid; j < nbq; j += kThreads) {
      bad_page |= (uint32_t)bt[j >> a.bt_shift] >= (uint32_t)a.num_pages;   // -1 (unmapped) included
      sm.boff[j] = (record_slot(bt, j, a.bt_shift) * (uint32_t)a.n_kv_heads + (uint32_t)kh) * rec256;
    }
  }
  for (int d = tid; d < D; d += kThreads) {
    const size_t qi = orow * D + d;
    const float qv = a.q_bf16 ? bf16f(reinterpret_cast<const uint16_t*>(a.q)[qi]) : reinterpret_cast<const float*>(a.q)[qi];
    sm.qs[d] = a.sm_scale * qv;
  }
  // OR of the page check over the workgroup: one flag per wave in the exchange words (written
  // again only after the row body's first barrier)
  const bool wave_bad = __any(bad_page);   // every lane of the wave votes
  if ((tid & 63) == 0) sm.misc[tid >> 6] = wave_bad ? 1.f : 0.f;
  __syncthreads();
  bool any_bad = false;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) any_bad |= sm.misc[i] != 0.f;
  if (any_bad) {   // no record of this row is read
    if (PH == PH_PART && tid == 0) a.part[(orow * (size_t)a.n_split + split) * (2 + D)] = __builtin_nanf("");
    empty_row(false);
    return;
  }

  if constexpr (VAR == VAR_KIVI) {
    row_body<D, GS, MODE_KIVI, false, PH>(a, r, sm, orow, split, fin);
  } else {
    if (cell.kind == KIND_Q2) row_body<D, GS, MODE_Q2, false, PH>(a, r, sm, orow, split, fin);
    else if (VAR == VAR_DENSE) row_body<D, GS, MODE_DENSE, false, PH>(a, r, sm, orow, split, fin);
    else if (VAR == VAR_COARSE) row_body<D, GS, MODE_COARSE, false, PH>(a, r, sm, orow, split, fin);
    else if (VAR == VAR_SKIP) row_body<D, GS, MODE_COARSE, true, PH, true>(a, r, sm, orow, split, fin);
    else row_body<D, GS, MODE_COARSE, true, PH>(a, r, sm, orow, split, fin);
  }
}

// Two objects are built from this file: records addressed with 32-bit offsets (pools below
// 4 GiB) and with 64-bit ones (LKV_DECODE_BIG=1); the host picks one per context.
#ifndef LKV_DECODE_BIG
#define LKV_DECODE_BIG 0
#endif
constexpr bool kBig = LKV_DECODE_BIG != 0;

#if !LKV_DECODE_BIG
size_t decode_lds_bytes(int max_len, int head_dim) { return decode_lds_floats(max_len, head_dim) * 4; }
#endif

template <int D, int GS, int VAR, int PH>
static void set_lds_attr() {
  static bool attr_set = false;
  if (!attr_set) {
    (void)hipFuncSetAttribute((const void*)k_decode<D, GS, VAR, PH, kBig>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    attr_set = true;
  }
}

template <int D, int GS, int VAR, int PH>
static void launch_phase(const DecodeArgs& a, size_t grid, size_t lds, hipStream_t stream) {
  set_lds_attr<D, GS, VAR, PH>();
  hipLaunchKernelGGL((k_decode<D, GS, VAR, PH, kBig>), dim3((unsigned)grid), dim3(kThreads), lds, stream, a);
}

// Sets the LDS attribute of every decode kernel of a shape, so that a graph capture that
// follows makes no attribute call.
template <int D, int GS>
static void prepare_dg() {
  set_lds_attr<D, GS, VAR_SKIP, PH_ROW>();
  set_lds_attr<D, GS, VAR_KIVI, PH_ROW>();
  set_lds_attr<D, GS, VAR_KIVI, PH_PART>();
  set_lds_attr<D, GS, VAR_KIVI, PH_FINISH>();
  set_lds_attr<D, GS, VAR_DENSE, PH_ROW>();
  set_lds_attr<D, GS, VAR_DENSE, PH_PART>();
  set_lds_attr<D, GS, VAR_DENSE, PH_FINISH>();
  set_lds_attr<D, GS, VAR_COARSE, PH_ROW>();
  set_lds_attr<D, GS, VAR_COARSE, PH_PART>();
  set_lds_attr<D, GS, VAR_COARSE, PH_FINISH>();
  set_lds_attr<D, GS, VAR_SPARSE, PH_ROW>();
  set_lds_attr<D, GS, VAR_SPARSE, PH_PART>();
  set_lds_attr<D, GS, VAR_SPARSE, PH_FINISH>();
}

template <int D>
static void prepare_d(int group) {
  if (group == 64) prepare_dg<D, 64>();
  else prepare_dg<D, 32>();
}

#if LKV_DECODE_BIG
void prepare_decode_big(int head_dim, int group) {
#else
void prepare_decode_small(int head_dim, int group) {
#endif
  if (head_dim == 128) prepare_d<128>(group);
  else if (head_dim == 256) prepare_d<256>(group);
  else prepare_d<64>(group);
}

// Grid of a one-workgroup-per-row launch: with grouped queries the rows of 8 KV heads form
// one span of 8 G block indices (see k_decode), padded to whole spans.
static size_t row_grid(const DecodeArgs& a, size_t rows) {
  const int G = a.n_heads / a.n_kv_heads;
  if (G == 1) return rows;
  const size_t groups = rows / G;
  return (groups + 7) / 8 * 8 * (size_t)G;
}

template <int D, int GS, int VAR>
static void launch_variant(const DecodeArgs& a, size_t rows, size_t lds, hipStream_t stream) {
  if constexpr (VAR == VAR_SKIP) {   // one workgroup per row only (the host refuses a split)
    launch_phase<D, GS, VAR, PH_ROW>(a, row_grid(a, rows), lds, stream);
  } else if (a.n_split < 1) {
    launch_phase<D, GS, VAR, PH_ROW>(a, row_grid(a, rows), lds, stream);
  } else {   // stream order: every partial is written before the finishing launch reads it
    launch_phase<D, GS, VAR, PH_PART>(a, rows * (size_t)a.n_split, lds, stream);
    launch_phase<D, GS, VAR, PH_FINISH>(a, rows, finish_lds_floats(a.max_len, D, a.n_split) * 4, stream);
  }
}

template <int D, int GS>
static void launch_dg(const DecodeArgs& a, size_t rows, size_t lds, hipStream_t stream) {
  if (a.cells[0].kind == KIND_KIVI4) launch_variant<D, GS, VAR_KIVI>(a, rows, lds, stream);
  else if (a.tau <= 0.f) launch_variant<D, GS, VAR_DENSE>(a, rows, lds, stream);   // everything kept
  else if (a.skip) launch_variant<D, GS, VAR_SKIP>(a, rows, lds, stream);
  else if (a.tau > 1.f) launch_variant<D, GS, VAR_COARSE>(a, rows, lds, stream);
  else launch_variant<D, GS, VAR_SPARSE>(a, rows, lds, stream);
}

template <int D>
static void launch_d(const DecodeArgs& a, size_t rows, size_t lds, hipStream_t stream) {
  if (a.group == 64) launch_dg<D, 64>(a, rows, lds, stream);
  else launch_dg<D, 32>(a, rows, lds, stream);
}

#if LKV_DECODE_BIG
hipError_t launch_decode_big(const DecodeArgs& a, int head_dim, hipStream_t stream) {
#else
hipError_t launch_decode_small(const DecodeArgs& a, int head_dim, hipStream_t stream) {
#endif
  const size_t rows = (size_t)a.n_cells * a.n_seqs * a.n_heads;
  if (rows == 0) return hipSuccess;
  size_t lds = decode_lds_floats(a.max_len, head_dim) * 4;
  if (a.app_k) lds = lds > fused_append_lds_bytes(head_dim, a.group) ? lds : fused_append_lds_bytes(head_dim, a.group);
  if (head_dim == 128) launch_d<128>(a, rows, lds, stream);
  else if (head_dim == 256) launch_d<256>(a, rows, lds, stream);
  else launch_d<64>(a, rows, lds, stream);
  return hipGetLastError();
}

}  // namespace lkv
