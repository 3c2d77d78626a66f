// Append and group quantization of the per-(loop, layer) KV cache (gfx950).
//
// Source: "LoopKV: Loop-Aware KV Cache Compression for Serving Looped
// Transformers" (arXiv:2611.04137), Abstract — every cell is stored as 4-bit
// (KIVI-4 style) or 2-bit, and decoding reads the high 2 bits of each 4-bit
// value apart from its low bits, so 4-bit codes are split into a high and a
// low 2-bit plane here.
//
// Quantizer (KIVI-style asymmetric groups of GS = 32, or 64): K per channel over GS
// consecutive tokens, V per token over GS consecutive channels;
// zero = f16(min), scale = f16((max - min) / (2^b - 1)),
// code = clamp(rint((x - zero) / scale), 0, 2^b - 1), scale 0 -> code 0.
// All of it in float64 with one round-to-nearest-even to f16, so codes and
// meta are reproducible bit for bit. Built with -ffp-contract=off.
//
// Appends of fewer than GS tokens per sequence (decode time) take one kernel:
//   k_quantize_groups<D, GS, true>  one workgroup per (head, cell x sequence): reads the
//                      old tail of the group this append completes (if any) into LDS,
//                      writes the new tokens that stay in the tail once every read of
//                      the old tail is done, then quantizes the completed group and
//                      writes the records of its GS / 16 blocks through the block table.
// Longer appends (a prefill) take two, on the caller's stream:
//   k_quantize_groups<D, GS, false> one workgroup per (group slot, head, cell x sequence):
//                      gathers the GS tokens of a group completed by this append
//                      (old tail + new input), quantizes, writes its records;
//   k_write_tail       copies the new tokens of the last, incomplete group into
//                      the tail (after the first kernel has read the old tail).
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

__device__ inline float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);   // NaN stays NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Quantize n values read through get(i) with M = 2^bits - 1 levels.
template <typename Get>
__device__ inline void quantize_group(Get get, int n, int M, uint8_t* codes, int stride, uint32_t* meta) {
  double mn = get(0), mx = mn;
  for (int i = 1; i < n; ++i) {
    double x = get(i);
    mn = fmin(mn, x);
    mx = fmax(mx, x);
  }
  uint32_t zb = f64_to_f16_bits(mn);
  uint32_t sb = f64_to_f16_bits((mx - mn) / (double)M);
  double z = f16_bits_to_f64(zb);
  double s = f16_bits_to_f64(sb);
  for (int i = 0; i < n; ++i) {
    int c = 0;
    if (s != 0.0) {
      double r = rint((get(i) - z) / s);
      r = fmin(fmax(r, 0.0), (double)M);
      c = (int)r;
    }
    codes[i * stride] = (uint8_t)c;
  }
  *meta = sb | (zb << 16);
}

// Channel stored at K-meta position i: the words of a K column follow the column's
// bit layout (2-bit: byte k, bit pair p; 4-bit: byte k, nibble n).
__device__ inline int kmeta_channel2(int i) { return (i & ~15) + 4 * (i & 3) + ((i >> 2) & 3); }
__device__ inline int kmeta_channel4(int i) { return (i & ~7) + 2 * (i & 3) + ((i >> 2) & 1); }

// The new tokens of (cell ci, sequence b, head h) that stay in the tail (those after the
// last group the append completes), rounded from f32 if needed.
template <int D, int GS>
__device__ void write_tail_tokens(const AppendArgs& a, const AppendCell& cell, int b, int h, int L0) {
  const int end = L0 + a.n_new;
  const int first = max(L0, (end / GS) * GS);   // first position that stays in the tail
  const int cnt = end - first;
  if (cnt <= 0) return;
  const int slot = a.seq_slots ? a.seq_slots[b] : b;
  if (L0 < 0 || (uint32_t)slot >= (uint32_t)a.max_seqs) return;   // invalid sequence: nothing written
  uint16_t* tail = reinterpret_cast<uint16_t*>(a.ws + cell.tail_off) + ((size_t)slot * a.n_heads + h) * tail_elems(D, GS);
  for (int idx = threadIdx.x; idx < cnt * D; idx += blockDim.x) {
    const int i = idx / D, d = idx % D;
    const int p = first + i;
    const size_t e = ((((size_t)cell.in_cell * a.n_seqs + b) * a.n_new + (p - L0)) * a.n_heads + h) * D + d;
    uint16_t kb, vb;
    if (a.kv_bf16) {
      kb = reinterpret_cast<const uint16_t*>(a.k)[e];
      vb = reinterpret_cast<const uint16_t*>(a.v)[e];
    } else {
      kb = f32_to_bf16_rne(reinterpret_cast<const float*>(a.k)[e]);
      vb = f32_to_bf16_rne(reinterpret_cast<const float*>(a.v)[e]);
    }
    tail[(0 * GS + (p % GS)) * D + d] = kb;
    tail[(1 * GS + (p % GS)) * D + d] = vb;
  }
}

// WITH_TAIL: the one-kernel append of fewer than GS tokens (grid x = 1).
template <int D, int GS, bool WITH_TAIL>
__global__ void __launch_bounds__(256) k_quantize_groups(AppendArgs a) {
  const int b = blockIdx.z % a.n_seqs;
  const int ci = blockIdx.z / a.n_seqs;
  const int h = blockIdx.y;
  const AppendCell cell = a.cells[ci];
  const int L0 = a.seq_lens[b];
  const int g = L0 / GS + (int)blockIdx.x;
  const bool complete = (g + 1) * GS <= L0 + a.n_new;   // uniform over the workgroup
  if (!WITH_TAIL && !complete) return;
  const int slot = a.seq_slots ? a.seq_slots[b] : b;
  if (L0 < 0 || (uint32_t)slot >= (uint32_t)a.max_seqs) return;   // invalid sequence (uniform): nothing written
  const int tid = threadIdx.x;
  constexpr int P = GS / kBlock;   // records per group

  __shared__ uint16_t kx[GS][D];   // bf16 bits of the group's GS tokens (exact values)
  __shared__ uint16_t vx[GS][D];
  __shared__ uint8_t kc[GS][D];
  __shared__ uint8_t vc[GS][D];
  __shared__ uint32_t kmeta[D];
  __shared__ uint32_t vmeta[GS][D / GS];

  const uint16_t* tail = reinterpret_cast<const uint16_t*>(a.ws + cell.tail_off) +
                         ((size_t)slot * a.n_heads + h) * tail_elems(D, GS);
  for (int idx = tid; complete && idx < GS * D; idx += blockDim.x) {
    const int i = idx / D, d = idx % D;
    const int p = g * GS + i;
    uint16_t kb, vb;
    if (p < L0) {
      kb = tail[(0 * GS + (p % GS)) * D + d];
      vb = tail[(1 * GS + (p % GS)) * D + d];
    } else {
      const size_t e = ((((size_t)cell.in_cell * a.n_seqs + b) * a.n_new + (p - L0)) * a.n_heads + h) * D + d;
      if (a.kv_bf16) {
        kb = reinterpret_cast<const uint16_t*>(a.k)[e];
        vb = reinterpret_cast<const uint16_t*>(a.v)[e];
      } else {
        kb = f32_to_bf16_rne(reinterpret_cast<const float*>(a.k)[e]);
        vb = f32_to_bf16_rne(reinterpret_cast<const float*>(a.v)[e]);
      }
    }
    kx[i][d] = kb;
    vx[i][d] = vb;
  }
  __syncthreads();
  if constexpr (WITH_TAIL) {   // every read of the old tail is done (barrier above)
    write_tail_tokens<D, GS>(a, cell, b, h, L0);
    if (!complete) return;
  }

  const int M = (cell.kind == KIND_Q2) ? 3 : 15;
  // K: one group per channel over the GS tokens.
  for (int d = tid; d < D; d += blockDim.x)
    quantize_group([&](int i) { return (double)bf16_to_f32(kx[i][d]); }, GS, M, &kc[0][d], D, &kmeta[d]);
  // V: one group per token over each run of GS channels.
  for (int task = tid; task < GS * (D / GS); task += blockDim.x) {
    const int i = task / (D / GS), e = task % (D / GS);
    quantize_group([&](int j) { return (double)bf16_to_f32(vx[i][e * GS + j]); }, GS, M, &vc[i][e * GS], 1,
                   &vmeta[i][e]);
  }
  __syncthreads();

  // The group's P records: record P g + part holds tokens 16 part .. 16 part + 15 and the
  // K-meta positions part D / P .. (part + 1) D / P - 1.
  const int rec = record_bytes(cell.kind, D, GS);
  for (int part = 0; part < P; ++part) {
    const int j = P * g + part;
    const int32_t* bt = a.block_table + (size_t)b * a.bt_stride;
    if ((j >> a.bt_shift) >= a.bt_stride || (uint32_t)bt[j >> a.bt_shift] >= (uint32_t)a.num_pages)
      continue;   // page not mapped (uniform over the workgroup): the record is not written
    const uint32_t phys = record_slot(bt, j, a.bt_shift);
    uint32_t* r = reinterpret_cast<uint32_t*>(a.ws + cell.pool_off + ((size_t)phys * a.n_heads + h) * rec);
    const int t0 = part * kBlock;
    if (cell.kind == KIND_KIVI4) {
      // K4: D/8 columns x 16 tokens; V4: D channels x 2 words.
      for (int idx = tid; idx < (D / 8) * kBlock; idx += blockDim.x) {
        const int w = idx / kBlock, t = idx % kBlock;
        uint32_t word = 0;
        for (int c = 0; c < 8; ++c) word |= (uint32_t)kc[t0 + t][8 * w + c] << (4 * c);
        r[idx] = word;
      }
      for (int idx = tid; idx < D * 2; idx += blockDim.x) {
        const int d = idx / 2, jj = idx % 2;
        uint32_t word = 0;
        for (int tp = 0; tp < 8; ++tp) word |= (uint32_t)vc[t0 + 8 * jj + tp][d] << (8 * (tp % 4) + 4 * (tp / 4));
        r[off_v_kivi(D, GS) / 4 + idx] = word;
      }
      for (int c = tid; c < D / P; c += blockDim.x) r[off_kmeta_kivi(D) / 4 + c] = kmeta[kmeta_channel4(part * (D / P) + c)];
      for (int idx = tid; idx < kBlock * (D / GS); idx += blockDim.x)
        r[off_vmeta_kivi(D, GS) / 4 + idx] = vmeta[t0 + idx % kBlock][idx / kBlock];
    } else {
      const bool q4 = cell.kind == KIND_Q4;
      // K planes: D/16 columns x 16 tokens.
      for (int idx = tid; idx < (D / 16) * kBlock; idx += blockDim.x) {
        const int w = idx / kBlock, t = idx % kBlock;
        uint32_t hi = 0, lo = 0;
        for (int c = 0; c < 16; ++c) {
          const uint32_t code = kc[t0 + t][16 * w + c];
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
      for (int d = tid; d < D; d += blockDim.x) {
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
        r[off_v_planes(D, GS) / 4 + d] = hi;
        if (q4) r[off_vlo(D, GS) / 4 + d] = lo;
      }
      for (int c = tid; c < D / P; c += blockDim.x) r[off_kmeta_planes(D) / 4 + c] = kmeta[kmeta_channel2(part * (D / P) + c)];
      for (int idx = tid; idx < kBlock * (D / GS); idx += blockDim.x)
        r[off_vmeta_planes(D, GS) / 4 + idx] = vmeta[t0 + idx % kBlock][idx / kBlock];
    }
  }
}

template <int D, int GS>
__global__ void __launch_bounds__(256) k_write_tail(AppendArgs a) {
  const int b = blockIdx.z % a.n_seqs;
  const int ci = blockIdx.z / a.n_seqs;
  write_tail_tokens<D, GS>(a, a.cells[ci], b, blockIdx.y, a.seq_lens[b]);
}

template <int D, int GS>
static void launch_dg(const AppendArgs& a, hipStream_t stream) {
  if (a.n_new < GS) {   // at most one group per (sequence, head) completes: one kernel
    hipLaunchKernelGGL((k_quantize_groups<D, GS, true>), dim3(1, a.n_heads, a.n_cells * a.n_seqs), dim3(256), 0,
                       stream, a);
    return;
  }
  const int slots = a.n_new / GS + 1;   // groups one append can complete
  hipLaunchKernelGGL((k_quantize_groups<D, GS, false>), dim3(slots, a.n_heads, a.n_cells * a.n_seqs), dim3(256), 0,
                     stream, a);
  hipLaunchKernelGGL((k_write_tail<D, GS>), dim3(1, a.n_heads, a.n_cells * a.n_seqs), dim3(256), 0, stream, a);
}

template <int D>
static void launch_d(const AppendArgs& a, hipStream_t stream) {
  if (a.group == 64) launch_dg<D, 64>(a, stream);
  else launch_dg<D, 32>(a, stream);
}

// End of a serving step: every sequence's lengths before and after the step's token advance
// by one (the arrays are distinct).
__global__ void __launch_bounds__(256) k_advance_lens(int32_t* before, int32_t* after, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) {
    before[i] += 1;
    after[i] += 1;
  }
}

hipError_t launch_advance_lens(int32_t* before, int32_t* after, int n, hipStream_t stream) {
  hipLaunchKernelGGL(k_advance_lens, dim3((n + 255) / 256), dim3(256), 0, stream, before, after, n);
  return hipGetLastError();
}

// Host launcher: quantize completed groups, then update tails (same stream).
hipError_t launch_append(const AppendArgs& a, int head_dim, hipStream_t stream) {
  if (a.n_cells == 0 || a.n_seqs == 0 || a.n_new == 0) return hipSuccess;
  if (head_dim == 128) launch_d<128>(a, stream);
  else if (head_dim == 256) launch_d<256>(a, stream);
  else launch_d<64>(a, stream);
  return hipGetLastError();
}

}  // namespace lkv
