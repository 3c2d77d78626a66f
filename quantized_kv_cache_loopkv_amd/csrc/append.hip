// Append and group quantization of the per-(loop, layer) KV cache (gfx950).
//
// Source: "LoopKV: Loop-Aware KV Cache Compression for Serving Looped
// Transformers" (arXiv:2611.04137), Abstract — every cell is stored as 4-bit
// (KIVI-4 style) or 2-bit, and a decoding loop can read the upper half of a 4-bit
// code without its lower half, so 4-bit codes are split into a high and a low
// 2-bit plane here.
//
// Quantizer (KIVI-style asymmetric groups of GS = 32, or 64): K per channel over GS
// consecutive tokens, V per token over GS consecutive channels;
// zero = f16(min), scale = f16((max - min) / (2^b - 1)),
// code = clamp(rint((x - zero) / scale), 0, 2^b - 1), scale 0 -> code 0.
// All of it in float64 with one round-to-nearest-even to f16, so codes and
// meta are reproducible bit for bit. Built with -ffp-contract=off.
//
// The one-token append of a decode step takes one kernel:
//   k_append_token<D, GS>  one workgroup per (cell, sequence, four KV heads): the token goes
//                      to its tail slot unless it completes a group, whose GS / 16 records
//                      the workgroup then quantizes and writes head by head.
// Other appends of fewer than GS tokens per sequence take one kernel:
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
#include "quantize.h"

namespace lkv {

constexpr int kAppendThreads = 256;   // workgroup size of every append kernel
constexpr int kQuantStep = 4;         // elements per quantizer loop step (their latencies overlap)
constexpr int kTokenHeads = 4;        // KV heads per workgroup of the one-token append

// Fills kx / vx (bf16 bits [GS][D] in LDS) with the GS tokens of a group: element (i, d) from
// value(i, d, is_k). Each thread takes the elements tid, tid + 256, ... and requests 16 of them
// (K and V) before it stores any, so the group costs one or a few memory round trips instead
// of one per element (the loads would otherwise wait on each other through the LDS stores).
template <int D, int GS, class Val>
__device__ inline void gather_group(uint16_t (*kx)[D], uint16_t (*vx)[D], int tid, Val value) {
  constexpr int PER = GS * D / kAppendThreads;   // 8 .. 64
  constexpr int CH = PER < 16 ? PER : 16;
  static_assert(PER % CH == 0, "gather batches");
#pragma unroll 1
  for (int k0 = 0; k0 < PER; k0 += CH) {
    uint16_t kv[CH], vv[CH];
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      const int idx = (k0 + k) * kAppendThreads + tid;
      kv[k] = value(idx / D, idx % D, true);
      vv[k] = value(idx / D, idx % D, false);
    }
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      const int idx = (k0 + k) * kAppendThreads + tid;
      kx[idx / D][idx % D] = kv[k];
      vx[idx / D][idx % D] = vv[k];
    }
  }
}

// Rows r0 .. r0 + n - 1 of kx / vx (bf16, D channels) from K rows at ksrc + r stride and V rows
// at vsrc + r stride (r = 0 .. n - 1; every row and both sources 16-byte aligned): 16-byte loads,
// two K and two V per thread requested before any is stored (named registers: an array here
// ends up in scratch memory).
template <int D, int GS>
__device__ inline void copy_rows16(uint16_t (*kx)[D], uint16_t (*vx)[D], int r0, int n, const uint16_t* ksrc,
                                   const uint16_t* vsrc, size_t stride, int tid) {
  constexpr int C8 = D / 8;   // 16-byte chunks per row
  const int total = n * C8;
  auto src = [&](int c) { return (size_t)(c / C8) * stride + 8 * (c % C8); };
#pragma unroll 1
  for (int c0 = tid; c0 < total; c0 += 2 * kAppendThreads) {
    const int c1 = c0 + kAppendThreads;
    const uint4 k0 = *reinterpret_cast<const uint4*>(ksrc + src(c0));
    const uint4 v0 = *reinterpret_cast<const uint4*>(vsrc + src(c0));
    uint4 k1 = k0, v1 = v0;
    if (c1 < total) {
      k1 = *reinterpret_cast<const uint4*>(ksrc + src(c1));
      v1 = *reinterpret_cast<const uint4*>(vsrc + src(c1));
    }
    *reinterpret_cast<uint4*>(&kx[r0 + c0 / C8][8 * (c0 % C8)]) = k0;
    *reinterpret_cast<uint4*>(&vx[r0 + c0 / C8][8 * (c0 % C8)]) = v0;
    if (c1 < total) {
      *reinterpret_cast<uint4*>(&kx[r0 + c1 / C8][8 * (c1 % C8)]) = k1;
      *reinterpret_cast<uint4*>(&vx[r0 + c1 / C8][8 * (c1 % C8)]) = v1;
    }
  }
}

// bf16 inputs whose K and V tensors start on 16-byte boundaries (rows of D channels then are
// too) take the 16-byte gathers; others the element-wise ones.
__device__ inline bool rows16_ok(const AppendArgs& a) {
  return a.kv_bf16 && ((reinterpret_cast<uintptr_t>(a.k) | reinterpret_cast<uintptr_t>(a.v)) & 15u) == 0;
}

// Codes and meta of the group in kx / vx: the D K groups (one per channel, over the GS tokens)
// and the GS * D / GS V groups (one per token and run of GS channels) form one task list over
// the workgroup's threads, so the K and V groups run side by side; kQuantStep elements per
// loop step and V groups at rotated starting elements (vgroup_rot). Each group is
// quantize_group's, as in quantize_group_codes.
template <int D, int GS>
__device__ inline void quantize_tasks(const uint16_t (*kx)[D], const uint16_t (*vx)[D], int M, uint8_t (*kc)[D],
                                      uint8_t (*vc)[D], uint32_t* kmeta, uint32_t (*vmeta)[D / GS], int tid) {
  constexpr int NV = GS * (D / GS);
  for (int task = tid; task < D + NV; task += kAppendThreads) {
    if (task < D) {
      const int d = task;
      quantize_group<kQuantStep>([&](int i) { return (double)bf16_bits_to_f32(kx[i][d]); }, GS, M, &kc[0][d], D,
                                 &kmeta[d]);
    } else {
      const int i = (task - D) / (D / GS), e = (task - D) % (D / GS);
      quantize_group<kQuantStep>([&](int j) { return (double)bf16_bits_to_f32(vx[i][e * GS + j]); }, GS, M,
                                 &vc[i][e * GS], 1, &vmeta[i][e], vgroup_rot<GS>(task - D));
    }
  }
}

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
__global__ void __launch_bounds__(kAppendThreads) k_quantize_groups(AppendArgs a) {
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

  __shared__ __align__(16) uint16_t kx[GS][D];   // bf16 bits of the group's GS tokens (exact values)
  __shared__ __align__(16) uint16_t vx[GS][D];
  __shared__ __align__(16) uint8_t kc[GS][D];   // rows read as 32-bit words by the packer
  __shared__ uint8_t vc[GS][D];
  __shared__ uint32_t kmeta[D];
  __shared__ uint32_t vmeta[GS][D / GS];

  const uint16_t* tail = reinterpret_cast<const uint16_t*>(a.ws + cell.tail_off) +
                         ((size_t)slot * a.n_heads + h) * tail_elems(D, GS);
  if (complete && g * GS >= L0 && rows16_ok(a)) {   // the whole group comes from the input
    const size_t row0 = (((size_t)cell.in_cell * a.n_seqs + b) * a.n_new + (size_t)(g * GS - L0)) * a.n_heads + h;
    copy_rows16<D, GS>(kx, vx, 0, GS, reinterpret_cast<const uint16_t*>(a.k) + row0 * D,
                       reinterpret_cast<const uint16_t*>(a.v) + row0 * D, (size_t)a.n_heads * D, tid);
  } else if (complete) {
    gather_group<D, GS>(kx, vx, tid, [&](int i, int d, bool is_k) -> uint16_t {
      const int p = g * GS + i;
      if (p < L0) return tail[((is_k ? 0 : GS) + (p % GS)) * D + d];
      const size_t e = ((((size_t)cell.in_cell * a.n_seqs + b) * a.n_new + (p - L0)) * a.n_heads + h) * D + d;
      const void* src = is_k ? a.k : a.v;
      return a.kv_bf16 ? reinterpret_cast<const uint16_t*>(src)[e]
                       : f32_to_bf16_rne(reinterpret_cast<const float*>(src)[e]);
    });
  }
  __syncthreads();
  if constexpr (WITH_TAIL) {   // every read of the old tail is done (barrier above)
    write_tail_tokens<D, GS>(a, cell, b, h, L0);
    if (!complete) return;
  }

  const int M = (cell.kind == KIND_Q2) ? 3 : 15;
  // K: one group per channel over the GS tokens; V: one group per token over each run of GS
  // channels.
  quantize_tasks<D, GS>(kx, vx, M, kc, vc, kmeta, vmeta, tid);
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
    pack_record<D, GS>(r, cell.kind, part, kc, vc, kmeta, vmeta, tid, (int)blockDim.x);
  }
}

// Waves per SIMD the one-token append asks the register allocator for: its workgroups' LDS
// (the group staging of k_append_token) allows floor(160 KB / LDS) of them per CU, each one wave
// per SIMD; at most four, three for groups of 64 (their gathers need more registers).
constexpr int append_token_waves(int D, int GS) {
  const int lds = GS * D * 2 * 2 + GS * D * 2 + 4 * D + 4 * GS * (D / GS);
  const int per_cu = 160 * 1024 / lds;
  const int cap = GS == 64 ? 3 : 4;
  return per_cu < 1 ? 1 : per_cu > cap ? cap : per_cu;
}

// The one-token append (n_new = 1) of (cell ci, sequence b) for kTokenHeads of its heads (the
// heads of a sequence whose token completes a group are quantized in turn, so with fewer heads
// per workgroup a step where only some sequences complete a group ends sooner). The
// token's K and V are requested together with the sequence's length (their addresses do not
// depend on it), so a step that completes no group costs one memory round trip; the token
// goes to tail slot L0 mod GS. When it completes group g = L0 / GS it stays out of the tail,
// and the group of each head in turn (GS - 1 tokens from the tail, the new one from the
// input) is quantized and packed exactly as in k_quantize_groups. Records, tails and the
// skipped cases (invalid sequence, unmapped page) are those of k_quantize_groups<D, GS, true>.
template <int D, int GS>
__global__ void __launch_bounds__(kAppendThreads, append_token_waves(D, GS)) k_append_token(AppendArgs a) {
  const int n_hs = (a.n_heads + kTokenHeads - 1) / kTokenHeads;   // head slices per sequence
  const int hs = blockIdx.x % n_hs;
  const int b = (blockIdx.x / n_hs) % a.n_seqs;
  const int ci = blockIdx.x / n_hs / a.n_seqs;
  const AppendCell cell = a.cells[ci];
  const int tid = threadIdx.x;
  const int h0 = hs * kTokenHeads, h1 = min(a.n_heads, h0 + kTokenHeads);   // this workgroup's heads
  const int HD = (h1 - h0) * D;
  // [cells][n_seqs][1][heads][D], from head h0
  const size_t e0 = ((size_t)cell.in_cell * a.n_seqs + b) * a.n_heads * D + (size_t)h0 * D;
  auto new_bits = [&](const void* src, size_t e) -> uint16_t {
    return a.kv_bf16 ? reinterpret_cast<const uint16_t*>(src)[e]
                     : f32_to_bf16_rne(reinterpret_cast<const float*>(src)[e]);
  };
  const int L0 = a.seq_lens[b];
  const int slot = a.seq_slots ? a.seq_slots[b] : b;
  const bool valid = L0 >= 0 && (uint32_t)slot < (uint32_t)a.max_seqs;   // uniform
  const bool complete = valid && (L0 + 1) % GS == 0;
  uint16_t* tail0 = reinterpret_cast<uint16_t*>(a.ws + cell.tail_off) +
                   ((size_t)(valid ? slot : 0) * a.n_heads + h0) * tail_elems(D, GS);   // head h0's tail
  const int pos = valid ? L0 % GS : 0;
  if (rows16_ok(a)) {   // 16-byte chunks of the token (8 channels of one head; tails are 16-byte aligned)
    constexpr int C8 = D / 8;
    const uint16_t* k16 = reinterpret_cast<const uint16_t*>(a.k) + e0;
    const uint16_t* v16 = reinterpret_cast<const uint16_t*>(a.v) + e0;
#pragma unroll 1
    for (int c = tid; c < HD / 8; c += kAppendThreads) {
      const uint4 kq = *reinterpret_cast<const uint4*>(k16 + 8 * c);
      const uint4 vq = *reinterpret_cast<const uint4*>(v16 + 8 * c);
      if (!valid || complete) break;   // uniform: nothing, or the records below
      uint16_t* th = tail0 + (size_t)(c / C8) * tail_elems(D, GS) + 8 * (c % C8);
      *reinterpret_cast<uint4*>(th + (size_t)pos * D) = kq;
      *reinterpret_cast<uint4*>(th + (size_t)(GS + pos) * D) = vq;
    }
  } else {
    for (int base = 0; base < HD; base += 8 * kAppendThreads) {
      uint16_t kb[8], vb[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int idx = base + u * kAppendThreads + tid;
        kb[u] = idx < HD ? new_bits(a.k, e0 + idx) : 0;
        vb[u] = idx < HD ? new_bits(a.v, e0 + idx) : 0;
      }
      if (!valid || complete) break;   // uniform: nothing, or the records below
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int idx = base + u * kAppendThreads + tid;
        if (idx >= HD) continue;
        uint16_t* th = tail0 + (size_t)(idx / D) * tail_elems(D, GS);
        th[(0 * GS + pos) * D + idx % D] = kb[u];
        th[(1 * GS + pos) * D + idx % D] = vb[u];
      }
    }
  }
  if (!complete) return;

  constexpr int P = GS / kBlock;   // records per group
  __shared__ __align__(16) uint16_t kx[GS][D];
  __shared__ __align__(16) uint16_t vx[GS][D];
  __shared__ __align__(16) uint8_t kc[GS][D];   // rows read as 32-bit words by the packer
  __shared__ uint8_t vc[GS][D];
  __shared__ uint32_t kmeta[D];
  __shared__ uint32_t vmeta[GS][D / GS];
  const int g = L0 / GS;
  const int M = (cell.kind == KIND_Q2) ? 3 : 15;
  const int rec = record_bytes(cell.kind, D, GS);
  const int32_t* bt = a.block_table + (size_t)b * a.bt_stride;
  for (int h = h0; h < h1; ++h) {
    const uint16_t* th = tail0 + (size_t)(h - h0) * tail_elems(D, GS);
    // positions g GS .. L0 - 1 sit in tail slots 0 .. GS - 2; the new token is the input's
    if (rows16_ok(a)) {   // tail rows and the input row with 16-byte loads (tails are 16-byte aligned)
      copy_rows16<D, GS>(kx, vx, 0, GS - 1, th, th + (size_t)GS * D, D, tid);
      copy_rows16<D, GS>(kx, vx, GS - 1, 1, reinterpret_cast<const uint16_t*>(a.k) + e0 + (size_t)(h - h0) * D,
                         reinterpret_cast<const uint16_t*>(a.v) + e0 + (size_t)(h - h0) * D, D, tid);
    } else {
      gather_group<D, GS>(kx, vx, tid, [&](int i, int d, bool is_k) -> uint16_t {
        return i < GS - 1 ? th[((is_k ? 0 : GS) + i) * D + d] : new_bits(is_k ? a.k : a.v, e0 + (size_t)(h - h0) * D + d);
      });
    }
    __syncthreads();
    quantize_tasks<D, GS>(kx, vx, M, kc, vc, kmeta, vmeta, tid);
    __syncthreads();
    for (int part = 0; part < P; ++part) {
      const int j = P * g + part;
      if ((j >> a.bt_shift) >= a.bt_stride || (uint32_t)bt[j >> a.bt_shift] >= (uint32_t)a.num_pages)
        continue;   // page not mapped (uniform over the workgroup): the record is not written
      const uint32_t phys = record_slot(bt, j, a.bt_shift);
      uint32_t* r = reinterpret_cast<uint32_t*>(a.ws + cell.pool_off + ((size_t)phys * a.n_heads + h) * rec);
      pack_record<D, GS>(r, cell.kind, part, kc, vc, kmeta, vmeta, tid, kAppendThreads);
    }
    __syncthreads();   // the group's LDS is reused for the next head
  }
}

template <int D, int GS>
__global__ void __launch_bounds__(kAppendThreads) k_write_tail(AppendArgs a) {
  const int b = blockIdx.z % a.n_seqs;
  const int ci = blockIdx.z / a.n_seqs;
  write_tail_tokens<D, GS>(a, a.cells[ci], b, blockIdx.y, a.seq_lens[b]);
}

template <int D, int GS>
static void launch_dg(const AppendArgs& a, hipStream_t stream) {
  if (a.n_new == 1) {   // a decode step's token: one workgroup per (cell, sequence, kTokenHeads heads)
    const int n_hs = (a.n_heads + kTokenHeads - 1) / kTokenHeads;
    hipLaunchKernelGGL((k_append_token<D, GS>), dim3(a.n_cells * a.n_seqs * n_hs), dim3(kAppendThreads), 0, stream,
                       a);
    return;
  }
  if (a.n_new < GS) {   // at most one group per (sequence, head) completes: one kernel
    hipLaunchKernelGGL((k_quantize_groups<D, GS, true>), dim3(1, a.n_heads, a.n_cells * a.n_seqs), dim3(kAppendThreads), 0,
                       stream, a);
    return;
  }
  const int slots = a.n_new / GS + 1;   // groups one append can complete
  hipLaunchKernelGGL((k_quantize_groups<D, GS, false>), dim3(slots, a.n_heads, a.n_cells * a.n_seqs), dim3(kAppendThreads), 0,
                     stream, a);
  hipLaunchKernelGGL((k_write_tail<D, GS>), dim3(1, a.n_heads, a.n_cells * a.n_seqs), dim3(kAppendThreads), 0, stream, a);
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
