// Record layout, kinds and launch descriptors shared by the host runtime and the kernels.
//
// Storage follows "LoopKV: Loop-Aware KV Cache Compression for Serving Looped
// Transformers" (arXiv:2611.04137), Abstract: each (loop, layer) cell is 4-bit
// (high and low 2-bit planes kept apart so a loop can read only the high
// bits), 2-bit, or a reuse of the final loop's KV. Byte layouts are spelled
// out in include/loopkv.h.
#pragma once
#include <stdint.h>

namespace lkv {

constexpr int kUnit = 32;       // tokens per decode unit and per selection-mask word
constexpr int kBlock = 16;      // tokens per record (a page of the block table holds 1 or 2)
constexpr int kMaxCells = 128;

// Kinds as the kernels see them (the storage a row reads).
enum : int32_t { KIND_Q4 = 0, KIND_Q2 = 1, KIND_SHARE = 2, KIND_KIVI4 = 3 };

// Byte offsets inside one record, for head dim D and quantization group GS (32 or 64).
// K meta and V meta take 64 D / GS bytes each: a group's D K-meta words are split over its
// GS / 16 records, and V meta is [D / GS][16 tokens].
__host__ __device__ constexpr int meta_bytes(int D, int GS) { return 64 * D / GS; }
__host__ __device__ constexpr int off_kmeta_planes(int D) { return 4 * D; }
__host__ __device__ constexpr int off_v_planes(int D, int GS) { return 4 * D + meta_bytes(D, GS); }
__host__ __device__ constexpr int off_vmeta_planes(int D, int GS) { return 8 * D + meta_bytes(D, GS); }
__host__ __device__ constexpr int off_klo(int D, int GS) { return 8 * D + 2 * meta_bytes(D, GS); }
__host__ __device__ constexpr int off_vlo(int D, int GS) { return 12 * D + 2 * meta_bytes(D, GS); }
__host__ __device__ constexpr int off_kmeta_kivi(int D) { return 8 * D; }
__host__ __device__ constexpr int off_v_kivi(int D, int GS) { return 8 * D + meta_bytes(D, GS); }
__host__ __device__ constexpr int off_vmeta_kivi(int D, int GS) { return 16 * D + meta_bytes(D, GS); }

// V planes store their 16-byte quads (four channel words; KIVI-4: two channels) transposed, so
// that the decode's value lanes, each reading R consecutive logical quads, read R contiguous
// spans with R load instructions: logical quad q of a plane of NQ quads sits at position
// (q mod R) * (NQ / R) + q / R. R = 2 for the 2-bit planes (NQ = D / 4); for the KIVI-4 V plane
// (NQ = D / 2) R = 2 at D <= 128 and 4 at D = 256.
__host__ __device__ constexpr int vquad_r(bool kivi, int D) { return kivi && D == 256 ? 4 : 2; }
__host__ __device__ constexpr int vquad_pos(int q, int nq, int r) { return (q % r) * (nq / r) + q / r; }
// Word position of logical word w of a V plane.
__host__ __device__ constexpr int vword_pos(int w, bool kivi, int D) {
  return vquad_pos(w / 4, kivi ? D / 2 : D / 4, vquad_r(kivi, D)) * 4 + w % 4;
}

// Record of one 16-token block and one KV head, padded to a multiple of 256 bytes (only
// D = 64 with groups of 64 pads: 1152 -> 1280, 640 -> 768).
__host__ __device__ constexpr int record_bytes(int kind, int D, int GS) {
  return ((kind == KIND_Q2 ? 8 * D : 16 * D) + 2 * meta_bytes(D, GS) + 255) / 256 * 256;
}
// Tail of one (cell, slot, head): [2 (K, V)][GS][D] bf16.
__host__ __device__ constexpr int tail_elems(int D, int GS) { return 2 * GS * D; }
// Pool index of 16-token record j of a sequence whose block-table row is bt: pages of
// 2^shift records are consecutive record slots, so record j sits in slot
// (bt[j >> shift] << shift) + (j mod 2^shift).
__host__ __device__ inline uint32_t record_slot(const int32_t* bt, int j, int shift) {
  return ((uint32_t)bt[j >> shift] << shift) + (uint32_t)(j & ((1 << shift) - 1));
}

// Per storing cell, for the append kernels.
struct AppendCell {
  uint64_t pool_off;   // byte offset of the cell's pool in the workspace
  uint64_t tail_off;   // byte offset of the cell's tails
  int32_t in_cell;     // index of the cell in the k/v input
  int32_t kind;        // KIND_Q4 / KIND_Q2 / KIND_KIVI4
};

struct AppendArgs {
  uint8_t* ws;
  const void* k;
  const void* v;
  const int32_t* seq_slots;
  const int32_t* block_table;
  const int32_t* seq_lens;
  int32_t kv_bf16;
  int32_t n_seqs, n_new, n_heads, bt_stride, n_cells;
  int32_t bt_shift;     // log2(records per page): 16-token record j lives in page j >> bt_shift
  int32_t group;        // quantization group: 32 or 64
  int32_t num_pages;    // pages per pool: records whose page lies outside [0, num_pages), or
                        // beyond the bt_stride entries of the row, are not written
  int32_t max_seqs;     // tail slots: a sequence whose slot lies outside [0, max_seqs), or whose
                        // length is negative, is not appended to
  AppendCell cells[kMaxCells];
};

// Per decoded cell, for the decode kernel.
struct DecodeCell {
  uint64_t pool_off;   // pool of the storage cell
  uint64_t tail_off;   // tails of the storage cell
  int32_t kind;        // kind of the storage cell (KIND_Q4 / KIND_Q2 / KIND_KIVI4)
  int32_t pad;
};

struct DecodeArgs {
  const uint8_t* ws;
  const void* q;
  void* out;
  uint32_t* sel_mask;
  const int32_t* seq_slots;
  const int32_t* block_table;
  const int32_t* seq_lens;
  int32_t q_bf16, out_bf16;
  int32_t n_seqs, n_heads, bt_stride, max_len, sel_words, n_cells;
  int32_t n_kv_heads;   // divides n_heads; query head h reads KV head h / (n_heads / n_kv_heads)
  int32_t bt_shift;     // log2(records per page): 16-token record j lives in page j >> bt_shift
  int32_t group;        // quantization group: 32 or 64
  int32_t num_pages;    // pages per pool: a row reading a page outside [0, num_pages) gets NaN
  int32_t max_seqs;     // tail slots: a row whose slot lies outside [0, max_seqs) gets NaN
  float tau, sm_scale;
  // Split of each row's tokens over n_split workgroups (n_split 0: one workgroup per row).
  // part: [rows][n_split][2 + D] floats (m, l, unnormalized o relative to m);
  // part_scores: [rows][split_row_stride] coarse scores (4-bit targets, 0 < tau <= 1).
  int32_t n_split, split_row_stride;
  int32_t skip;   // token-skipping ablation: unselected quantized tokens leave the attention
  float* part;
  float* part_scores;
  // In-launch append of a serving step (one cell, every KV head read by one row): the token of
  // (sequence b, KV head h) is app_k / app_v [n_seqs][1][n_kv_heads][D] (bf16 when app_bf16,
  // else f32 rounded to bf16), appended at position app_lens[b] by the workgroup that decodes
  // the row (the last split's, in a split decode) before it reads anything. Null: no append.
  const void* app_k;
  const void* app_v;
  const int32_t* app_lens;
  int32_t app_bf16;
  DecodeCell cells[kMaxCells];
};

// LDS of the in-launch append, in bytes: the group's bf16 K and V, their codes, K meta (one
// word per channel) and V meta (one word per token and channel group).
__host__ __device__ constexpr size_t fused_append_lds_bytes(int D, int GS) {
  return (size_t)6 * GS * D + (size_t)8 * D;
}

// Scratch of a split decode, in floats: partials (padded to 64 floats), then one score line
// per decoded row (lines of a multiple of 64 floats, so every line is 256-byte aligned
// relative to the scratch base).
__host__ __device__ inline size_t split_row_stride(int max_len) { return ((size_t)max_len + 63) / 64 * 64; }
__host__ __device__ inline size_t split_part_floats(size_t rows, int n_split, int D) {
  return (rows * (size_t)n_split * (size_t)(2 + D) + 63) / 64 * 64;
}
__host__ __device__ inline size_t split_scratch_floats(size_t rows, int n_split, int max_len, int D) {
  return split_part_floats(rows, n_split, D) + rows * split_row_stride(max_len);
}

}  // namespace lkv
