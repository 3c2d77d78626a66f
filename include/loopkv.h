/*
 * loopkv.h — C ABI of the loop-aware mixed-precision KV cache and its decode attention.
 *
 * Method: "LoopKV: Loop-Aware KV Cache Compression for Serving Looped
 * Transformers" (arXiv:2611.04137), Abstract. A looped transformer keeps a KV
 * cache per (loop, layer) cell; each cell is stored as 4-bit, as 2-bit, or as
 * a reuse of the final loop's KV of the same layer (abstract: the sentence on
 * the one-time offline profile). A decoding loop scores every key from the
 * upper half of its 4-bit code and loads the lower half only for the tokens
 * whose weight in that loop is large enough to need the full code (abstract:
 * the sentence on decoding); tokens of small weight still count, read at 2
 * bits, and are never dropped (abstract: the sentence on skipping). KIVI-4, uniform 4-bit quantization,
 * is the baseline run on the same kernel (abstract: the serving sentence).
 *
 * The abstract gives no formula; this library fixes:
 *   - KIVI-style asymmetric groups of G = group_size (32, or 64): K per channel
 *     over G consecutive tokens, V per token over G consecutive channels. zero = f16(min),
 *     scale = f16((max - min) / (2^b - 1)), code = clamp(rint((x - zero) /
 *     scale), 0, 2^b - 1), all in float64 with a single round-to-nearest-even
 *     to f16; scale 0 gives code 0.
 *   - 4-bit codes are split into hi = code >> 2 and lo = code & 3 and stored
 *     in separate planes. A value read from its high bits only is
 *     zero + scale * (4*hi + 3/2).
 *   - Selection: a token t of the quantized prefix is fetched at 4 bits when
 *     its coarse softmax weight (scores from high bits, softmax over the whole
 *     row) is >= tau. tau = 0 fetches every token, tau > 1 none.
 *   - The last (len mod G) tokens of a sequence are kept exact in bf16 (the
 *     tail) and quantized by the append that completes their group.
 *
 * Storage (per storing cell, caller-allocated workspace):
 *   pool  [num_blocks * block_tokens/16][KV heads][record]   record of 16 tokens, one KV head
 *   tails [max_seqs][KV heads][2 (K,V)][G][head_dim] bf16
 * Record layouts (D = head_dim, M = 64D/G meta bytes: 2D for G = 32, D for G = 64; all
 * words little-endian u32; each record padded to a multiple of 256 bytes, which only
 * D = 64 with G = 64 needs):
 *   4-bit planes : [K_hi 4D | K_meta M | V_hi 4D | V_meta M | K_lo 4D | V_lo 4D]  = 20D (G 32), 18D (G 64)
 *   2-bit        : [K2 4D   | K_meta M | V2 4D   | V_meta M]                      = 12D (G 32), 10D (G 64)
 *   KIVI-4       : [K4 8D   | K_meta M | V4 8D   | V_meta M]                      = 20D (G 32), 18D (G 64)
 *   (the bytes a decode reads for every token — high K part, then high V part — are
 *   each contiguous; the low planes follow and are read only where selected)
 *   K plane (2-bit): D/16 columns x 16 tokens of u32; word (w, t) holds channels
 *     16w..16w+15 of token t, channel 16w+4k+p at bit 8k+2p.
 *   K plane (4-bit): D/8 columns x 16 tokens; channel 8w+2k+n at bit 8k+4n.
 *   V plane (2-bit): D words; logical word d holds channel d of the 16 tokens, token t at
 *     bit 8*(t%4) + 2*(t/4).
 *   V plane (4-bit): D x 2 words; logical word 2d+j holds tokens 8j..8j+7 of channel d,
 *     token t' = t-8j at bit 8*(t'%4) + 4*(t'/4).
 *   V planes are stored as 16-byte quads of four logical words, transposed: logical quad
 *     q = r*a + i of a plane of Q quads sits at quad position i*(Q/r) + a, with r = 2 for
 *     the 2-bit planes and r = 2 (head_dim <= 128) or 4 (head_dim 256) for the 4-bit plane
 *     (a value lane's r quads are then r contiguous spans read by r load instructions).
 *   Meta word: f16 scale in bits 0-15, f16 zero in bits 16-31.
 *   K_meta of group g: one word per channel, permuted inside each K column so that a
 *     column's words follow its bit layout — 2-bit: position 16w+4p+k holds channel
 *     16w+4k+p; 4-bit: position 8w+4n+k holds channel 8w+2k+n — and split over the
 *     group's P = G/16 blocks: logical block P*g + i holds positions i*D/P .. (i+1)*D/P - 1.
 *   V_meta: [D/G channel groups][16 tokens].
 *
 * Paging: block_table[b * bt_stride + p] is the physical page of logical page p
 * (tokens block_tokens*p .. block_tokens*(p+1)-1) of sequence b; the same id addresses
 * every cell's pool. A page of 16 tokens is one record slot; a page of 32 tokens is the
 * two consecutive slots 2*id and 2*id+1, holding its first and second 16 tokens.
 * The kernels check page ids against the pool: a decode row whose quantized prefix maps a
 * page outside [0, num_blocks) (an unmapped -1 included) gets NaN output and an empty
 * selection instead of reading it; an append does not write a record whose page is out of
 * range or lies beyond the row's bt_stride entries. Likewise a seq_slots entry outside
 * [0, max_seqs) gives a decode row NaN and makes an append skip that sequence, as does a
 * negative length in an append.
 *
 * Ownership: the caller owns every device buffer (workspace, q, k, v, out,
 * tables, masks). The library never allocates device memory and never
 * synchronizes a stream. A context is not thread-safe; separate contexts are
 * independent.
 *
 * Errors: every call validates its arguments on the host before enqueuing
 * anything; on error nothing is enqueued and loopkv_last_error() describes it.
 * Kernel faults surface at the caller's next synchronization.
 */
#ifndef LOOPKV_H
#define LOOPKV_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LOOPKV_OK = 0,
  LOOPKV_ERR_INVALID_ARG = 1, /* null / out-of-range argument, bad dtype, tau < 0 or NaN, sm_scale <= 0 */
  LOOPKV_ERR_PLAN = 2,        /* no plan loaded, kind > 2, reuse cell in the final loop, bad cell index */
  LOOPKV_ERR_WORKSPACE = 3,   /* workspace not bound, too small, or not 256-byte aligned */
  LOOPKV_ERR_CAPACITY = 4,    /* bt_stride * block_tokens < max_len, max_len above the supported maximum */
  LOOPKV_ERR_UNSUPPORTED = 5, /* head_dim not 64/128/256, group not 32/64, block not 16/32, too many
                                 cells; at the first launch on a device: the device is not gfx950 */
  LOOPKV_ERR_HIP = 6          /* HIP runtime / launch failure */
} loopkv_status;

typedef enum { LOOPKV_CELL_Q4 = 0, LOOPKV_CELL_Q2 = 1, LOOPKV_CELL_SHARE = 2 } loopkv_cell_kind;
typedef enum { LOOPKV_F32 = 0, LOOPKV_BF16 = 1 } loopkv_dtype;
typedef enum { LOOPKV_LAYOUT_PLANES = 0, LOOPKV_LAYOUT_KIVI4 = 1 } loopkv_layout;

/* Largest supported max_len of one decode call (coarse scores of a row live in LDS). */
#define LOOPKV_MAX_LEN 32768
#define LOOPKV_MAX_SPLIT 64   /* workgroups per row of a split decode */
/* Largest n_loops * n_layers. */
#define LOOPKV_MAX_CELLS 128
#define LOOPKV_MAX_PLAN_CELLS 4096   /* cells of one plan search */

typedef struct {
  int32_t n_loops, n_layers; /* cells = n_loops * n_layers, row-major [loop][layer] */
  int32_t n_heads;           /* query heads */
  int32_t head_dim;          /* 64, 128 or 256 */
  int32_t group_size;        /* quantization group G: 32 (the default reading) or 64 */
  int32_t block_tokens;      /* tokens per page of the block table: 16 or 32 */
  int32_t num_blocks;        /* physical pages in each storing cell's pool; a pool (num_blocks x
                                block_tokens/16 x KV heads x 20*head_dim bytes) stays below 1 TiB
                                (pools of 4 GiB or more are read with 64-bit record offsets) */
  int32_t max_seqs;          /* sequence slots (tail buffers) */
  int32_t layout;            /* loopkv_layout; KIVI4 requires an all-4-bit plan */
  int32_t n_kv_heads;        /* KV heads (0: = n_heads, MHA); divides n_heads. Query head h
                                reads KV head h / (n_heads / n_kv_heads) (grouped queries) */
} loopkv_config;

typedef struct loopkv_ctx loopkv_ctx;

/* Validate cfg and create a context (host memory only). */
loopkv_status loopkv_create(const loopkv_config* cfg, loopkv_ctx** out);
void loopkv_destroy(loopkv_ctx* ctx);

/* Load the plan: host array kinds[n_loops * n_layers] of loopkv_cell_kind, row-major
 * [loop][layer]. A reuse cell (SHARE) of layer l reads cell (n_loops-1, l); the final
 * loop may not be SHARE. With the KIVI4 layout every cell must be Q4. Resets any
 * bound workspace. */
loopkv_status loopkv_plan(loopkv_ctx* ctx, const uint8_t* kinds);

/* Bytes of workspace the loaded plan needs (pools + tails of the storing cells). */
loopkv_status loopkv_workspace_bytes(const loopkv_ctx* ctx, size_t* bytes);

/* Bind caller-owned device memory (>= loopkv_workspace_bytes, 256-byte aligned).
 * The library does not clear it: a fresh cache is valid for any sequence whose
 * seq_lens entry starts at 0. */
loopkv_status loopkv_bind_workspace(loopkv_ctx* ctx, void* dev, size_t bytes);

/* Where a cell's storage lives inside the workspace (for inspection and tests):
 * byte offsets of its pool and tails and its record size; a SHARE cell reports the
 * final-loop cell it reads. */
loopkv_status loopkv_cell_storage(const loopkv_ctx* ctx, int32_t loop, int32_t layer,
                                  size_t* pool_offset, size_t* tail_offset,
                                  size_t* record_bytes, int32_t* storage_cell);

/* Append n_new tokens to every sequence of one cell ((loop, layer)) or of every
 * storing cell ((-1, -1)). k, v: device [cells][n_seqs][n_new][H][D] (whole plan,
 * cells = n_loops*n_layers, SHARE entries ignored) or [n_seqs][n_new][H][D]; F32 input
 * is rounded to bf16 (nearest even). seq_slots: device [n_seqs] tail slot of each
 * sequence or NULL for slot = b. block_table: device [n_seqs][bt_stride]; the pages of
 * tokens G*g .. G*g+G-1 must be mapped before the append that completes group g. seq_lens: device
 * [n_seqs], length before the append (read only; the caller advances it). Completed
 * groups of G tokens are quantized into the pool; the rest goes to the tail. Appending to
 * a SHARE cell is a no-op. */
loopkv_status loopkv_append(loopkv_ctx* ctx, hipStream_t stream, int32_t loop, int32_t layer,
                            const void* k, const void* v, int32_t kv_dtype,
                            int32_t n_seqs, int32_t n_new, const int32_t* seq_slots,
                            const int32_t* block_table, int32_t bt_stride,
                            const int32_t* seq_lens);

/* Loop-aware decode attention of one cell ((loop, layer)) or of the whole plan ((-1, -1)).
 * q: device [cells][n_seqs][H][D] (whole plan) or [n_seqs][H][D], dtype q_dtype.
 * seq_lens: device lengths (tail included); max_len: host upper bound of them
 * (<= LOOPKV_MAX_LEN, <= block_tokens * bt_stride). Rows whose length exceeds max_len get NaN
 * output. tau >= 0: selection threshold on the coarse softmax; sm_scale > 0.
 * out: device [cells][n_seqs][H][D] (or [n_seqs][H][D]) of out_dtype, accumulated in fp32.
 * sel_mask: NULL or device [cells][n_seqs][H][ceil(max_len/32)] u32; bit t%32 of word
 * t/32 is set iff token t was fetched at 4 bits (all quantized tokens for KIVI4 and
 * tau = 0; none for 2-bit targets). */
loopkv_status loopkv_decode_attn(loopkv_ctx* ctx, hipStream_t stream, int32_t loop, int32_t layer,
                                 const void* q, int32_t q_dtype, int32_t n_seqs,
                                 const int32_t* seq_slots, const int32_t* block_table,
                                 int32_t bt_stride, const int32_t* seq_lens, int32_t max_len,
                                 float tau, float sm_scale, void* out, int32_t out_dtype,
                                 uint32_t* sel_mask);

/* Scratch bytes a split decode of this (loop, layer) ((-1, -1): whole plan) needs for
 * n_seqs sequences, max_len and n_split (1..LOOPKV_MAX_SPLIT): n_split partials of
 * (2 + head_dim) floats per row (the region rounded up to 64 floats), then one line of
 * ceil(max_len/64)*64 coarse scores per row. */
loopkv_status loopkv_split_scratch_bytes(const loopkv_ctx* ctx, int32_t loop, int32_t layer,
                                         int32_t n_seqs, int32_t max_len, int32_t n_split,
                                         size_t* bytes);

/* The same decode as loopkv_decode_attn (same arguments, same results up to the order of
 * fp32 additions), with each row's tokens split over n_split workgroups, for calls with
 * few rows (one cell at a small batch), where one workgroup per row leaves most of the
 * GPU idle. The split follows the split-K online softmax of the decode: every workgroup
 * streams a range of the row's tokens and leaves a partial (max, weight, values); a
 * second launch on the same stream merges the partials, selects the tokens whose coarse
 * weight over the whole row reaches tau (the row-global softmax of the Abstract's
 * decoding sentence), fetches their low bits and writes the row.
 * scratch: caller-owned device memory of >= loopkv_split_scratch_bytes bytes, 16-byte
 * aligned; its contents are overwritten and need no initialization. Calls that share a
 * scratch buffer must be ordered (one stream). Errors as for loopkv_decode_attn, plus
 * LOOPKV_ERR_INVALID_ARG for n_split outside [1, LOOPKV_MAX_SPLIT] and
 * LOOPKV_ERR_WORKSPACE for a missing, misaligned or short scratch. */
loopkv_status loopkv_decode_attn_split(loopkv_ctx* ctx, hipStream_t stream, int32_t loop,
                                       int32_t layer, const void* q, int32_t q_dtype,
                                       int32_t n_seqs, const int32_t* seq_slots,
                                       const int32_t* block_table, int32_t bt_stride,
                                       const int32_t* seq_lens, int32_t max_len, float tau,
                                       float sm_scale, void* out, int32_t out_dtype,
                                       uint32_t* sel_mask, int32_t n_split, void* scratch,
                                       size_t scratch_bytes);

/* Bytes of the fixed device array behind loopkv_decode_attn_split_noalloc (one per GPU). */
#define LOOPKV_NOALLOC_SCRATCH_BYTES (16u << 20)

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): loopkv_decode_attn_split with the scratch taken
 * from a file-scope device array of LOOPKV_NOALLOC_SCRATCH_BYTES bytes inside the library
 * instead of a caller buffer. Same arguments (without scratch), same kernels, same results.
 * The library allocates nothing here; each GPU the call runs on holds its own copy of the
 * array until the process ends (its address is resolved on the first call on a device, which
 * callers that capture should make once before capturing). Every call on one GPU shares that
 * GPU's array and overwrites it (no initialization needed): calls that overlap on one GPU
 * (different streams, or contexts used from several threads) race and must be ordered by the
 * caller. Errors as loopkv_decode_attn_split, and LOOPKV_ERR_WORKSPACE when the call needs
 * more than LOOPKV_NOALLOC_SCRATCH_BYTES of scratch (loopkv_split_scratch_bytes tells). */
loopkv_status loopkv_decode_attn_split_noalloc(loopkv_ctx* ctx, hipStream_t stream, int32_t loop,
                                               int32_t layer, const void* q, int32_t q_dtype,
                                               int32_t n_seqs, const int32_t* seq_slots,
                                               const int32_t* block_table, int32_t bt_stride,
                                               const int32_t* seq_lens, int32_t max_len, float tau,
                                               float sm_scale, void* out, int32_t out_dtype,
                                               uint32_t* sel_mask, int32_t n_split);

/* The token-skipping ablation (the alternative the Abstract's sentence on skipping rejects;
 * not the method): arguments, selection and sel_mask as loopkv_decode_attn, but a 4-bit
 * target's unselected quantized tokens are dropped instead of read at 2 bits: their values
 * are never read and the softmax runs over the selected tokens (at 4 bits) and the exact
 * tail; a row that keeps nothing gets 0. tau = 0 keeps every token (the decode of
 * loopkv_decode_attn at tau = 0); tau > 1 keeps the tail only. 2-bit targets decode as in
 * loopkv_decode_attn. Errors as loopkv_decode_attn, plus LOOPKV_ERR_UNSUPPORTED with the
 * KIVI4 layout. */
loopkv_status loopkv_decode_attn_skip(loopkv_ctx* ctx, hipStream_t stream, int32_t loop,
                                      int32_t layer, const void* q, int32_t q_dtype,
                                      int32_t n_seqs, const int32_t* seq_slots,
                                      const int32_t* block_table, int32_t bt_stride,
                                      const int32_t* seq_lens, int32_t max_len, float tau,
                                      float sm_scale, void* out, int32_t out_dtype,
                                      uint32_t* sel_mask);

/* Costs of one cell for the planner, indexed by loopkv_cell_kind (Q4, Q2, SHARE): the
 * predicted damage of storing the cell that way (damages of cells add up: the additive
 * model of the Abstract's sentence on measurements on Ouro), the bytes (or any one unit) the
 * cell reads per decode step, and its storage in integer units. */
typedef struct {
  double damage[3];
  double reads[3];
  int64_t storage[3];
} loopkv_cell_cost;

/* The planner (Abstract, sentence on the planner): choose a kind for each of the
 * n_loops * n_layers cells (costs row-major [loop][layer]) that minimizes the total reads
 * subject to total damage <= damage_budget (may be +inf) and total storage <=
 * storage_budget, cells of the final loop never SHARE. Exact (dynamic programming over
 * non-dominated partial plans; host only, no GPU). kinds_out: host [cells] loopkv_cell_kind,
 * ready for loopkv_plan; the plan's sums go to damage_out / reads_out / storage_out
 * (each nullable). Among plans of equal least reads the one returned is unspecified but
 * fixed for a given table. Errors: LOOPKV_ERR_INVALID_ARG (null costs or kinds_out, cell
 * count outside [1, LOOPKV_MAX_PLAN_CELLS], a NaN, infinite or negative cost, a negative
 * or NaN budget), LOOPKV_ERR_PLAN (no plan meets the budgets; kinds_out untouched),
 * LOOPKV_ERR_UNSUPPORTED (the search outgrows its state limit, 2^22 partial plans). */
loopkv_status loopkv_plan_search(int32_t n_loops, int32_t n_layers, const loopkv_cell_cost* costs,
                                 double damage_budget, int64_t storage_budget,
                                 uint8_t* kinds_out, double* damage_out, double* reads_out,
                                 int64_t* storage_out);

/* One serving decode step in the order a looped model runs it, captured once into a HIP
 * graph and replayed (the pages serve their fused kernel under a graph: Abstract, serving
 * sentence). For every cell (loop, layer) in row-major order: the append of the step's token
 * (storing cells) and the decode of that cell with its query. A reuse cell decodes over
 * seq_lens_before (its final-loop cell runs later in the step, so that cache does not hold
 * the step's token yet), every other cell over seq_lens_after; the step ends by adding 1 to
 * both length arrays, so consecutive launches are consecutive decode steps.
 *   k, v: device [cells][n_seqs][1][KV heads][D] of kv_dtype (reuse entries ignored);
 *   q: device [cells][n_seqs][H][D] of q_dtype; out: device [cells][n_seqs][H][D] of
 *   out_dtype; sel_mask: NULL or device [cells][n_seqs][H][ceil(max_len/32)] u32;
 *   seq_lens_before, seq_lens_after: device [n_seqs], distinct, advanced in place;
 *   max_len: bound on seq_lens_after over every launch the graph will make.
 *   n_split 0: one workgroup per row; 1..LOOPKV_MAX_SPLIT: the split decode, scratch of at
 *   least loopkv_split_scratch_bytes(ctx, 0, 0, n_seqs, max_len, n_split) bytes, shared by
 *   the cells one after another (the graph orders them).
 * Every pointer is fixed at creation and read at each launch: the caller refills k, v and q
 * between launches. Capture runs on a private stream and enqueues nothing; the graph keeps
 * the context's workspace and plan as they are at creation (rebinding the workspace or
 * reloading the plan needs a new graph). Records no memset node. Errors: argument errors
 * as loopkv_append / loopkv_decode_attn_split (checked before capture), LOOPKV_ERR_HIP if
 * capture or instantiation fails; *graph is NULL on error. */
typedef struct loopkv_step_graph loopkv_step_graph;
loopkv_status loopkv_step_graph_create(loopkv_ctx* ctx, const void* k, const void* v, int32_t kv_dtype,
                                       const void* q, int32_t q_dtype, int32_t n_seqs,
                                       const int32_t* seq_slots, const int32_t* block_table,
                                       int32_t bt_stride, int32_t* seq_lens_before,
                                       int32_t* seq_lens_after, int32_t max_len, float tau,
                                       float sm_scale, void* out, int32_t out_dtype,
                                       uint32_t* sel_mask, int32_t n_split, void* scratch,
                                       size_t scratch_bytes, loopkv_step_graph** graph);
/* Replay the step on a stream (asynchronous, like every other call). */
loopkv_status loopkv_step_graph_launch(loopkv_step_graph* graph, hipStream_t stream);
/* Release a step graph (NULL is a no-op). Work already enqueued is not affected. */
void loopkv_step_graph_destroy(loopkv_step_graph* graph);

/* Thread-local description of the last error on this thread ("" after success). */
const char* loopkv_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* LOOPKV_H */
