// Host runtime of the C ABI declared in include/loopkv.h: plan validation,
// workspace carving, argument checks, kernel launches and the capture of a serving
// step into a HIP graph. Nothing here touches the GPU except the launches and the
// capture, and every argument check comes first, so every validation path runs (and
// is tested) on a machine without a GPU.
//
// Plan semantics follow "LoopKV: Loop-Aware KV Cache Compression for Serving
// Looped Transformers" (arXiv:2611.04137), Abstract: a cell is 4-bit, 2-bit or
// a reuse of the final loop's KV of its layer.
#include <hip/hip_runtime.h>
#include <atomic>
#include <mutex>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "loopkv.h"
#include "layout.h"

namespace lkv {
hipError_t launch_append(const AppendArgs& a, int head_dim, hipStream_t stream);
// decode.hip is built twice: records addressed by 32-bit offsets (every pool below 4 GiB) and
// by 64-bit ones
hipError_t launch_decode_small(const DecodeArgs& a, int head_dim, hipStream_t stream);
hipError_t launch_decode_big(const DecodeArgs& a, int head_dim, hipStream_t stream);
void prepare_decode_small(int head_dim, int group);
void prepare_decode_big(int head_dim, int group);
hipError_t launch_advance_lens(int32_t* before, int32_t* after, int n, hipStream_t stream);
size_t decode_lds_bytes(int max_len, int head_dim);
}  // namespace lkv

struct loopkv_ctx {
  loopkv_config cfg;
  int kvh = 0;                    // KV heads (cfg.n_kv_heads, or n_heads when 0)
  bool big = false;               // a pool reaches 4 GiB: the decode addresses records in 64 bits
  bool has_plan = false;
  std::vector<uint8_t> kinds;     // per cell, loopkv_cell_kind
  std::vector<int> storage;       // per cell: cell whose cache it reads
  std::vector<size_t> pool_off;   // per cell (valid for storing cells)
  std::vector<size_t> tail_off;
  size_t ws_need = 0;
  uint8_t* ws = nullptr;
  size_t ws_bytes = 0;
};

namespace {
thread_local std::string g_err;

loopkv_status fail(loopkv_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
loopkv_status fail(loopkv_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}
loopkv_status ok() {
  g_err.clear();
  return LOOPKV_OK;
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

int n_cells(const loopkv_ctx* c) { return c->cfg.n_loops * c->cfg.n_layers; }

int device_kind(const loopkv_ctx* c, int storage_cell) {
  if (c->cfg.layout == LOOPKV_LAYOUT_KIVI4) return lkv::KIND_KIVI4;
  return c->kinds[storage_cell] == LOOPKV_CELL_Q2 ? lkv::KIND_Q2 : lkv::KIND_Q4;
}

// Resolve (loop, layer) to a list of cells: (-1, -1) = all cells.
loopkv_status resolve_cells(const loopkv_ctx* c, int loop, int layer, int* first, int* count) {
  if (loop == -1 && layer == -1) {
    *first = 0;
    *count = n_cells(c);
    return LOOPKV_OK;
  }
  if (loop < 0 || loop >= c->cfg.n_loops || layer < 0 || layer >= c->cfg.n_layers)
    return fail(LOOPKV_ERR_PLAN, "cell (%d, %d) out of range for %d loops x %d layers", loop, layer,
                c->cfg.n_loops, c->cfg.n_layers);
  *first = loop * c->cfg.n_layers + layer;
  *count = 1;
  return LOOPKV_OK;
}

// The kernels are built for gfx950 only: the current device is checked once (per device id)
// before the first launch on it.
loopkv_status check_device() {
  static std::atomic<int> state[64];   // 0 unknown, 1 gfx950, -1 another device
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(LOOPKV_ERR_HIP, "no current HIP device: %s", hipGetErrorString(e));
  if (dev >= 0 && dev < 64 && state[dev].load(std::memory_order_relaxed) == 1) return LOOPKV_OK;
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess) return fail(LOOPKV_ERR_HIP, "device properties: %s", hipGetErrorString(e));
  const bool ok950 = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev >= 0 && dev < 64) state[dev].store(ok950 ? 1 : -1, std::memory_order_relaxed);
  if (!ok950) return fail(LOOPKV_ERR_UNSUPPORTED, "device %d is %s; the kernels are built for gfx950", dev,
                          prop.gcnArchName);
  return LOOPKV_OK;
}

loopkv_status check_ready(const loopkv_ctx* c) {
  if (!c) return fail(LOOPKV_ERR_INVALID_ARG, "null context");
  if (!c->has_plan) return fail(LOOPKV_ERR_PLAN, "no plan loaded");
  if (!c->ws) return fail(LOOPKV_ERR_WORKSPACE, "no workspace bound");
  return LOOPKV_OK;
}
}  // namespace

namespace lkv {   // error reporting for the planner (planner.cpp)
loopkv_status planner_fail(loopkv_status s, const char* msg) { return fail(s, "%s", msg); }
loopkv_status planner_ok() { return ok(); }
}  // namespace lkv

extern "C" {

const char* loopkv_last_error(void) { return g_err.c_str(); }

loopkv_status loopkv_create(const loopkv_config* cfg, loopkv_ctx** out) {
  if (!cfg || !out) return fail(LOOPKV_ERR_INVALID_ARG, "null argument");
  *out = nullptr;
  if (cfg->n_loops < 1 || cfg->n_layers < 1 || cfg->n_heads < 1 || cfg->num_blocks < 1 || cfg->max_seqs < 1)
    return fail(LOOPKV_ERR_INVALID_ARG, "n_loops, n_layers, n_heads, num_blocks and max_seqs must be >= 1");
  if (cfg->n_kv_heads < 0 || (cfg->n_kv_heads > 0 && cfg->n_heads % cfg->n_kv_heads != 0))
    return fail(LOOPKV_ERR_INVALID_ARG, "n_kv_heads %d must be 0 or divide n_heads %d", cfg->n_kv_heads, cfg->n_heads);
  const int kvh = cfg->n_kv_heads ? cfg->n_kv_heads : cfg->n_heads;
  if (cfg->head_dim != 64 && cfg->head_dim != 128 && cfg->head_dim != 256)
    return fail(LOOPKV_ERR_UNSUPPORTED, "head_dim %d not supported (64, 128 or 256)", cfg->head_dim);
  if (cfg->group_size != 32 && cfg->group_size != 64)
    return fail(LOOPKV_ERR_UNSUPPORTED, "group_size %d not supported (32 or 64)", cfg->group_size);
  if (cfg->block_tokens != 16 && cfg->block_tokens != 32)
    return fail(LOOPKV_ERR_UNSUPPORTED, "block_tokens %d not supported (16 or 32)", cfg->block_tokens);
  const uint64_t recs = (uint64_t)cfg->num_blocks * (uint64_t)(cfg->block_tokens / lkv::kBlock);
  const uint64_t pool_bytes = recs * (uint64_t)kvh * lkv::record_bytes(lkv::KIND_Q4, cfg->head_dim, cfg->group_size);
  if (pool_bytes >= (1ull << 40))   // record offsets are 32-bit counts of 256-byte units
    return fail(LOOPKV_ERR_UNSUPPORTED, "a cell's pool of %llu bytes reaches 1 TiB",
                (unsigned long long)pool_bytes);
  if ((long long)cfg->n_loops * cfg->n_layers > lkv::kMaxCells)
    return fail(LOOPKV_ERR_UNSUPPORTED, "at most %d cells", lkv::kMaxCells);
  if (cfg->layout != LOOPKV_LAYOUT_PLANES && cfg->layout != LOOPKV_LAYOUT_KIVI4)
    return fail(LOOPKV_ERR_INVALID_ARG, "unknown layout %d", cfg->layout);
  loopkv_ctx* c = new loopkv_ctx();
  c->cfg = *cfg;
  c->kvh = kvh;
  c->big = pool_bytes > 0xFFFFFFFFull;
  *out = c;
  return ok();
}

void loopkv_destroy(loopkv_ctx* ctx) { delete ctx; }

loopkv_status loopkv_plan(loopkv_ctx* c, const uint8_t* kinds) {
  if (!c || !kinds) return fail(LOOPKV_ERR_INVALID_ARG, "null argument");
  const int n = n_cells(c);
  const int L = c->cfg.n_loops, NL = c->cfg.n_layers;
  for (int i = 0; i < n; ++i) {
    if (kinds[i] > LOOPKV_CELL_SHARE) return fail(LOOPKV_ERR_PLAN, "cell %d: kind %u > 2", i, kinds[i]);
    if (kinds[i] == LOOPKV_CELL_SHARE && i / NL == L - 1)
      return fail(LOOPKV_ERR_PLAN, "cell %d: the final loop cannot reuse its own KV", i);
    if (c->cfg.layout == LOOPKV_LAYOUT_KIVI4 && kinds[i] != LOOPKV_CELL_Q4)
      return fail(LOOPKV_ERR_PLAN, "KIVI-4 layout needs an all-4-bit plan (cell %d)", i);
  }
  c->kinds.assign(kinds, kinds + n);
  c->storage.resize(n);
  c->pool_off.assign(n, 0);
  c->tail_off.assign(n, 0);
  const int D = c->cfg.head_dim, H = c->kvh;   // records and tails per KV head
  size_t off = 0;
  for (int i = 0; i < n; ++i) {
    c->storage[i] = kinds[i] == LOOPKV_CELL_SHARE ? (L - 1) * NL + i % NL : i;
    if (kinds[i] == LOOPKV_CELL_SHARE) continue;
    c->pool_off[i] = off;
    off = align256(off + (size_t)c->cfg.num_blocks * (c->cfg.block_tokens / lkv::kBlock) * H *
                             lkv::record_bytes(device_kind(c, i), D, c->cfg.group_size));
  }
  for (int i = 0; i < n; ++i) {
    if (kinds[i] == LOOPKV_CELL_SHARE) continue;
    c->tail_off[i] = off;
    off = align256(off + (size_t)c->cfg.max_seqs * H * lkv::tail_elems(D, c->cfg.group_size) * 2);
  }
  for (int i = 0; i < n; ++i) {
    if (kinds[i] != LOOPKV_CELL_SHARE) continue;
    c->pool_off[i] = c->pool_off[c->storage[i]];
    c->tail_off[i] = c->tail_off[c->storage[i]];
  }
  c->ws_need = off;
  c->has_plan = true;
  c->ws = nullptr;
  c->ws_bytes = 0;
  return ok();
}

loopkv_status loopkv_workspace_bytes(const loopkv_ctx* c, size_t* bytes) {
  if (!c || !bytes) return fail(LOOPKV_ERR_INVALID_ARG, "null argument");
  if (!c->has_plan) return fail(LOOPKV_ERR_PLAN, "no plan loaded");
  *bytes = c->ws_need;
  return ok();
}

loopkv_status loopkv_bind_workspace(loopkv_ctx* c, void* dev, size_t bytes) {
  if (!c || !dev) return fail(LOOPKV_ERR_INVALID_ARG, "null argument");
  if (!c->has_plan) return fail(LOOPKV_ERR_PLAN, "no plan loaded");
  if (((uintptr_t)dev & 255u) != 0) return fail(LOOPKV_ERR_WORKSPACE, "workspace not 256-byte aligned");
  if (bytes < c->ws_need)
    return fail(LOOPKV_ERR_WORKSPACE, "workspace of %zu bytes, plan needs %zu", bytes, c->ws_need);
  c->ws = static_cast<uint8_t*>(dev);
  c->ws_bytes = bytes;
  return ok();
}

loopkv_status loopkv_cell_storage(const loopkv_ctx* c, int32_t loop, int32_t layer, size_t* pool_offset,
                                  size_t* tail_offset, size_t* record_bytes, int32_t* storage_cell) {
  if (!c) return fail(LOOPKV_ERR_INVALID_ARG, "null context");
  if (!c->has_plan) return fail(LOOPKV_ERR_PLAN, "no plan loaded");
  if (loop < 0 || layer < 0) return fail(LOOPKV_ERR_PLAN, "cell (%d, %d) out of range", loop, layer);
  int first, count;
  loopkv_status s = resolve_cells(c, loop, layer, &first, &count);
  if (s != LOOPKV_OK) return s;
  const int st = c->storage[first];
  if (pool_offset) *pool_offset = c->pool_off[st];
  if (tail_offset) *tail_offset = c->tail_off[st];
  if (record_bytes) *record_bytes = lkv::record_bytes(device_kind(c, st), c->cfg.head_dim, c->cfg.group_size);
  if (storage_cell) *storage_cell = st;
  return ok();
}

loopkv_status loopkv_append(loopkv_ctx* c, hipStream_t stream, int32_t loop, int32_t layer, const void* k,
                            const void* v, int32_t kv_dtype, int32_t n_seqs, int32_t n_new,
                            const int32_t* seq_slots, const int32_t* block_table, int32_t bt_stride,
                            const int32_t* seq_lens) {
  loopkv_status s = check_ready(c);
  if (s != LOOPKV_OK) return s;
  int first, count;
  s = resolve_cells(c, loop, layer, &first, &count);
  if (s != LOOPKV_OK) return s;
  if (kv_dtype != LOOPKV_F32 && kv_dtype != LOOPKV_BF16) return fail(LOOPKV_ERR_INVALID_ARG, "bad kv dtype %d", kv_dtype);
  if (n_seqs < 0 || n_new < 0) return fail(LOOPKV_ERR_INVALID_ARG, "n_seqs and n_new must be >= 0");
  if (!seq_slots && n_seqs > c->cfg.max_seqs)
    return fail(LOOPKV_ERR_CAPACITY, "n_seqs %d > max_seqs %d with identity slots", n_seqs, c->cfg.max_seqs);
  if (n_seqs == 0 || n_new == 0) return ok();
  if (!k || !v || !block_table || !seq_lens) return fail(LOOPKV_ERR_INVALID_ARG, "null device pointer");
  if (bt_stride < 1) return fail(LOOPKV_ERR_INVALID_ARG, "bt_stride must be >= 1");
  lkv::AppendArgs a;
  std::memset(&a, 0, sizeof(a));
  a.ws = c->ws;
  a.k = k;
  a.v = v;
  a.seq_slots = seq_slots;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.kv_bf16 = kv_dtype == LOOPKV_BF16;
  a.n_seqs = n_seqs;
  a.n_new = n_new;
  a.n_heads = c->kvh;   // the append's inputs hold the KV heads
  a.bt_stride = bt_stride;
  a.bt_shift = c->cfg.block_tokens == 32 ? 1 : 0;
  a.group = c->cfg.group_size;
  a.num_pages = c->cfg.num_blocks;
  a.max_seqs = c->cfg.max_seqs;
  int nc = 0;
  for (int i = first; i < first + count; ++i) {
    if (c->kinds[i] == LOOPKV_CELL_SHARE) continue;
    a.cells[nc].pool_off = c->pool_off[i];
    a.cells[nc].tail_off = c->tail_off[i];
    a.cells[nc].in_cell = count == 1 ? 0 : i;
    a.cells[nc].kind = device_kind(c, i);
    ++nc;
  }
  a.n_cells = nc;
  if (nc == 0) return ok();
  s = check_device();
  if (s != LOOPKV_OK) return s;
  hipError_t e = lkv::launch_append(a, c->cfg.head_dim, stream);
  if (e != hipSuccess) return fail(LOOPKV_ERR_HIP, "append launch: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"

// The split-decode scratch of loopkv_decode_attn_split_noalloc: a fixed array in device
// memory, one copy per GPU for the life of the process. Host code never uses the name
// itself (on the host it is a stand-in, not a device address): the device address is
// resolved once per device and passed to the kernels as the split decode's scratch.
static __device__ __align__(256) unsigned char scratch[LOOPKV_NOALLOC_SCRATCH_BYTES];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_dev[64] = {};   // device address of `scratch`, per device id

loopkv_status noalloc_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(LOOPKV_ERR_HIP, "no current HIP device: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(LOOPKV_ERR_UNSUPPORTED, "device id %d above 63", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(LOOPKV_ERR_HIP, "device address of the fixed scratch: %s", hipGetErrorString(e));
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return LOOPKV_OK;
}
}  // namespace

namespace {
// Shared by the one-workgroup-per-row decode (n_split 0) and the split decode.
loopkv_status decode_common(loopkv_ctx* c, hipStream_t stream, int32_t loop, int32_t layer, const void* q,
                            int32_t q_dtype, int32_t n_seqs, const int32_t* seq_slots, const int32_t* block_table,
                            int32_t bt_stride, const int32_t* seq_lens, int32_t max_len, float tau, float sm_scale,
                            void* out, int32_t out_dtype, uint32_t* sel_mask, int32_t n_split, void* scratch,
                            size_t scratch_bytes, bool skip, bool fixed_scratch = false,
                            const void* app_k = nullptr, const void* app_v = nullptr, int32_t app_dtype = LOOPKV_BF16,
                            const int32_t* app_lens = nullptr) {
  loopkv_status s = check_ready(c);
  if (s != LOOPKV_OK) return s;
  int first, count;
  s = resolve_cells(c, loop, layer, &first, &count);
  if (s != LOOPKV_OK) return s;
  if (q_dtype != LOOPKV_F32 && q_dtype != LOOPKV_BF16) return fail(LOOPKV_ERR_INVALID_ARG, "bad q dtype %d", q_dtype);
  if (out_dtype != LOOPKV_F32 && out_dtype != LOOPKV_BF16)
    return fail(LOOPKV_ERR_INVALID_ARG, "bad out dtype %d", out_dtype);
  if (!(tau >= 0.f)) return fail(LOOPKV_ERR_INVALID_ARG, "tau must be >= 0 (got %g)", (double)tau);
  if (!(sm_scale > 0.f) || !std::isfinite(sm_scale))
    return fail(LOOPKV_ERR_INVALID_ARG, "sm_scale must be finite and > 0 (got %g)", (double)sm_scale);
  if (n_seqs < 0) return fail(LOOPKV_ERR_INVALID_ARG, "n_seqs must be >= 0");
  if (!seq_slots && n_seqs > c->cfg.max_seqs)
    return fail(LOOPKV_ERR_CAPACITY, "n_seqs %d > max_seqs %d with identity slots", n_seqs, c->cfg.max_seqs);
  if (max_len < 0 || max_len > LOOPKV_MAX_LEN)
    return fail(LOOPKV_ERR_CAPACITY, "max_len %d outside [0, %d]", max_len, LOOPKV_MAX_LEN);
  if (bt_stride < 1 || (long long)bt_stride * c->cfg.block_tokens < max_len)
    return fail(LOOPKV_ERR_CAPACITY, "bt_stride %d too small for max_len %d", bt_stride, max_len);
  if (skip && c->cfg.layout == LOOPKV_LAYOUT_KIVI4)
    return fail(LOOPKV_ERR_UNSUPPORTED, "token skipping needs the planes layout");
  if (skip && n_split != 0) return fail(LOOPKV_ERR_INVALID_ARG, "token skipping runs one workgroup per row");
  if (n_split != 0) {
    if (n_split < 1 || n_split > LOOPKV_MAX_SPLIT)
      return fail(LOOPKV_ERR_INVALID_ARG, "n_split %d outside [1, %d]", n_split, LOOPKV_MAX_SPLIT);
    if (n_seqs > 0 && !fixed_scratch && (!scratch || ((uintptr_t)scratch & 15u) != 0))
      return fail(LOOPKV_ERR_WORKSPACE, "split scratch is null or not 16-byte aligned");
    const size_t need = lkv::split_scratch_floats((size_t)count * n_seqs * c->cfg.n_heads, n_split, max_len,
                                                  c->cfg.head_dim) * sizeof(float);
    if (n_seqs > 0 && scratch_bytes < need)
      return fail(LOOPKV_ERR_WORKSPACE, "split scratch of %zu bytes, this call needs %zu", scratch_bytes, need);
  }
  if (n_seqs == 0) return ok();
  if (!q || !out || !block_table || !seq_lens) return fail(LOOPKV_ERR_INVALID_ARG, "null device pointer");
  lkv::DecodeArgs a;
  std::memset(&a, 0, sizeof(a));
  a.ws = c->ws;
  a.q = q;
  a.out = out;
  a.sel_mask = sel_mask;
  a.seq_slots = seq_slots;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.q_bf16 = q_dtype == LOOPKV_BF16;
  a.out_bf16 = out_dtype == LOOPKV_BF16;
  a.n_seqs = n_seqs;
  a.n_heads = c->cfg.n_heads;
  a.n_kv_heads = c->kvh;
  a.bt_stride = bt_stride;
  a.bt_shift = c->cfg.block_tokens == 32 ? 1 : 0;
  a.group = c->cfg.group_size;
  a.num_pages = c->cfg.num_blocks;
  a.max_seqs = c->cfg.max_seqs;
  a.max_len = max_len;
  a.sel_words = (max_len + 31) / 32;
  a.n_cells = count;
  a.tau = tau;
  a.sm_scale = sm_scale;
  a.n_split = n_split;
  a.skip = skip ? 1 : 0;
  if (app_k) {   // serving step: the row's workgroup appends the step's token first
    a.app_k = app_k;
    a.app_v = app_v;
    a.app_lens = app_lens;
    a.app_bf16 = app_dtype == LOOPKV_BF16;
  }
  for (int i = 0; i < count; ++i) {
    const int st = c->storage[first + i];
    a.cells[i].pool_off = c->pool_off[st];
    a.cells[i].tail_off = c->tail_off[st];
    a.cells[i].kind = device_kind(c, st);
  }
  s = check_device();
  if (s != LOOPKV_OK) return s;
  if (n_split > 0 && fixed_scratch) {   // every host check has passed: now the device address
    s = noalloc_scratch(&scratch);
    if (s != LOOPKV_OK) return s;
  }
  if (n_split > 0) {
    const size_t rows = (size_t)count * n_seqs * c->cfg.n_heads;
    a.split_row_stride = (int32_t)lkv::split_row_stride(max_len);
    a.part = static_cast<float*>(scratch);
    a.part_scores = a.part + lkv::split_part_floats(rows, n_split, c->cfg.head_dim);
  }
  hipError_t e = c->big ? lkv::launch_decode_big(a, c->cfg.head_dim, stream)
                         : lkv::launch_decode_small(a, c->cfg.head_dim, stream);
  if (e != hipSuccess) return fail(LOOPKV_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
  return ok();
}
}  // namespace

extern "C" {

loopkv_status loopkv_decode_attn(loopkv_ctx* c, hipStream_t stream, int32_t loop, int32_t layer, const void* q,
                                 int32_t q_dtype, int32_t n_seqs, const int32_t* seq_slots,
                                 const int32_t* block_table, int32_t bt_stride, const int32_t* seq_lens,
                                 int32_t max_len, float tau, float sm_scale, void* out, int32_t out_dtype,
                                 uint32_t* sel_mask) {
  return decode_common(c, stream, loop, layer, q, q_dtype, n_seqs, seq_slots, block_table, bt_stride, seq_lens,
                       max_len, tau, sm_scale, out, out_dtype, sel_mask, 0, nullptr, 0, false);
}

loopkv_status loopkv_decode_attn_skip(loopkv_ctx* c, hipStream_t stream, int32_t loop, int32_t layer, const void* q,
                                      int32_t q_dtype, int32_t n_seqs, const int32_t* seq_slots,
                                      const int32_t* block_table, int32_t bt_stride, const int32_t* seq_lens,
                                      int32_t max_len, float tau, float sm_scale, void* out, int32_t out_dtype,
                                      uint32_t* sel_mask) {
  return decode_common(c, stream, loop, layer, q, q_dtype, n_seqs, seq_slots, block_table, bt_stride, seq_lens,
                       max_len, tau, sm_scale, out, out_dtype, sel_mask, 0, nullptr, 0, true);
}

loopkv_status loopkv_split_scratch_bytes(const loopkv_ctx* c, int32_t loop, int32_t layer, int32_t n_seqs,
                                         int32_t max_len, int32_t n_split, size_t* bytes) {
  if (!c || !bytes) return fail(LOOPKV_ERR_INVALID_ARG, "null argument");
  if (!c->has_plan) return fail(LOOPKV_ERR_PLAN, "no plan loaded");
  int first, count;
  loopkv_status s = resolve_cells(c, loop, layer, &first, &count);
  if (s != LOOPKV_OK) return s;
  if (n_seqs < 0) return fail(LOOPKV_ERR_INVALID_ARG, "n_seqs must be >= 0");
  if (max_len < 0 || max_len > LOOPKV_MAX_LEN)
    return fail(LOOPKV_ERR_CAPACITY, "max_len %d outside [0, %d]", max_len, LOOPKV_MAX_LEN);
  if (n_split < 1 || n_split > LOOPKV_MAX_SPLIT)
    return fail(LOOPKV_ERR_INVALID_ARG, "n_split %d outside [1, %d]", n_split, LOOPKV_MAX_SPLIT);
  *bytes = lkv::split_scratch_floats((size_t)count * n_seqs * c->cfg.n_heads, n_split, max_len, c->cfg.head_dim) *
           sizeof(float);
  return ok();
}

loopkv_status loopkv_decode_attn_split(loopkv_ctx* c, hipStream_t stream, int32_t loop, int32_t layer,
                                       const void* q, int32_t q_dtype, int32_t n_seqs, const int32_t* seq_slots,
                                       const int32_t* block_table, int32_t bt_stride, const int32_t* seq_lens,
                                       int32_t max_len, float tau, float sm_scale, void* out, int32_t out_dtype,
                                       uint32_t* sel_mask, int32_t n_split, void* scratch, size_t scratch_bytes) {
  if (n_split == 0) return fail(LOOPKV_ERR_INVALID_ARG, "n_split %d outside [1, %d]", n_split, LOOPKV_MAX_SPLIT);
  return decode_common(c, stream, loop, layer, q, q_dtype, n_seqs, seq_slots, block_table, bt_stride, seq_lens,
                       max_len, tau, sm_scale, out, out_dtype, sel_mask, n_split, scratch, scratch_bytes, false);
}

loopkv_status loopkv_decode_attn_split_noalloc(loopkv_ctx* c, hipStream_t stream, int32_t loop, int32_t layer,
                                               const void* q, int32_t q_dtype, int32_t n_seqs,
                                               const int32_t* seq_slots, const int32_t* block_table,
                                               int32_t bt_stride, const int32_t* seq_lens, int32_t max_len,
                                               float tau, float sm_scale, void* out, int32_t out_dtype,
                                               uint32_t* sel_mask, int32_t n_split) {
  if (n_split == 0) return fail(LOOPKV_ERR_INVALID_ARG, "n_split %d outside [1, %d]", n_split, LOOPKV_MAX_SPLIT);
  size_t need = 0;
  loopkv_status s = loopkv_split_scratch_bytes(c, loop, layer, n_seqs, max_len, n_split, &need);
  if (s != LOOPKV_OK) return s;
  if (need > LOOPKV_NOALLOC_SCRATCH_BYTES)
    return fail(LOOPKV_ERR_WORKSPACE,
                "this call needs %zu bytes of split scratch, above the %u-byte fixed array of the "
                "no-allocation decode (fewer sequences, cells, splits or a shorter max_len fit)",
                need, (unsigned)LOOPKV_NOALLOC_SCRATCH_BYTES);
  // the array's device address is resolved inside, after every host check
  return decode_common(c, stream, loop, layer, q, q_dtype, n_seqs, seq_slots, block_table, bt_stride, seq_lens,
                       max_len, tau, sm_scale, out, out_dtype, sel_mask, n_split, nullptr,
                       LOOPKV_NOALLOC_SCRATCH_BYTES, false, true);
}

}  // extern "C"

// ----------------------------------------------------------------------------- step graph
struct loopkv_step_graph {
  hipGraphExec_t exec = nullptr;
};

namespace {
size_t dtype_bytes(int32_t dt) { return dt == LOOPKV_BF16 ? 2 : 4; }

// Enqueue one serving step on a stream (the body of the captured graph).
loopkv_status enqueue_step(loopkv_ctx* c, hipStream_t s, const uint8_t* k, const uint8_t* v, int32_t kv_dtype,
                           const uint8_t* q, int32_t q_dtype, int32_t n_seqs, const int32_t* seq_slots,
                           const int32_t* block_table, int32_t bt_stride, int32_t* before, int32_t* after,
                           int32_t max_len, float tau, float sm_scale, uint8_t* out, int32_t out_dtype,
                           uint32_t* sel_mask, int32_t n_split, void* scratch, size_t scratch_bytes) {
  const int D = c->cfg.head_dim, H = c->cfg.n_heads, L = c->cfg.n_loops, NL = c->cfg.n_layers;
  const size_t kv_cell = (size_t)n_seqs * c->kvh * D * dtype_bytes(kv_dtype);
  const size_t q_cell = (size_t)n_seqs * H * D * dtype_bytes(q_dtype);
  const size_t o_cell = (size_t)n_seqs * H * D * dtype_bytes(out_dtype);
  const size_t m_cell = (size_t)n_seqs * H * ((max_len + 31) / 32);
  // With one query head per KV head, a storing cell's append runs inside its decode launch:
  // the workgroup of each (sequence, KV head) appends the token and then decodes the row (in a
  // split decode, the last split's workgroup, which alone reads the appended token's group).
  // With grouped queries several rows read one KV head, so the append is its own launch.
  const bool fuse = c->kvh == H;
  for (int i = 0; i < L * NL; ++i) {
    const int loop = i / NL, layer = i % NL;
    const bool share = c->kinds[i] == LOOPKV_CELL_SHARE;
    loopkv_status st;
    if (!share && !fuse) {
      st = loopkv_append(c, s, loop, layer, k + i * kv_cell, v + i * kv_cell, kv_dtype, n_seqs, 1, seq_slots,
                         block_table, bt_stride, before);
      if (st != LOOPKV_OK) return st;
    }
    const bool app = !share && fuse;
    st = decode_common(c, s, loop, layer, q + i * q_cell, q_dtype, n_seqs, seq_slots, block_table, bt_stride,
                       share ? before : after, max_len, tau, sm_scale, out + i * o_cell, out_dtype,
                       sel_mask ? sel_mask + i * m_cell : nullptr, n_split, scratch, scratch_bytes, false, false,
                       app ? k + i * kv_cell : nullptr, app ? v + i * kv_cell : nullptr, kv_dtype,
                       app ? before : nullptr);
    if (st != LOOPKV_OK) return st;
  }
  hipError_t e = lkv::launch_advance_lens(before, after, n_seqs, s);
  if (e != hipSuccess) return fail(LOOPKV_ERR_HIP, "length update launch: %s", hipGetErrorString(e));
  return ok();
}
}  // namespace

extern "C" {

loopkv_status loopkv_step_graph_create(loopkv_ctx* c, const void* k, const void* v, int32_t kv_dtype, const void* q,
                                       int32_t q_dtype, int32_t n_seqs, const int32_t* seq_slots,
                                       const int32_t* block_table, int32_t bt_stride, int32_t* seq_lens_before,
                                       int32_t* seq_lens_after, int32_t max_len, float tau, float sm_scale,
                                       void* out, int32_t out_dtype, uint32_t* sel_mask, int32_t n_split,
                                       void* scratch, size_t scratch_bytes, loopkv_step_graph** graph) {
  if (!graph) return fail(LOOPKV_ERR_INVALID_ARG, "null graph pointer");
  *graph = nullptr;
  loopkv_status s = check_ready(c);
  if (s != LOOPKV_OK) return s;
  if (n_seqs < 1) return fail(LOOPKV_ERR_INVALID_ARG, "a step graph needs n_seqs >= 1");
  if (!k || !v || !q || !out || !block_table || !seq_lens_before || !seq_lens_after)
    return fail(LOOPKV_ERR_INVALID_ARG, "null device pointer");
  if (seq_lens_before == seq_lens_after)
    return fail(LOOPKV_ERR_INVALID_ARG, "seq_lens_before and seq_lens_after must be distinct arrays");
  if (kv_dtype != LOOPKV_F32 && kv_dtype != LOOPKV_BF16) return fail(LOOPKV_ERR_INVALID_ARG, "bad kv dtype %d", kv_dtype);
  if (q_dtype != LOOPKV_F32 && q_dtype != LOOPKV_BF16) return fail(LOOPKV_ERR_INVALID_ARG, "bad q dtype %d", q_dtype);
  if (out_dtype != LOOPKV_F32 && out_dtype != LOOPKV_BF16)
    return fail(LOOPKV_ERR_INVALID_ARG, "bad out dtype %d", out_dtype);
  if (!seq_slots && n_seqs > c->cfg.max_seqs)
    return fail(LOOPKV_ERR_CAPACITY, "n_seqs %d > max_seqs %d with identity slots", n_seqs, c->cfg.max_seqs);
  if (max_len < 1 || max_len > LOOPKV_MAX_LEN)
    return fail(LOOPKV_ERR_CAPACITY, "max_len %d outside [1, %d]", max_len, LOOPKV_MAX_LEN);
  if (bt_stride < 1 || (long long)bt_stride * c->cfg.block_tokens < max_len)
    return fail(LOOPKV_ERR_CAPACITY, "bt_stride %d too small for max_len %d", bt_stride, max_len);
  if (!(tau >= 0.f)) return fail(LOOPKV_ERR_INVALID_ARG, "tau must be >= 0 (got %g)", (double)tau);
  if (!(sm_scale > 0.f) || !std::isfinite(sm_scale))
    return fail(LOOPKV_ERR_INVALID_ARG, "sm_scale must be finite and > 0 (got %g)", (double)sm_scale);
  if (n_split != 0) {
    if (n_split < 1 || n_split > LOOPKV_MAX_SPLIT)
      return fail(LOOPKV_ERR_INVALID_ARG, "n_split %d outside [1, %d]", n_split, LOOPKV_MAX_SPLIT);
    const size_t need = lkv::split_scratch_floats((size_t)n_seqs * c->cfg.n_heads, n_split, max_len,
                                                  c->cfg.head_dim) * sizeof(float);
    if (!scratch || ((uintptr_t)scratch & 15u) != 0 || scratch_bytes < need)
      return fail(LOOPKV_ERR_WORKSPACE, "split scratch null, unaligned or below %zu bytes", need);
  }

  // every check passed: capture on a private stream (default priority)
  s = check_device();   // before the capture: no property query inside it
  if (s != LOOPKV_OK) return s;
  if (c->big) lkv::prepare_decode_big(c->cfg.head_dim, c->cfg.group_size);
  else lkv::prepare_decode_small(c->cfg.head_dim, c->cfg.group_size);
  hipStream_t cap = nullptr;
  hipError_t e = hipStreamCreateWithFlags(&cap, hipStreamNonBlocking);
  if (e != hipSuccess) return fail(LOOPKV_ERR_HIP, "capture stream: %s", hipGetErrorString(e));
  e = hipStreamBeginCapture(cap, hipStreamCaptureModeThreadLocal);
  if (e != hipSuccess) {
    (void)hipStreamDestroy(cap);
    return fail(LOOPKV_ERR_HIP, "begin capture: %s", hipGetErrorString(e));
  }
  s = enqueue_step(c, cap, static_cast<const uint8_t*>(k), static_cast<const uint8_t*>(v), kv_dtype,
                   static_cast<const uint8_t*>(q), q_dtype, n_seqs, seq_slots, block_table, bt_stride,
                   seq_lens_before, seq_lens_after, max_len, tau, sm_scale, static_cast<uint8_t*>(out), out_dtype,
                   sel_mask, n_split, scratch, scratch_bytes);
  const std::string err = g_err;
  hipGraph_t g = nullptr;
  e = hipStreamEndCapture(cap, &g);
  (void)hipStreamDestroy(cap);
  if (s != LOOPKV_OK || e != hipSuccess || !g) {
    if (g) (void)hipGraphDestroy(g);
    if (s != LOOPKV_OK) return fail(s, "%s", err.c_str());
    return fail(LOOPKV_ERR_HIP, "end capture: %s", hipGetErrorString(e));
  }
  hipGraphExec_t exec = nullptr;
  e = hipGraphInstantiate(&exec, g, nullptr, nullptr, 0);
  (void)hipGraphDestroy(g);
  if (e != hipSuccess) return fail(LOOPKV_ERR_HIP, "graph instantiation: %s", hipGetErrorString(e));
  loopkv_step_graph* out_g = new loopkv_step_graph();
  out_g->exec = exec;
  *graph = out_g;
  return ok();
}

loopkv_status loopkv_step_graph_launch(loopkv_step_graph* graph, hipStream_t stream) {
  if (!graph || !graph->exec) return fail(LOOPKV_ERR_INVALID_ARG, "null step graph");
  hipError_t e = hipGraphLaunch(graph->exec, stream);
  if (e != hipSuccess) return fail(LOOPKV_ERR_HIP, "graph launch: %s", hipGetErrorString(e));
  return ok();
}

void loopkv_step_graph_destroy(loopkv_step_graph* graph) {
  if (!graph) return;
  if (graph->exec) (void)hipGraphExecDestroy(graph->exec);
  delete graph;
}

}  // extern "C"
