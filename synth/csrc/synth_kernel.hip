// GPU side of the seeded input generator (no step of the attention method here).
//
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy
// as 1, 2, 3", SC'11) and the Irwin-Hall(12) normal draw defined in
// synth/philox.py: element i of stream s evaluates Philox at counters
// (i lo, i hi, s, 0) and (i lo, i hi, s, 1) under key (seed lo, seed hi); the
// first twelve 16-bit halves h_j give z = (sum h_j - 393210) / 65536 exactly;
// a scaled value is bf16_rne(z * f) with one float32 multiply.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__device__ inline void philox(uint32_t c[4], uint32_t k0, uint32_t k1) {
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t p0 = (uint64_t)0xD2511F53u * c[0];
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c[2];
    const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    const uint32_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
  }
}

__device__ inline float normal12(uint64_t seed, uint32_t stream, uint64_t i) {
  uint32_t a[4] = {(uint32_t)i, (uint32_t)(i >> 32), stream, 0u};
  uint32_t b[4] = {(uint32_t)i, (uint32_t)(i >> 32), stream, 1u};
  philox(a, (uint32_t)seed, (uint32_t)(seed >> 32));
  philox(b, (uint32_t)seed, (uint32_t)(seed >> 32));
  int32_t s = 0;
  for (int j = 0; j < 4; ++j) s += (int32_t)(a[j] & 0xffffu) + (int32_t)(a[j] >> 16);
  for (int j = 0; j < 2; ++j) s += (int32_t)(b[j] & 0xffffu) + (int32_t)(b[j] >> 16);
  return (float)(s - 393210) / 65536.0f;
}

__device__ inline uint16_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// out[((b * n_tok + i) * H + h) * D + d] for token t = t0 (or t0s[b]) + i, element
// index ((b * T + t) * H + h) * D + d, factor factors[h * D + d].
__global__ void k_kv(uint64_t seed, uint32_t stream, int B, int n_tok, int t0, const int32_t* t0s, int T, int H,
                     int D, const float* factors, uint16_t* out) {
  const size_t n = (size_t)B * n_tok * H * D;
  for (size_t o = (size_t)blockIdx.x * blockDim.x + threadIdx.x; o < n; o += (size_t)gridDim.x * blockDim.x) {
    const int d = (int)(o % D);
    const int h = (int)((o / D) % H);
    const int i = (int)((o / ((size_t)D * H)) % n_tok);
    const int b = (int)(o / ((size_t)D * H * n_tok));
    const int t = (t0s ? t0s[b] : t0) + i;
    const uint64_t idx = (((uint64_t)b * T + t) * H + h) * D + d;
    const float z = normal12(seed, stream, idx);
    out[o] = bf16_rne(__fmul_rn(z, factors[h * D + d]));
  }
}

__global__ void k_normal(uint64_t seed, uint32_t stream, uint64_t offset, size_t n, int as_bf16, void* out) {
  for (size_t o = (size_t)blockIdx.x * blockDim.x + threadIdx.x; o < n; o += (size_t)gridDim.x * blockDim.x) {
    const float z = normal12(seed, stream, offset + o);
    if (as_bf16) reinterpret_cast<uint16_t*>(out)[o] = bf16_rne(z);
    else reinterpret_cast<float*>(out)[o] = z;
  }
}

// Read-bandwidth probes (no method arithmetic): stream a buffer, or read chunk_bytes at
// the starts of records taken in the order of a permutation (the decode's access shape).
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// Streaming read: workgroup b reads its contiguous span [b, b + 1) * ceil(n16 / grid) of the
// buffer in workgroup-wide sweeps, eight nontemporal 16-byte loads per thread in flight (on
// MI355X this beat grid-stride reads by 3-7% and temporal loads by ~12%).
__global__ void k_stream_read(const u32x4_t* p, size_t n16, unsigned* out) {
  u32x4_t acc = {0u, 0u, 0u, 0u};
  const size_t span = (n16 + gridDim.x - 1) / gridDim.x;
  const size_t b0 = (size_t)blockIdx.x * span;
  const size_t e = b0 + span < n16 ? b0 + span : n16;
  const size_t step = blockDim.x;
  size_t i = b0 + threadIdx.x;
  for (; i + 7 * step < e; i += 8 * step) {
    u32x4_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(p + i + u * step);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u];
  }
  for (; i < e; i += step) acc ^= __builtin_nontemporal_load(p + i);
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

// Each wave reads whole chunks (up to 4096 bytes): wave k of the grid takes chunks k,
// k + waves, ...; chunk c starts at order[c] * record_bytes.
__global__ void k_chunk_read(const unsigned char* base, const unsigned* order, int n_chunks, int record_bytes,
                             int chunk_bytes, unsigned* out) {
  const int lane = threadIdx.x & 63;
  const int wave = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int waves = (gridDim.x * blockDim.x) >> 6;
  const int per = chunk_bytes / 16;
  u32x4_t acc = {0u, 0u, 0u, 0u};
  for (int c = wave; c < n_chunks; c += 4 * waves) {
    u32x4_t v[4][4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int cc = c + u * waves;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = lane + 64 * r;
        v[u][r] = (u32x4_t){0u, 0u, 0u, 0u};
        if (cc < n_chunks && i < per)
          v[u][r] = __builtin_nontemporal_load(
              reinterpret_cast<const u32x4_t*>(base + (size_t)order[cc] * record_bytes) + i);
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  out[blockIdx.x * blockDim.x + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

unsigned grid_for(size_t n) {
  size_t g = (n + 255) / 256;
  if (g > 65536) g = 65536;
  if (g == 0) g = 1;
  return (unsigned)g;
}
}  // namespace

extern "C" {

// K or V values of one cell as bf16 bits, in the append input layout [B][n_tok][H][D].
int synth_kv_bf16(hipStream_t s, uint64_t seed, uint32_t stream, int B, int n_tok, int t0, const int32_t* t0s,
                  int T, int H, int D, const float* factors, uint16_t* out) {
  const size_t n = (size_t)B * n_tok * H * D;
  if (n == 0) return 0;
  hipLaunchKernelGGL(k_kv, dim3(grid_for(n)), dim3(256), 0, s, seed, stream, B, n_tok, t0, t0s, T, H, D, factors, out);
  return (int)hipGetLastError();
}

// Streaming read of n16 16-byte words; out: one word per thread of a grid of 256-thread blocks.
int synth_stream_read(hipStream_t s, const void* p, size_t n16, int blocks, unsigned* out) {
  hipLaunchKernelGGL(k_stream_read, dim3(blocks), dim3(256), 0, s, (const u32x4_t*)p, n16, out);
  return (int)hipGetLastError();
}

// Chunk reads (chunk_bytes <= 4096, a multiple of 16) at permuted record starts (see k_chunk_read).
int synth_chunk_read(hipStream_t s, const void* base, const unsigned* order, int n_chunks, int record_bytes,
                     int chunk_bytes, int blocks, unsigned* out) {
  hipLaunchKernelGGL(k_chunk_read, dim3(blocks), dim3(256), 0, s, (const unsigned char*)base, order, n_chunks,
                     record_bytes, chunk_bytes, out);
  return (int)hipGetLastError();
}

// n consecutive draws starting at element offset, as bf16 bits or float32.
int synth_normal(hipStream_t s, uint64_t seed, uint32_t stream, uint64_t offset, size_t n, int as_bf16, void* out) {
  if (n == 0) return 0;
  hipLaunchKernelGGL(k_normal, dim3(grid_for(n)), dim3(256), 0, s, seed, stream, offset, n, as_bf16, out);
  return (int)hipGetLastError();
}
}
