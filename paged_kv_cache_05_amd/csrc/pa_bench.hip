// Reference read kernels for the benchmark: the bandwidth the decode's access
// pattern can reach on this GPU, with no attention arithmetic and no work
// structure.  Not part of the attention library (libpa.so); built into
// libpa_bench.so and declared in include/pa_bench.h.
//
//  * stream_read_kernel: one contiguous buffer read once, 16-byte
//    non-temporal loads, workgroups striding over tiles with 1 to 8 loads
//    in flight per thread.  The ceiling of a pure stream.
//  * gather_read_kernel: pieces of piece_bytes at caller-given byte offsets
//    in two pools (K and V), one wave per piece of each pool, read with the
//    same non-temporal 16-byte loads the decode uses.  Given the decode's
//    (block, head) tiles as pieces, it is the ceiling of the decode's
//    scattered reads with every other cost taken away.
//
// Both fold the words they read into a value that is stored only if it
// equals a constant no input produces in practice, so the loads cannot be
// removed and almost nothing is written.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "pa_bench.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t fold(u32x4 x) { return x.x ^ x.y ^ x.z ^ x.w; }

constexpr uint32_t kNever = 0x9E3779B9u;
constexpr int kStreamThreads = 256;

// Each workgroup reads tiles of 256 * U chunks (each thread U 16-byte
// chunks, U KiB contiguous per wave), tile blockIdx.x, then + gridDim.x,
// ...: at any time the grid covers one contiguous span.  U = 1 is the plain
// grid-stride loop.
template <int U>
__global__ void __launch_bounds__(kStreamThreads)
stream_read_kernel(const u32x4 *__restrict__ p, size_t n16, uint32_t *sink) {
  constexpr size_t kTile = (size_t)kStreamThreads * U;   // chunks per tile
  uint32_t acc = 0;
  for (size_t t0 = (size_t)blockIdx.x * kTile; t0 < n16; t0 += (size_t)gridDim.x * kTile) {
    u32x4 a[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t i = t0 + (size_t)u * kStreamThreads + threadIdx.x;
      a[u] = i < n16 ? __builtin_nontemporal_load(p + i) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= fold(a[u]);
  }
  if (acc == kNever) sink[blockIdx.x] = acc;
}

constexpr int kGatherWaves = 4;

__global__ void __launch_bounds__(64 * kGatherWaves)
gather_read_kernel(const char *__restrict__ k, const char *__restrict__ v, size_t pool_bytes,
                   const int64_t *__restrict__ offsets, int num_pieces, int piece_bytes,
                   uint32_t *sink) {
  const int lane = threadIdx.x & 63;
  const int piece = blockIdx.x * kGatherWaves + (int)(threadIdx.x >> 6);
  if (piece >= num_pieces) return;
  const int64_t off = offsets[piece];
  // a piece outside the pools is skipped, never read
  if (off < 0 || (uint64_t)off > pool_bytes - (uint64_t)piece_bytes) return;
  const int chunks = piece_bytes / 16;
  const u32x4 *kp = reinterpret_cast<const u32x4 *>(k + off);
  const u32x4 *vp = reinterpret_cast<const u32x4 *>(v + off);
  uint32_t acc = 0;
  // four chunks of each pool per lane in flight (a 4 KiB piece in one pass)
  for (int c0 = lane; c0 < chunks; c0 += 4 * 64) {
    u32x4 a[4], b[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = c0 + 64 * u;
      a[u] = c < chunks ? __builtin_nontemporal_load(kp + c) : u32x4{0, 0, 0, 0};
      b[u] = c < chunks ? __builtin_nontemporal_load(vp + c) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) acc ^= fold(a[u]) ^ fold(b[u]);
  }
  if (acc == kNever) sink[blockIdx.x] = acc;
}

int status_of(hipError_t e) { return e == hipSuccess ? 0 : -5; }

}  // namespace

extern "C" {

int pa_bench_stream_read(const void *buf, size_t bytes, int grid, int unroll, void *sink,
                         void *stream) {
  if (!buf || !sink) return -1;
  if (grid <= 0 || bytes % 16 != 0 || ((uintptr_t)buf & 15u) || ((uintptr_t)sink & 3u))
    return -2;
  if (bytes == 0) return 0;
  (void)hipGetLastError();
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const u32x4 *p = static_cast<const u32x4 *>(buf);
  uint32_t *out = static_cast<uint32_t *>(sink);
  switch (unroll) {
    case 1: stream_read_kernel<1><<<grid, kStreamThreads, 0, s>>>(p, bytes / 16, out); break;
    case 2: stream_read_kernel<2><<<grid, kStreamThreads, 0, s>>>(p, bytes / 16, out); break;
    case 4: stream_read_kernel<4><<<grid, kStreamThreads, 0, s>>>(p, bytes / 16, out); break;
    case 8: stream_read_kernel<8><<<grid, kStreamThreads, 0, s>>>(p, bytes / 16, out); break;
    default: return -2;
  }
  return status_of(hipGetLastError());
}

int pa_bench_gather_read(const void *k_pool, const void *v_pool, size_t pool_bytes,
                         const int64_t *offsets, int num_pieces, int piece_bytes, void *sink,
                         void *stream) {
  if (!k_pool || !v_pool || !offsets || !sink) return -1;
  if (num_pieces < 0 || piece_bytes <= 0 || piece_bytes % 16 != 0 ||
      (size_t)piece_bytes > pool_bytes || ((uintptr_t)k_pool & 15u) ||
      ((uintptr_t)v_pool & 15u) || ((uintptr_t)offsets & 7u) || ((uintptr_t)sink & 3u))
    return -2;
  if (num_pieces == 0) return 0;
  (void)hipGetLastError();
  const int grid = (num_pieces + kGatherWaves - 1) / kGatherWaves;
  gather_read_kernel<<<grid, 64 * kGatherWaves, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const char *>(k_pool), static_cast<const char *>(v_pool), pool_bytes, offsets,
      num_pieces, piece_bytes, static_cast<uint32_t *>(sink));
  return status_of(hipGetLastError());
}

}  // extern "C"
