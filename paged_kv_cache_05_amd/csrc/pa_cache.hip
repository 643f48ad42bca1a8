// KV-cache maintenance kernels: the per-step slot write and the
// copy-on-write block copy.  Both move bits (16-byte vector copies), so the
// element type only matters through the row size.
//
//  * write_kv: each decoding step produces K and V for the new token only,
//    stored at the next free position of the sequence's last block (the
//    wywy.jp notes on PagedAttention, Keyword "autoregressive generation
//    phase" and "KV cache manager"; zhaifeiyue.github.io summary, "KV Cache
//    Manager" paragraph).  The caller's manager turns that position into a
//    slot = physical_block * B + offset.
//  * copy_blocks: when a block shared by several sequences (reference count
//    above 1) is about to be written, the manager allocates a new block and
//    the block engine copies the old one into it (wywy.jp WHERE, the
//    parallel-sampling example with physical blocks 1 and 3; zhaifeiyue
//    memory-management table, "Copy-on-Write").
//  * swap_blocks: swapping moves every block of an evicted sequence from GPU
//    memory to CPU memory and back whole when it resumes (wywy.jp Keyword
//    "Swapping" and Overview, scheduling and preemption; zhaifeiyue
//    "Scheduling & Preemption" table, row "Swap").  The host pools are
//    pinned memory the GPU reaches directly, so the kernel itself moves the
//    bytes over PCIe: one launch for any number of blocks, instead of one
//    DMA transfer per block (the pages note that small blocks make swapping
//    slow through many small CPU-GPU transfers).
//
// With the [num_blocks][num_heads][block_size][head_dim] pool layout a whole
// block is one contiguous span, and a token row of one head is one contiguous
// row_bytes span, so all kernels are streams of aligned 16-byte moves.
#include "pa_kernels.h"

namespace pa {
namespace {

constexpr int kThreads = 256;

// One thread per 16-byte chunk of one (token, head) row: reads key and value
// chunk i (coalesced along the row), writes both pools at the slot.
__global__ void __launch_bounds__(kThreads)
write_kv_kernel(const uint4 *__restrict__ key, const uint4 *__restrict__ value,
                uint4 *__restrict__ k_pool, uint4 *__restrict__ v_pool,
                const int64_t *__restrict__ slot_mapping, int64_t total_chunks, int num_heads,
                int chunks_per_row, int block_size, int64_t num_slots) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= total_chunks) return;
  const int64_t token_head = i / chunks_per_row;
  const int c = (int)(i - token_head * chunks_per_row);
  const int64_t token = token_head / num_heads;
  const int h = (int)(token_head - token * num_heads);
  const int64_t slot = slot_mapping[token];
  if (slot < 0 || slot >= num_slots) return;  // padding, or outside the pool
  const int64_t block = slot / block_size;
  const int offset = (int)(slot - block * block_size);
  const int64_t dst = ((block * num_heads + h) * block_size + offset) * chunks_per_row + c;
  k_pool[dst] = key[i];
  v_pool[dst] = value[i];
}

// grid.x = block pair, grid.y strides over the block's 16-byte chunks.
// Copies block src of (src_k, src_v) onto block dst of (dst_k, dst_v); the
// copy-on-write copy passes the same pools on both sides.  Each thread keeps
// kUnroll chunks of K and of V in flight before storing them, which hides the
// latency of reads from host memory over PCIe.
constexpr int kUnroll = 4;

__global__ void __launch_bounds__(kThreads)
move_blocks_kernel(uint4 *dst_k, uint4 *dst_v, const uint4 *src_k, const uint4 *src_v,
                   const int64_t *__restrict__ block_mapping, int64_t chunks_per_block,
                   int64_t src_blocks, int64_t dst_blocks) {
  const int64_t pair = blockIdx.x;
  const int64_t src = block_mapping[2 * pair];
  const int64_t dst = block_mapping[2 * pair + 1];
  if (src < 0 || src >= src_blocks || dst < 0 || dst >= dst_blocks) return;
  const uint4 *ks = src_k + src * chunks_per_block;
  const uint4 *vs = src_v + src * chunks_per_block;
  uint4 *kd = dst_k + dst * chunks_per_block;
  uint4 *vd = dst_v + dst * chunks_per_block;
  const int64_t stride = (int64_t)gridDim.y * kThreads;
  int64_t c = (int64_t)blockIdx.y * kThreads + threadIdx.x;
  for (; c + (kUnroll - 1) * stride < chunks_per_block; c += kUnroll * stride) {
    uint4 a[kUnroll], b[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      a[u] = ks[c + u * stride];
      b[u] = vs[c + u * stride];
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      kd[c + u * stride] = a[u];
      vd[c + u * stride] = b[u];
    }
  }
  for (; c < chunks_per_block; c += stride) {
    const uint4 a = ks[c];
    const uint4 b = vs[c];
    kd[c] = a;
    vd[c] = b;
  }
}

}  // namespace

hipError_t launch_write_kv(const void *key, const void *value, void *k_pool, void *v_pool,
                           const int64_t *slot_mapping, int num_tokens, int num_heads,
                           int row_bytes, int block_size, int num_blocks, hipStream_t stream) {
  const int chunks_per_row = row_bytes / 16;
  const int64_t total = (int64_t)num_tokens * num_heads * chunks_per_row;
  const int64_t blocks = (total + kThreads - 1) / kThreads;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  write_kv_kernel<<<dim3((unsigned)blocks), kThreads, 0, stream>>>(
      static_cast<const uint4 *>(key), static_cast<const uint4 *>(value),
      static_cast<uint4 *>(k_pool), static_cast<uint4 *>(v_pool), slot_mapping, total, num_heads,
      chunks_per_row, block_size, (int64_t)num_blocks * block_size);
  return hipGetLastError();
}

hipError_t launch_move_blocks(void *dst_k, void *dst_v, const void *src_k, const void *src_v,
                              const int64_t *block_mapping, int num_pairs, size_t block_bytes,
                              int src_blocks, int dst_blocks, hipStream_t stream) {
  const int64_t chunks = (int64_t)(block_bytes / 16);
  int64_t ys = (chunks + kThreads - 1) / kThreads;
  if (ys > 64) ys = 64;  // each thread then copies several chunks
  move_blocks_kernel<<<dim3((unsigned)num_pairs, (unsigned)ys), kThreads, 0, stream>>>(
      static_cast<uint4 *>(dst_k), static_cast<uint4 *>(dst_v),
      static_cast<const uint4 *>(src_k), static_cast<const uint4 *>(src_v), block_mapping,
      chunks, (int64_t)src_blocks, (int64_t)dst_blocks);
  return hipGetLastError();
}

hipError_t launch_copy_blocks(void *k_pool, void *v_pool, const int64_t *block_mapping,
                              int num_pairs, size_t block_bytes, int num_blocks,
                              hipStream_t stream) {
  return launch_move_blocks(k_pool, v_pool, k_pool, v_pool, block_mapping, num_pairs,
                            block_bytes, num_blocks, num_blocks, stream);
}

}  // namespace pa
