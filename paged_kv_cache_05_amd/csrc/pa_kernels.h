// Internal interface between the C ABI (pa_api.hip) and the kernel files.
// Not installed; the public contract is include/pa.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "pa_plan.h"

namespace pa {

// Everything the decode kernel reads besides its template parameters.
struct DecodeParams {
  void *out;
  const void *q;
  const void *k_pool;
  const void *v_pool;
  const int32_t *block_tables;
  const int32_t *context_lens;
  int num_seqs;
  int num_heads;
  int num_blocks;
  int max_blocks_per_seq;
  int max_context_len;
  int partition_size;   // tokens per partition, multiple of 16
  int num_partitions;   // ceil(max_context_len / partition_size)
  float scale_log2;     // scale * log2(e): scores are kept in base 2
  float2 *part_ml;      // [num_seqs * num_heads][num_partitions] (max, sum)
  float *part_o;        // [num_seqs * num_heads][num_partitions][head_dim]
  // Fused append (all null for a plain decode): the new token of sequence b
  // (rows [b][h][:] of new_key / new_value) is stored at slot_mapping[b] and
  // is the token at position context_lens[b] - 1 of the attention.
  const void *new_key;
  const void *new_value;
  const int64_t *slot_mapping;
};

// dtype: 0 = f16, 1 = f32.  `items` (optional) lists the (sequence,
// partition) work items in launch order, `merge_rows` (optional, needed when
// items is given and num_partitions > 1) the sequences that span several
// partitions; `waves` (4 or 8) is the listed launch's waves per
// workgroup (the grid launch uses 8).  Returns the launch status.
hipError_t launch_decode(const DecodeParams &p, int num_seqs, int head_dim, int block_size,
                         int dtype, const WorkList *items, const WorkList *merge_rows,
                         int waves, hipStream_t stream);

hipError_t launch_write_kv(const void *key, const void *value, void *k_pool, void *v_pool,
                           const int64_t *slot_mapping, int num_tokens, int num_heads,
                           int row_bytes, int block_size, int num_blocks, hipStream_t stream);

hipError_t launch_copy_blocks(void *k_pool, void *v_pool, const int64_t *block_mapping,
                              int num_pairs, size_t block_bytes, int num_blocks,
                              hipStream_t stream);

// Block src of (src_k, src_v) onto block dst of (dst_k, dst_v), per pair;
// either side may be pinned host memory the GPU reaches at that address.
hipError_t launch_move_blocks(void *dst_k, void *dst_v, const void *src_k, const void *src_v,
                              const int64_t *block_mapping, int num_pairs, size_t block_bytes,
                              int src_blocks, int dst_blocks, hipStream_t stream);

}  // namespace pa
