// Launch interface of the paged prefill kernels (pa_prefill.hip).
#pragma once

#include "pa_kernels.h"

namespace pa {

// Paged prefill: rows query_start[b] .. query_start[b+1]-1 of q / out are the
// last tokens of sequence b's context.
struct PrefillParams {
  void *out;                      // [num_query_rows][num_heads][head_dim]
  const void *q;                  // same layout
  const void *k_pool;
  const void *v_pool;
  const int32_t *block_tables;
  const int32_t *context_lens;
  const int32_t *query_start;     // [num_seqs + 1]
  int num_heads;
  int num_blocks;
  int max_blocks_per_seq;
  int max_context_len;
  int num_query_rows;
  float scale_log2;
};

int prefill_query_tile();
// items: (sequence << 16 | query tile) in launch order, or nullptr for the
// grid over (heads, tiles, sequences).
hipError_t launch_prefill(const PrefillParams &p, int num_seqs, int head_dim, int block_size,
                          int max_query_len, const WorkList *items, hipStream_t stream);

}  // namespace pa
