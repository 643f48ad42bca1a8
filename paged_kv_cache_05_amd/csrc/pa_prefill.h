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
  // Split launch only: partial results of key chunks, per slot
  // [slot][head][128 rows][head_dim] fp32 (output before normalisation) and
  // [slot][head][128 rows] (running max in log2 units, sum).
  float *part_o;
  float2 *part_ml;
  int num_heads;
  int num_blocks;
  int max_blocks_per_seq;
  int max_context_len;
  int num_query_rows;
  float scale_log2;
};

int prefill_query_tile();
int prefill_key_tile();
// Workspace bytes of one partial-result slot.
size_t prefill_slot_bytes(int num_heads, int head_dim);
// Workgroups of the prefill kernel that one CU holds at once.
int prefill_groups_per_cu();
// items: (sequence << 16 | query tile) in launch order, or nullptr for the
// grid over (heads, tiles, sequences).  split / merges: the split form
// (items unused).
hipError_t launch_prefill(const PrefillParams &p, int num_seqs, int head_dim, int block_size,
                          int max_query_len, const WorkList *items, const SplitList *split,
                          const SplitList *merges, hipStream_t stream);

}  // namespace pa
