// Host-side launch planning of the decode and prefill kernels.
//
// Plain C++: no HIP call and no heap allocation.  Every list is a
// fixed-size array that reaches the GPU by value as a kernel argument.  The
// planners are built into libpa.so and, with the address and
// undefined-behaviour sanitizers, into a CPU test driver that checks their
// invariants (tests/native/plan_check.cpp).
//
// Where the plans come from: the pages' central KV cache manager knows every
// sequence's length and sends each step's inputs to the workers (the
// wywy.jp notes, WHERE), so the host can list the non-empty work items of a
// step instead of launching a grid over the longest row.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace pa {

// A host-built work list, passed by value as kernel arguments (so it must
// stay under the 4 KiB argument limit together with the kernel's other
// parameters).  Each entry packs (sequence << 16) | partition (decode) or
// (sequence << 16) | query tile (prefill).
constexpr int kMaxListed = 960;
struct WorkList {
  int count;
  uint32_t item[kMaxListed];
};

// Launch list of the prefill's split form: each entry is one workgroup's
// (sequence, query tile) and its key chunk; part = slot << 8 | chunk << 4 |
// (chunks - 1) with the chunk's own workspace slot, 0 for a whole tile.  A
// tile's chunks use consecutive slots.  The merge list holds one entry per
// split tile: part = slot << 8 | (chunks - 1), slot being its first chunk's.
constexpr int kMaxSplitItems = 448;
constexpr int kMaxChunks = 16;
struct SplitList {
  int count;
  uint32_t item[kMaxSplitItems];   // sequence << 16 | query tile
  uint32_t part[kMaxSplitItems];
};

// Decode workspace carve-up: float2 (max, sum) per (row, partition), then
// the fp32 partial output rows, each part 256-byte aligned.
struct WorkspaceLayout {
  size_t ml_off, o_off, total;
};
WorkspaceLayout decode_workspace_layout(int num_seqs, int num_heads, int head_dim,
                                        int num_partitions);

// Context length clamped to [0, max_context_len], as the kernels clamp it.
int clamp_ctx(int32_t c, int max_context_len);

// ceil(max_context_len / part), at least 1.
int num_partitions(int max_context_len, int part);

// Decode work list from host-side context lengths: every non-empty
// (sequence, partition) item (one entry for an empty sequence, whose row is
// zeroed), and the sequences that span several partitions.  Items longer
// than twice the mean go first, longest first; the rest keep (sequence,
// partition) order.  *waves: 8, or 4 when the mean item is shorter than 12
// 16-token tiles.  False when either list would exceed kMaxListed (the
// caller then launches the grid).
bool plan_work(const int32_t *host_ctx, int num_seqs, int max_context_len, int part,
               WorkList *items, WorkList *merge_rows, int *waves);

// Partition length chosen from host-side lengths: start at 4096 tokens and
// halve while the batch offers fewer than 2048 (head, sequence, partition)
// items, down to 256, never to a length whose workspace exceeds
// workspace_bytes (or, without a workspace, never to more than one
// partition).
int plan_partition(const int32_t *host_ctx, int num_seqs, int num_heads, int head_dim,
                   int max_context_len, size_t workspace_bytes, bool have_workspace);

// One prefill query tile to launch: code = sequence << 16 | tile, work =
// the keys its last query sees.
struct PrefillItem {
  uint32_t code;
  int64_t work;
};
struct PrefillPlan {
  int count;
  PrefillItem item[kMaxListed];
};

// Every (sequence, query tile) the grid would cover, grouped by sequence:
// sequences by their heaviest tile, descending, and each sequence's tiles
// heaviest first.  hqs: host query_start [num_seqs + 1]; hctx (may be NULL):
// host context lengths.  False if there are more than kMaxListed tiles or a
// code does not fit 16 + 16 bits.
bool plan_prefill(const int32_t *hqs, const int32_t *hctx, int num_seqs, int max_context_len,
                  int max_query_len, int query_tile, PrefillPlan *out);

// Split plan of a prefill launch that would leave the GPU mostly idle: the
// tile whose current key chunk is longest takes one more chunk while idle
// workgroup slots remain (resident = workgroups the GPU holds at once,
// groups_per_cu of them per CU).  False when nothing is split or the lists
// would not fit; then the plain list is launched.
bool plan_prefill_split(const PrefillPlan &list, int num_heads, int resident, int groups_per_cu,
                        int key_tile, size_t slots, SplitList *split, SplitList *merges);

}  // namespace pa
