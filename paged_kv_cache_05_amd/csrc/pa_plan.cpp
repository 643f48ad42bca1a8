// Host-side launch planning (declared in pa_plan.h).  No HIP, no heap: the
// sorts below work in fixed buffers on the stack, so a planned launch
// allocates nothing.
#include "pa_plan.h"

#include <algorithm>

namespace pa {
namespace {

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Stable merge sort of a[0..n) in the order `before` (a strict weak
// order), through tmp[0..n).  Bottom-up, so no recursion and no allocation.
template <class T, class Before>
void stable_sort_fixed(T *a, T *tmp, int n, Before before) {
  for (int w = 1; w < n; w *= 2) {
    for (int lo = 0; lo < n; lo += 2 * w) {
      const int mid = std::min(lo + w, n), hi = std::min(lo + 2 * w, n);
      int i = lo, j = mid, k = lo;
      // the right run's element goes first only when strictly before
      while (i < mid && j < hi) tmp[k++] = before(a[j], a[i]) ? a[j++] : a[i++];
      while (i < mid) tmp[k++] = a[i++];
      while (j < hi) tmp[k++] = a[j++];
    }
    std::copy(tmp, tmp + n, a);
  }
}

}  // namespace

WorkspaceLayout decode_workspace_layout(int num_seqs, int num_heads, int head_dim,
                                        int num_partitions) {
  WorkspaceLayout w{};
  const size_t rows = (size_t)num_seqs * num_heads;
  const size_t parts = rows * (size_t)num_partitions;
  w.ml_off = 0;
  w.o_off = align256(parts * 2 * sizeof(float));
  w.total = w.o_off + align256(parts * (size_t)head_dim * sizeof(float));
  return w;
}

int clamp_ctx(int32_t c, int max_context_len) {
  return c < 0 ? 0 : (c > max_context_len ? max_context_len : c);
}

int num_partitions(int max_context_len, int part) {
  return max_context_len <= 0 ? 1 : (max_context_len + part - 1) / part;
}

// Measured on 256 sequences of 20..200 tokens (fused step): 4 waves 12-23%
// faster than 8 at B = 8 / 16 / 64, and 2-6% faster than 2 waves; 8 waves
// best on the lognormal batch (median 300 tokens).  Keeping short items in
// (sequence, partition) order keeps neighbouring sequences (for instance
// parallel samples sharing prompt blocks) close in time and mixes sizes.
bool plan_work(const int32_t *host_ctx, int num_seqs, int max_context_len, int part,
               WorkList *items, WorkList *merge_rows, int *waves) {
  if (num_seqs < 0 || part <= 0) return false;
  int total = 0;
  long long tokens = 0;
  for (int b = 0; b < num_seqs; ++b) {
    const int c = clamp_ctx(host_ctx[b], max_context_len);
    total += c == 0 ? 1 : (c + part - 1) / part;
    tokens += c;
    if (total > kMaxListed) return false;
  }
  struct Entry {
    int tokens;
    uint32_t item;
  };
  Entry e[kMaxListed], tmp[kMaxListed];
  int n = 0;
  merge_rows->count = 0;
  for (int b = 0; b < num_seqs; ++b) {
    const int c = clamp_ctx(host_ctx[b], max_context_len);
    const int np = c == 0 ? 1 : (c + part - 1) / part;
    if (b > 0xffff || np - 1 > 0xffff) return false;
    for (int q = 0; q < np; ++q)
      e[n++] = Entry{std::min(part, c - q * part), ((uint32_t)b << 16) | (uint32_t)q};
    if (np > 1) merge_rows->item[merge_rows->count++] = (uint32_t)b;
  }
  items->count = n;
  if (n == 0) {
    *waves = 8;
    return true;
  }
  // Long items (more than twice the mean) first, longest first, stably.
  const long long long_item = 2 * tokens / n;
  int n_long = 0;
  for (int i = 0; i < n; ++i)
    if ((long long)e[i].tokens > long_item) tmp[n_long++] = e[i];
  int k = n_long;
  for (int i = 0; i < n; ++i)
    if ((long long)e[i].tokens <= long_item) tmp[k++] = e[i];
  std::copy(tmp, tmp + n, e);
  stable_sort_fixed(e, tmp, n_long,
                    [](const Entry &x, const Entry &y) { return x.tokens > y.tokens; });
  for (int i = 0; i < n; ++i) items->item[i] = e[i].item;
  constexpr long long kShortItemTokens = 12 * 16;
  *waves = (long long)n * kShortItemTokens > tokens ? 4 : 8;
  return true;
}

int plan_partition(const int32_t *host_ctx, int num_seqs, int num_heads, int head_dim,
                   int max_context_len, size_t workspace_bytes, bool have_workspace) {
  constexpr long long kPlanTargetItems = 2048;
  constexpr int kPlanMinPartition = 256;
  int part = 4096;
  for (;;) {
    long long items = 0;
    for (int b = 0; b < num_seqs; ++b) {
      const int c = clamp_ctx(host_ctx[b], max_context_len);
      items += (long long)num_heads * (c == 0 ? 1 : (c + part - 1) / part);
    }
    const int next = part / 2;
    if (items >= kPlanTargetItems || next < kPlanMinPartition) break;
    const int np = num_partitions(max_context_len, next);
    if (np > 1 && (!have_workspace ||
                   decode_workspace_layout(num_seqs, num_heads, head_dim, np).total >
                       workspace_bytes))
      break;
    part = next;
  }
  return part;
}

bool plan_prefill(const int32_t *hqs, const int32_t *hctx, int num_seqs, int max_context_len,
                  int max_query_len, int query_tile, PrefillPlan *out) {
  out->count = 0;
  if (num_seqs < 0 || query_tile <= 0 || max_query_len < 0) return false;
  const int64_t max_tiles = ((int64_t)max_query_len + query_tile - 1) / query_tile;
  int64_t seq_weight[kMaxListed];
  int n = 0;
  for (int b = 0; b < num_seqs; ++b) {
    const int64_t m = (int64_t)hqs[b + 1] - hqs[b];
    if (m <= 0) continue;
    const int64_t c = hctx ? std::min<int64_t>(std::max<int32_t>(hctx[b], 0), max_context_len)
                           : m;
    const int64_t tiles = std::min<int64_t>((m + query_tile - 1) / query_tile, max_tiles);
    const int first = n;
    int64_t heaviest = INT64_MIN;
    for (int64_t t = 0; t < tiles; ++t) {
      if (n >= kMaxListed || b > 0xffff || t > 0xffff) return false;
      const int64_t work = c - m + std::min<int64_t>(m, (t + 1) * query_tile);
      out->item[n++] = PrefillItem{(uint32_t)b << 16 | (uint32_t)t, work};
      heaviest = std::max(heaviest, work);
    }
    for (int i = first; i < n; ++i) seq_weight[i] = heaviest;
  }
  out->count = n;
  // Sequence-major: sequences by their heaviest tile, descending, and each
  // sequence's tiles heaviest first.  The tiles of one sequence then run
  // together and share the K/V rows they stream in the L2.  Indices are
  // sorted (small stack buffers), then the items are permuted.
  uint16_t idx[kMaxListed], tmp[kMaxListed];
  for (int i = 0; i < n; ++i) idx[i] = (uint16_t)i;
  const PrefillItem *it = out->item;
  stable_sort_fixed(idx, tmp, n, [&](uint16_t a, uint16_t b) {
    const uint32_t sa = it[a].code >> 16, sb = it[b].code >> 16;
    if (sa != sb)
      return seq_weight[a] != seq_weight[b] ? seq_weight[a] > seq_weight[b] : sa < sb;
    return it[a].work > it[b].work;
  });
  PrefillItem sorted[kMaxListed];
  for (int i = 0; i < n; ++i) sorted[i] = it[idx[i]];
  std::copy(sorted, sorted + n, out->item);
  return true;
}

// Measured on 40 heads x 128 (single prompts of 1024..4096 tokens, one or a
// few; suffixes of 64..256 queries over 2048..8192 cached tokens): shorter
// tiles, shorter chunks or more than two workgroups per CU cost full
// prompts time (partial results are fp32 rows of 512 bytes per query and
// head, written and read back).
bool plan_prefill_split(const PrefillPlan &list, int num_heads, int resident, int groups_per_cu,
                        int key_tile, size_t slots, SplitList *split, SplitList *merges) {
  const int n = list.count;
  if (n <= 0 || n > kMaxListed || resident <= 0 || groups_per_cu <= 0 || key_tile <= 0 ||
      num_heads <= 0 || slots < 2)
    return false;
  constexpr int64_t kMinSplitTiles = 48, kMinChunkTiles = 16;
  int64_t free_groups = (int64_t)resident * 2 / groups_per_cu - (int64_t)n * num_heads;
  if (free_groups < num_heads) return false;
  int chunks[kMaxListed];
  int64_t tiles[kMaxListed];
  int heap[kMaxListed];
  for (int i = 0; i < n; ++i) {
    chunks[i] = 1;
    tiles[i] = (list.item[i].work + key_tile - 1) / key_tile;
    heap[i] = i;
  }
  // largest current chunk first (tiles / chunks, rounded up)
  auto chunk_len = [&](int i) { return (tiles[i] + chunks[i] - 1) / chunks[i]; };
  auto less = [&](int a, int b) { return chunk_len(a) < chunk_len(b); };
  int live = n;
  std::make_heap(heap, heap + live, less);
  size_t used = 0;
  while (live > 0 && free_groups >= num_heads) {
    std::pop_heap(heap, heap + live, less);
    const int i = heap[--live];
    const int nc = chunks[i] + 1;
    const size_t need = nc == 2 ? 2 : 1;   // slots this step takes
    if (tiles[i] < kMinSplitTiles || nc > kMaxChunks || tiles[i] / nc < kMinChunkTiles ||
        used + need > slots)
      continue;
    chunks[i] = nc;
    used += need;
    free_groups -= num_heads;
    heap[live++] = i;
    std::push_heap(heap, heap + live, less);
  }
  if (used == 0) return false;
  int entries = 0;
  for (int i = 0; i < n; ++i) entries += chunks[i];
  if (entries > kMaxSplitItems || used > (1u << 24)) return false;
  split->count = 0;
  merges->count = 0;
  uint32_t slot = 0;
  for (int i = 0; i < n; ++i) {
    const int nc = chunks[i];
    for (int c = 0; c < nc; ++c) {
      split->item[split->count] = list.item[i].code;
      split->part[split->count] =   // each chunk its own slot: slot + c
          nc > 1 ? ((slot + (uint32_t)c) << 8 | (uint32_t)c << 4 | (uint32_t)(nc - 1)) : 0u;
      ++split->count;
    }
    if (nc > 1) {
      merges->item[merges->count] = list.item[i].code;
      merges->part[merges->count] = slot << 8 | (uint32_t)(nc - 1);
      ++merges->count;
      slot += (uint32_t)nc;
    }
  }
  return true;
}

}  // namespace pa
