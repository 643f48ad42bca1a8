// C ABI of libpa.so: argument validation and dispatch to the kernels.  The
// contract (shapes, layouts, ownership, errors) is documented in
// include/pa.h; this file checks scalars and pointers only and never reads
// device memory.
#include <math.h>
#include <stdio.h>

#include <algorithm>
#include <atomic>
#include <vector>

#include "pa.h"
#include "pa_manager.h"
#include "pa_kernels.h"
#include "pa_prefill.h"

namespace {

constexpr int kMaxPartition = 65536;
constexpr int kGridYZ = 65535;

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

int elem_bytes(int dtype) {
  if (dtype == PA_F16) return 2;
  if (dtype == PA_F32) return 4;
  return 0;
}

bool supported_head_dim(int d) { return d == 64 || d == 128; }
bool supported_block(int b) { return b == 8 || b == 16 || b == 32 || b == 64; }

// Shared checks of the pool geometry.  0 or an error code.
int check_pool(int num_heads, int head_dim, int block_size, int num_blocks, int dtype) {
  if (!elem_bytes(dtype) || !supported_head_dim(head_dim) || !supported_block(block_size))
    return PA_ERR_UNSUPPORTED;
  if (num_heads <= 0 || num_blocks <= 0) return PA_ERR_SHAPE;
  return PA_OK;
}

// partition_size 0: PA_DEFAULT_PARTITION, or PA_LONG_PARTITION once the
// longest context exceeds PA_LONG_CONTEXT (fewer, longer partitions amortise
// each workgroup's epilogue when every row is long).
int effective_partition(int partition_size, int max_context_len) {
  if (partition_size != 0) return partition_size;
  return max_context_len > PA_LONG_CONTEXT ? PA_LONG_PARTITION : PA_DEFAULT_PARTITION;
}

bool valid_partition(int part) { return part >= 16 && part <= kMaxPartition && part % 16 == 0; }

int num_partitions(int max_context_len, int part) {
  return max_context_len <= 0 ? 1 : (max_context_len + part - 1) / part;
}

// Description of the last HIP error this library saw on the calling thread.
thread_local char t_detail[384] = "";

// hipGetLastError reports the last failure of any HIP call on the thread,
// so a launch first takes whatever an earlier call (of the caller, or of a
// framework around it) left behind; the status read after the launch then
// belongs to the launch.  Both are described for pa_last_error.
// True if the GPU can reach p at that address: device memory, or pinned
// host memory mapped at the same address.  Pageable host memory (which a
// kernel cannot touch without faulting) and managed memory are refused, and
// the reason goes to pa_last_error.
bool gpu_reachable(const void *p, const char *what) {
  hipPointerAttribute_t a{};
  const hipError_t e = hipPointerGetAttributes(&a, p);
  if (e != hipSuccess) {
    (void)hipGetLastError();  // do not leave the query's failure pending
    snprintf(t_detail, sizeof t_detail,
             "%s is not memory the HIP runtime knows (%s): pageable host memory is not "
             "reachable by the GPU; use device or pinned host memory",
             what, hipGetErrorName(e));
    return false;
  }
  if (a.type == hipMemoryTypeDevice) return true;
  if (a.type == hipMemoryTypeHost && a.devicePointer == p) return true;
  snprintf(t_detail, sizeof t_detail,
           "%s: memory type %d (device pointer %p for %p) is neither device memory nor pinned "
           "host memory at the same address",
           what, (int)a.type, a.devicePointer, p);
  return false;
}

template <class Launch>
int launch_checked(const char *what, Launch &&launch) {
  const hipError_t stale = hipGetLastError();
  const hipError_t e = launch();
  if (e != hipSuccess) {
    snprintf(t_detail, sizeof t_detail, "%s: %s (%s)%s%s", what, hipGetErrorName(e),
             hipGetErrorString(e),
             stale != hipSuccess ? "; an earlier HIP call on this thread had failed with " : "",
             stale != hipSuccess ? hipGetErrorName(stale) : "");
  } else if (stale != hipSuccess) {
    snprintf(t_detail, sizeof t_detail,
             "%s launched; it cleared the error %s (%s) that an earlier HIP call on this "
             "thread had left",
             what, hipGetErrorName(stale), hipGetErrorString(stale));
  }
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

int clamp_ctx(int32_t c, int max_context_len) {
  return c < 0 ? 0 : (c > max_context_len ? max_context_len : c);
}

// Work list from host-side context lengths: every (sequence, partition)
// with at least one token (one entry for an empty sequence, whose row is
// zeroed); and the sequences that span several partitions.  Items longer
// than twice the mean go first, longest first, so that no long item starts
// late; the rest keep (sequence, partition) order, which keeps neighbouring
// sequences (for instance parallel samples sharing prompt blocks) close in
// time and mixes sizes so that concurrently running workgroups stay busy.
// Waves per workgroup: 8, or 4 when the mean item is shorter than 12
// 16-token tiles (8 waves would leave most of them one tile or none).
// Measured on 256 sequences of 20..200 tokens (fused step): 4 waves 12-23%
// faster than 8 at B = 8 / 16 / 64, and 2-6% faster than 2 waves; 8 waves
// best on the lognormal batch (median 300 tokens).
// False when either list would exceed the kernel-argument capacity.
bool plan_work(const int32_t *host_ctx, int num_seqs, int max_context_len, int part,
               int block_size, pa::WorkList *items, pa::WorkList *merge_rows, int *waves) {
  int total = 0;
  long long tokens = 0;
  for (int b = 0; b < num_seqs; ++b) {
    const int c = clamp_ctx(host_ctx[b], max_context_len);
    total += c == 0 ? 1 : (c + part - 1) / part;
    tokens += c;
    if (total > pa::kMaxListed) return false;
  }
  struct Entry {
    int tokens;
    uint32_t item;
  };
  Entry e[pa::kMaxListed];
  int n = 0;
  merge_rows->count = 0;
  for (int b = 0; b < num_seqs; ++b) {
    const int c = clamp_ctx(host_ctx[b], max_context_len);
    const int np = c == 0 ? 1 : (c + part - 1) / part;
    for (int q = 0; q < np; ++q)
      e[n++] = Entry{std::min(part, c - q * part), ((uint32_t)b << 16) | (uint32_t)q};
    if (np > 1) merge_rows->item[merge_rows->count++] = (uint32_t)b;
  }
  const long long long_item = 2 * tokens / n;  // twice the mean item length
  Entry *mid = std::stable_partition(
      e, e + n, [long_item](const Entry &x) { return (long long)x.tokens > long_item; });
  std::stable_sort(e, mid, [](const Entry &x, const Entry &y) { return x.tokens > y.tokens; });
  items->count = n;
  for (int i = 0; i < n; ++i) items->item[i] = e[i].item;
  constexpr long long kShortItemTokens = 12 * 16;
  *waves = (long long)n * kShortItemTokens > tokens ? 4 : 8;
  return true;
}

// Partition length when the caller leaves it to the library and passes
// host-side lengths: start from PA_LONG_PARTITION and halve while the batch
// offers fewer than kPlanTargetItems workgroups' worth of (head, sequence,
// partition) items, down to kPlanMinPartition, never below what the
// workspace can hold.
constexpr long long kPlanTargetItems = 2048;
constexpr int kPlanMinPartition = 256;

int plan_partition(const int32_t *host_ctx, int num_seqs, int num_heads, int head_dim,
                   int max_context_len, size_t workspace_bytes, bool have_workspace) {
  int part = PA_LONG_PARTITION;
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
                   pa::decode_workspace_layout(num_seqs, num_heads, head_dim, np).total >
                       workspace_bytes))
      break;
    part = next;
  }
  return part;
}

}  // namespace

extern "C" {

// Work list of the prefill: every (sequence, query tile) that the grid
// would cover, with its weight (the keys its last query sees), grouped by
// sequence (see the order below).  False if it has more than kMaxListed
// entries.
struct PrefillItem {
  uint32_t code;   // sequence << 16 | query tile
  int64_t work;
};

bool plan_prefill(const int32_t *hqs, const int32_t *hctx, int num_seqs, int max_context_len,
                  int max_query_len, std::vector<PrefillItem> *out) {
  const int tile = pa::prefill_query_tile();
  const int max_tiles = (max_query_len + tile - 1) / tile;
  std::vector<PrefillItem> &list = *out;
  list.clear();
  for (int b = 0; b < num_seqs; ++b) {
    const int m = hqs[b + 1] - hqs[b];
    if (m <= 0) continue;
    const int n = hctx ? std::min(std::max(hctx[b], 0), max_context_len) : m;
    const int tiles = std::min((m + tile - 1) / tile, max_tiles);
    for (int t = 0; t < tiles; ++t) {
      if (list.size() >= (size_t)pa::kMaxListed || b > 0xffff) return false;
      list.push_back({(uint32_t)b << 16 | (uint32_t)t,
                      (int64_t)n - m + std::min(m, (t + 1) * tile)});
    }
  }
  // Sequence-major: sequences by their heaviest tile, descending, and each
  // sequence's tiles heaviest first.  The tiles of one sequence then run
  // together and share the K/V rows they stream in the L2 (a head's
  // workgroups all land on one XCD: the grid's fastest index is the head).
  std::vector<int64_t> seq_work(num_seqs > 0 ? num_seqs : 1, 0);
  for (const PrefillItem &it : list)
    seq_work[it.code >> 16] = std::max(seq_work[it.code >> 16], it.work);
  std::stable_sort(list.begin(), list.end(), [&](const PrefillItem &a, const PrefillItem &b) {
    const int sa = (int)(a.code >> 16), sb = (int)(b.code >> 16);
    if (sa != sb) return seq_work[sa] != seq_work[sb] ? seq_work[sa] > seq_work[sb] : sa < sb;
    return a.work > b.work;
  });
  return true;
}

// Prefill workgroups the current device holds at once (CUs times the
// kernel's workgroups per CU), cached per device; 0 if unknown.
int prefill_resident_groups() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      return 0;
    v = cus * pa::prefill_groups_per_cu();
    cache[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

// Split plan.  When the launch leaves the GPU mostly idle (its tiles times
// heads fall short of two workgroups per CU), the idle slots take extra key
// chunks: the tile whose current chunk has the most key tiles gets one more
// chunk (all heads), if it has at least 48 key tiles, its chunks stay at
// least 16 key tiles long, it has at most kMaxChunks and workspace slots
// last.  The chunks of a split tile run side by side and a merge pass
// combines them.  A launch that already fills the GPU is never split.
// False when no tile is split or the launch list would not fit: the plain
// list is used.
bool plan_prefill_split(const std::vector<PrefillItem> &list, int num_heads, int resident,
                        size_t slots, pa::SplitList *split, pa::SplitList *merges) {
  if (list.empty() || resident <= 0 || slots < 2) return false;
  const int kt = pa::prefill_key_tile();
  // Measured on 40 heads x 128 (single prompts of 1024..4096 tokens, one or
  // a few; suffixes of 64..256 queries over 2048..8192 cached tokens):
  // shorter tiles, shorter chunks or more than two workgroups per CU cost
  // full prompts time (partial results are fp32 rows of 512 bytes per query
  // and head, written and read back).
  constexpr int64_t kMinSplitTiles = 48, kMinChunkTiles = 16;
  int64_t free_groups = (int64_t)resident * 2 / pa::prefill_groups_per_cu() -
                        (int64_t)list.size() * num_heads;
  if (free_groups < num_heads) return false;
  std::vector<int> chunks(list.size(), 1);
  std::vector<int64_t> tiles(list.size());
  for (size_t i = 0; i < list.size(); ++i) tiles[i] = (list[i].work + kt - 1) / kt;
  // largest current chunk first (tiles / chunks, rounded up)
  auto chunk_len = [&](size_t i) { return (tiles[i] + chunks[i] - 1) / chunks[i]; };
  std::vector<size_t> heap(list.size());
  for (size_t i = 0; i < heap.size(); ++i) heap[i] = i;
  auto less = [&](size_t a, size_t b) { return chunk_len(a) < chunk_len(b); };
  std::make_heap(heap.begin(), heap.end(), less);
  size_t used = 0;
  while (!heap.empty() && free_groups >= num_heads) {
    std::pop_heap(heap.begin(), heap.end(), less);
    const size_t i = heap.back();
    heap.pop_back();
    const int nc = chunks[i] + 1;
    const size_t need = nc == 2 ? 2 : 1;   // slots this step takes
    if (tiles[i] < kMinSplitTiles || nc > pa::kMaxChunks || tiles[i] / nc < kMinChunkTiles ||
        used + need > slots)
      continue;
    chunks[i] = nc;
    used += need;
    free_groups -= num_heads;
    heap.push_back(i);
    std::push_heap(heap.begin(), heap.end(), less);
  }
  if (used == 0) return false;
  size_t entries = 0;
  for (int nc : chunks) entries += nc;
  if (entries > (size_t)pa::kMaxSplitItems) return false;
  split->count = 0;
  merges->count = 0;
  uint32_t slot = 0;
  for (size_t i = 0; i < list.size(); ++i) {
    const int nc = chunks[i];
    for (int c = 0; c < nc; ++c) {
      split->item[split->count] = list[i].code;
      split->part[split->count] =   // each chunk its own slot: slot + c
          nc > 1 ? ((slot + (uint32_t)c) << 8 | (uint32_t)c << 4 | (uint32_t)(nc - 1)) : 0u;
      ++split->count;
    }
    if (nc > 1) {
      merges->item[merges->count] = list[i].code;
      merges->part[merges->count] = slot << 8 | (uint32_t)(nc - 1);
      ++merges->count;
      slot += (uint32_t)nc;
    }
  }
  return true;
}

size_t pa_prefill_workspace_bytes(int num_heads, int head_dim, int slots) {
  if (num_heads <= 0 || (head_dim != 64 && head_dim != 128) || slots <= 0) return 0;
  return pa::prefill_slot_bytes(num_heads, head_dim) * (size_t)slots;
}

int pa_prefill(void *out, const void *q, const void *k_pool, const void *v_pool,
               const int32_t *block_tables, const int32_t *context_lens,
               const int32_t *query_start, int num_seqs, int num_query_rows, int num_heads,
               int head_dim, int block_size, int num_blocks, int max_blocks_per_seq,
               int max_context_len, int max_query_len, float scale, int dtype,
               const int32_t *host_query_start, const int32_t *host_context_lens,
               void *workspace, size_t workspace_bytes, void *stream) {
  int rc = check_pool(num_heads, head_dim, block_size, num_blocks, dtype);
  if (rc != PA_OK) return rc;
  if (dtype != PA_F16) return PA_ERR_UNSUPPORTED;
  if (num_seqs < 0 || num_query_rows < 0 || max_blocks_per_seq <= 0 || max_context_len < 0 ||
      max_query_len < 0 || max_query_len > max_context_len ||
      (int64_t)max_context_len > (int64_t)max_blocks_per_seq * block_size || !isfinite(scale))
    return PA_ERR_SHAPE;
  if (num_seqs == 0 || num_query_rows == 0 || max_query_len == 0) return PA_OK;
  if (!out || !q || !k_pool || !v_pool || !block_tables || !context_lens || !query_start)
    return PA_ERR_NULL;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) ||
      ((uintptr_t)block_tables & 3u) || ((uintptr_t)context_lens & 3u) ||
      ((uintptr_t)query_start & 3u) || (workspace && !aligned16(workspace)))
    return PA_ERR_SHAPE;
  const int64_t tiles = ((int64_t)max_query_len + pa::prefill_query_tile() - 1) /
                        pa::prefill_query_tile();
  if (tiles > kGridYZ || num_seqs > kGridYZ) return PA_ERR_SHAPE;
  pa::PrefillParams p{};
  p.out = out;
  p.q = q;
  p.k_pool = k_pool;
  p.v_pool = v_pool;
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  p.query_start = query_start;
  p.num_heads = num_heads;
  p.num_blocks = num_blocks;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.max_context_len = max_context_len;
  p.num_query_rows = num_query_rows;
  p.scale_log2 = scale * 1.44269504088896340736f;
  std::vector<PrefillItem> list;
  const bool listed = host_query_start &&
                      plan_prefill(host_query_start, host_context_lens, num_seqs,
                                   max_context_len, max_query_len, &list);
  const size_t slot_bytes = pa::prefill_slot_bytes(num_heads, head_dim);
  const size_t slots = workspace ? workspace_bytes / slot_bytes : 0;
  pa::SplitList split, merges;
  const bool is_split =
      listed && slots >= 2 &&
      plan_prefill_split(list, num_heads, prefill_resident_groups(), slots, &split, &merges);
  if (is_split) {
    p.part_o = static_cast<float *>(workspace);
    // [slots][H][128][D] outputs, then [slots][H][128] (max, sum)
    const size_t o_bytes =
        slots * (size_t)num_heads * pa::prefill_query_tile() * head_dim * sizeof(float);
    p.part_ml = reinterpret_cast<float2 *>(static_cast<char *>(workspace) + o_bytes);
  }
  pa::WorkList items;
  if (listed && !is_split) {
    items.count = (int)list.size();
    for (size_t i = 0; i < list.size(); ++i) items.item[i] = list[i].code;
  }
  return launch_checked("pa_prefill", [&] {
    return pa::launch_prefill(p, num_seqs, head_dim, block_size, max_query_len,
                              listed && !is_split ? &items : nullptr, is_split ? &split : nullptr,
                              is_split ? &merges : nullptr, static_cast<hipStream_t>(stream));
  });
}

int pa_swap_blocks(void *dst_k, void *dst_v, const void *src_k, const void *src_v,
                   const int64_t *block_mapping, int num_pairs, int num_heads, int head_dim,
                   int block_size, int src_num_blocks, int dst_num_blocks, int dtype,
                   void *stream) {
  // Whole blocks move as bytes: any geometry whose block span is a whole
  // number of 16-byte chunks.
  if (!elem_bytes(dtype)) return PA_ERR_UNSUPPORTED;
  if (num_heads <= 0 || head_dim <= 0 || block_size <= 0 || src_num_blocks <= 0 ||
      dst_num_blocks <= 0)
    return PA_ERR_SHAPE;
  const int64_t span = (int64_t)num_heads * block_size * head_dim * elem_bytes(dtype);
  if (span % 16 != 0 || span > ((int64_t)1 << 40)) return PA_ERR_SHAPE;
  if (num_pairs < 0) return PA_ERR_SHAPE;
  if (num_pairs == 0) return PA_OK;
  if (!dst_k || !dst_v || !src_k || !src_v || !block_mapping) return PA_ERR_NULL;
  if (!aligned16(dst_k) || !aligned16(dst_v) || !aligned16(src_k) || !aligned16(src_v) ||
      ((uintptr_t)block_mapping & 7u))
    return PA_ERR_SHAPE;
  if (!gpu_reachable(dst_k, "dst_k") || !gpu_reachable(dst_v, "dst_v") ||
      !gpu_reachable(src_k, "src_k") || !gpu_reachable(src_v, "src_v") ||
      !gpu_reachable(block_mapping, "block_mapping"))
    return PA_ERR_UNSUPPORTED;
  const size_t block_bytes = (size_t)num_heads * block_size * head_dim * elem_bytes(dtype);
  return launch_checked("pa_swap_blocks", [&] {
    return pa::launch_move_blocks(dst_k, dst_v, src_k, src_v, block_mapping, num_pairs,
                                  block_bytes, src_num_blocks, dst_num_blocks,
                                  static_cast<hipStream_t>(stream));
  });
}

const char *pa_last_error(void) { return t_detail; }

const char *pa_status_string(int status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_NULL: return "a required pointer is NULL";
    case PA_ERR_SHAPE: return "a size is out of range or a pointer is misaligned";
    case PA_ERR_UNSUPPORTED:
      return "unsupported head_dim, block_size or dtype, or memory the GPU cannot reach";
    case PA_ERR_WORKSPACE: return "workspace missing or too small";
    case PA_ERR_HIP: return "HIP runtime error at launch";
    case PA_ERR_NO_SEQUENCE: return "no sequence with that id";
    case PA_ERR_EXISTS: return "a sequence with that id already exists";
    case PA_ERR_NO_BLOCKS: return "not enough free KV blocks";
    case PA_ERR_SWAPPED: return "the sequence is swapped out";
  }
  return "unknown status";
}

size_t pa_decode_workspace_bytes(int num_seqs, int num_heads, int head_dim, int max_context_len,
                                 int partition_size) {
  const int part = effective_partition(partition_size, max_context_len);
  if (num_seqs < 0 || num_heads <= 0 || !supported_head_dim(head_dim) || max_context_len < 0 ||
      !valid_partition(part))
    return (size_t)-1;
  const int np = num_partitions(max_context_len, part);
  if (np <= 1 || num_seqs == 0) return 0;
  return pa::decode_workspace_layout(num_seqs, num_heads, head_dim, np).total;
}

int pa_decode_partition_size(const int32_t *host_context_lens, int num_seqs, int num_heads,
                             int head_dim, int max_context_len, int partition_size,
                             size_t workspace_bytes) {
  if (num_seqs < 0 || num_heads <= 0 || max_context_len < 0) return PA_ERR_SHAPE;
  if (!supported_head_dim(head_dim)) return PA_ERR_UNSUPPORTED;
  const int part = effective_partition(partition_size, max_context_len);
  if (!valid_partition(part)) return PA_ERR_SHAPE;
  if (host_context_lens && partition_size == 0)
    return plan_partition(host_context_lens, num_seqs, num_heads, head_dim, max_context_len,
                          workspace_bytes, workspace_bytes > 0);
  return part;
}

// pa_decode and pa_decode_append: the append arguments are all null for a
// plain decode.
static int decode_impl(const char *what, void *out, const void *q, const void *new_key,
                       const void *new_value, const void *k_pool, const void *v_pool,
                       const int32_t *block_tables, const int32_t *context_lens,
                       const int64_t *slot_mapping, int num_seqs, int num_heads, int head_dim,
                       int block_size, int num_blocks, int max_blocks_per_seq, int max_context_len,
                       float scale, int dtype, int partition_size, const int32_t *host_context_lens,
                       void *workspace, size_t workspace_bytes, void *stream) {
  int rc = check_pool(num_heads, head_dim, block_size, num_blocks, dtype);
  if (rc != PA_OK) return rc;
  int part = effective_partition(partition_size, max_context_len);
  if (num_seqs < 0 || max_blocks_per_seq <= 0 || max_context_len < 0 ||
      (int64_t)max_context_len > (int64_t)max_blocks_per_seq * block_size ||
      !valid_partition(part) || !isfinite(scale) || num_seqs > kGridYZ || num_heads > kGridYZ ||
      num_partitions(max_context_len, part) > kGridYZ)
    return PA_ERR_SHAPE;
  if (num_seqs == 0) return PA_OK;
  if (!out || !q || !k_pool || !v_pool || !block_tables || !context_lens) return PA_ERR_NULL;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) ||
      ((uintptr_t)block_tables & 3u) || ((uintptr_t)context_lens & 3u))
    return PA_ERR_SHAPE;
  const bool append = new_key || new_value || slot_mapping;
  if (append) {
    if (!new_key || !new_value || !slot_mapping) return PA_ERR_NULL;
    if (!aligned16(new_key) || !aligned16(new_value) || ((uintptr_t)slot_mapping & 7u))
      return PA_ERR_SHAPE;
  }
  if (host_context_lens && partition_size == 0)
    part = plan_partition(host_context_lens, num_seqs, num_heads, head_dim, max_context_len,
                          workspace_bytes, workspace != nullptr);

  pa::DecodeParams p{};
  p.out = out;
  p.q = q;
  p.k_pool = k_pool;
  p.v_pool = v_pool;
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  p.num_seqs = num_seqs;
  p.num_heads = num_heads;
  p.num_blocks = num_blocks;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.max_context_len = max_context_len;
  p.partition_size = part;
  p.num_partitions = num_partitions(max_context_len, part);
  p.scale_log2 = scale * 1.44269504088896340736f;
  p.new_key = new_key;
  p.new_value = new_value;
  p.slot_mapping = slot_mapping;
  if (p.num_partitions > 1) {
    const pa::WorkspaceLayout w =
        pa::decode_workspace_layout(num_seqs, num_heads, head_dim, p.num_partitions);
    if (!workspace || workspace_bytes < w.total) return PA_ERR_WORKSPACE;
    if (((uintptr_t)workspace & 255u) != 0) return PA_ERR_SHAPE;
    char *base = static_cast<char *>(workspace);
    p.part_ml = reinterpret_cast<float2 *>(base + w.ml_off);
    p.part_o = reinterpret_cast<float *>(base + w.o_off);
  }
  if (host_context_lens) {
    pa::WorkList items, merge_rows;
    int waves = 8;
    if (plan_work(host_context_lens, num_seqs, max_context_len, part, block_size, &items,
                  &merge_rows, &waves))
      return launch_checked(what, [&] {
        return pa::launch_decode(p, num_seqs, head_dim, block_size, dtype, &items, &merge_rows,
                                 waves, static_cast<hipStream_t>(stream));
      });
  }
  return launch_checked(what, [&] {
    return pa::launch_decode(p, num_seqs, head_dim, block_size, dtype, nullptr, nullptr, 8,
                             static_cast<hipStream_t>(stream));
  });
}

int pa_decode(void *out, const void *q, const void *k_pool, const void *v_pool,
              const int32_t *block_tables, const int32_t *context_lens, int num_seqs,
              int num_heads, int head_dim, int block_size, int num_blocks,
              int max_blocks_per_seq, int max_context_len, float scale, int dtype,
              int partition_size, const int32_t *host_context_lens, void *workspace,
              size_t workspace_bytes, void *stream) {
  return decode_impl("pa_decode", out, q, nullptr, nullptr, k_pool, v_pool, block_tables,
                     context_lens, nullptr, num_seqs, num_heads, head_dim, block_size,
                     num_blocks, max_blocks_per_seq, max_context_len, scale, dtype,
                     partition_size, host_context_lens, workspace, workspace_bytes, stream);
}

int pa_decode_append(void *out, const void *q, const void *new_key, const void *new_value,
                     void *k_pool, void *v_pool, const int32_t *block_tables,
                     const int32_t *context_lens, const int64_t *slot_mapping, int num_seqs,
                     int num_heads, int head_dim, int block_size, int num_blocks,
                     int max_blocks_per_seq, int max_context_len, float scale, int dtype,
                     int partition_size, const int32_t *host_context_lens, void *workspace,
                     size_t workspace_bytes, void *stream) {
  if (num_seqs > 0 && (!new_key || !new_value || !slot_mapping)) return PA_ERR_NULL;
  return decode_impl("pa_decode_append", out, q, new_key, new_value, k_pool, v_pool,
                     block_tables, context_lens, slot_mapping, num_seqs, num_heads, head_dim,
                     block_size, num_blocks, max_blocks_per_seq, max_context_len, scale, dtype,
                     partition_size, host_context_lens, workspace, workspace_bytes, stream);
}

int pa_write_kv(const void *key, const void *value, void *k_pool, void *v_pool,
                const int64_t *slot_mapping, int num_tokens, int num_heads, int head_dim,
                int block_size, int num_blocks, int dtype, void *stream) {
  int rc = check_pool(num_heads, head_dim, block_size, num_blocks, dtype);
  if (rc != PA_OK) return rc;
  if (num_tokens < 0) return PA_ERR_SHAPE;
  if (num_tokens == 0) return PA_OK;
  if (!key || !value || !k_pool || !v_pool || !slot_mapping) return PA_ERR_NULL;
  if (!aligned16(key) || !aligned16(value) || !aligned16(k_pool) || !aligned16(v_pool) ||
      ((uintptr_t)slot_mapping & 7u))
    return PA_ERR_SHAPE;
  return launch_checked("pa_write_kv", [&] {
    return pa::launch_write_kv(key, value, k_pool, v_pool, slot_mapping, num_tokens, num_heads,
                               head_dim * elem_bytes(dtype), block_size, num_blocks,
                               static_cast<hipStream_t>(stream));
  });
}

int pa_copy_blocks(void *k_pool, void *v_pool, const int64_t *block_mapping, int num_pairs,
                   int num_heads, int head_dim, int block_size, int num_blocks, int dtype,
                   void *stream) {
  int rc = check_pool(num_heads, head_dim, block_size, num_blocks, dtype);
  if (rc != PA_OK) return rc;
  if (num_pairs < 0) return PA_ERR_SHAPE;
  if (num_pairs == 0) return PA_OK;
  if (!k_pool || !v_pool || !block_mapping) return PA_ERR_NULL;
  if (!aligned16(k_pool) || !aligned16(v_pool) || ((uintptr_t)block_mapping & 7u))
    return PA_ERR_SHAPE;
  const size_t block_bytes = (size_t)num_heads * block_size * head_dim * elem_bytes(dtype);
  return launch_checked("pa_copy_blocks", [&] {
    return pa::launch_copy_blocks(k_pool, v_pool, block_mapping, num_pairs, block_bytes,
                                  num_blocks, static_cast<hipStream_t>(stream));
  });
}

}  // extern "C"
