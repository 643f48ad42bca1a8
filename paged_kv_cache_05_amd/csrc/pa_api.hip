// C ABI of libpa.so: argument validation and dispatch to the kernels.  The
// contract (shapes, layouts, ownership, errors) is documented in
// include/pa.h; this file checks scalars and pointers only and never reads
// device memory.
#include <math.h>
#include <stdio.h>

#include <atomic>

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

// Description of the last HIP error this library saw on the calling thread.
thread_local char t_detail[384] = "";

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

// hipGetLastError reports the last failure of any HIP call on the thread,
// so a launch first takes whatever an earlier call (of the caller, or of a
// framework around it) left behind; the status read after the launch then
// belongs to the launch.  Both are described for pa_last_error.
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

}  // namespace

extern "C" {

// Prefill workgroups the current device holds at once (CUs times the
// kernel's workgroups per CU); 0 if unknown.  Queried on every planned call:
// the runtime answers from its cached device properties.
static int prefill_resident_groups() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0) {
    (void)hipGetLastError();
    return 0;
  }
  return cus * pa::prefill_groups_per_cu();
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
  pa::PrefillPlan list;
  const bool listed = host_query_start &&
                      pa::plan_prefill(host_query_start, host_context_lens, num_seqs,
                                       max_context_len, max_query_len, pa::prefill_query_tile(),
                                       &list);
  const size_t slot_bytes = pa::prefill_slot_bytes(num_heads, head_dim);
  const size_t slots = workspace ? workspace_bytes / slot_bytes : 0;
  pa::SplitList split, merges;
  const bool is_split =
      listed && slots >= 2 &&
      pa::plan_prefill_split(list, num_heads, prefill_resident_groups(),
                             pa::prefill_groups_per_cu(), pa::prefill_key_tile(), slots, &split,
                             &merges);
  if (is_split) {
    p.part_o = static_cast<float *>(workspace);
    // [slots][H][128][D] outputs, then [slots][H][128] (max, sum)
    const size_t o_bytes =
        slots * (size_t)num_heads * pa::prefill_query_tile() * head_dim * sizeof(float);
    p.part_ml = reinterpret_cast<float2 *>(static_cast<char *>(workspace) + o_bytes);
  }
  pa::WorkList items;
  if (listed && !is_split) {
    items.count = list.count;
    for (int i = 0; i < list.count; ++i) items.item[i] = list.item[i].code;
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
  const int np = pa::num_partitions(max_context_len, part);
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
    return pa::plan_partition(host_context_lens, num_seqs, num_heads, head_dim,
                              max_context_len, workspace_bytes, workspace_bytes > 0);
  return part;
}

// Allocation-free decode (pa_decode_noalloc): the partial results of rows
// that span several partitions live in this file-scope device array, one
// copy per GPU, held until the process ends.  In host code `scratch` only
// names the symbol; its device address on each GPU comes from
// hipGetSymbolAddress, taken once per device with that device current and
// kept in g_scratch.  Calls that overlap on one GPU share the array and
// race; nothing in it needs clearing (the kernels write every partial
// result before the merge reads it).
static __device__ __align__(256) unsigned char scratch[PA_NOALLOC_SCRATCH_BYTES];
static constexpr int kMaxDevices = 64;
static std::atomic<void *> g_scratch[kMaxDevices];

// Device address of `scratch` on the current device, or null with the
// reason in pa_last_error.
static void *scratch_on_current_device() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    snprintf(t_detail, sizeof t_detail, "pa_decode_noalloc: no usable current device (%s, %d)",
             hipGetErrorName(e), dev);
    return nullptr;
  }
  void *ptr = g_scratch[dev].load(std::memory_order_acquire);
  if (ptr) return ptr;
  e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess || !ptr) {
    (void)hipGetLastError();
    snprintf(t_detail, sizeof t_detail,
             "pa_decode_noalloc: hipGetSymbolAddress of the scratch array failed on device %d: "
             "%s (%s)",
             dev, hipGetErrorName(e), hipGetErrorString(e));
    return nullptr;
  }
  g_scratch[dev].store(ptr, std::memory_order_release);   // same value if two threads race
  return ptr;
}

// pa_decode, pa_decode_append and pa_decode_noalloc: the append arguments
// are all null for a plain decode; static_scratch selects the
// allocation-free form (workspace arguments ignored).
static int decode_impl(const char *what, void *out, const void *q, const void *new_key,
                       const void *new_value, const void *k_pool, const void *v_pool,
                       const int32_t *block_tables, const int32_t *context_lens,
                       const int64_t *slot_mapping, int num_seqs, int num_heads, int head_dim,
                       int block_size, int num_blocks, int max_blocks_per_seq, int max_context_len,
                       float scale, int dtype, int partition_size, const int32_t *host_context_lens,
                       void *workspace, size_t workspace_bytes, void *stream,
                       bool static_scratch = false) {
  int rc = check_pool(num_heads, head_dim, block_size, num_blocks, dtype);
  if (rc != PA_OK) return rc;
  int part = effective_partition(partition_size, max_context_len);
  if (num_seqs < 0 || max_blocks_per_seq <= 0 || max_context_len < 0 ||
      (int64_t)max_context_len > (int64_t)max_blocks_per_seq * block_size ||
      !valid_partition(part) || !isfinite(scale) || num_seqs > kGridYZ || num_heads > kGridYZ ||
      pa::num_partitions(max_context_len, part) > kGridYZ)
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
    // the grid launch adds ceil(num_seqs / num_heads) writer rows
    if (num_seqs + (num_seqs + num_heads - 1) / num_heads > kGridYZ) return PA_ERR_SHAPE;
  }
  if (static_scratch) {
    workspace = scratch_on_current_device();
    if (!workspace) return PA_ERR_HIP;
    workspace_bytes = PA_NOALLOC_SCRATCH_BYTES;
  }
  if (host_context_lens && partition_size == 0)
    part = pa::plan_partition(host_context_lens, num_seqs, num_heads, head_dim,
                              max_context_len, workspace_bytes, workspace != nullptr);
  if (static_scratch) {
    const int np = pa::num_partitions(max_context_len, part);
    const size_t need = np > 1 ? pa::decode_workspace_layout(num_seqs, num_heads, head_dim,
                                                             np).total
                               : 0;
    if (need > PA_NOALLOC_SCRATCH_BYTES) {
      snprintf(t_detail, sizeof t_detail,
               "pa_decode_noalloc: %d sequences x %d heads x %d partitions of %d tokens need "
               "%zu bytes of partial results; the static scratch holds %zu (use a longer "
               "partition_size, or pa_decode with a workspace)",
               num_seqs, num_heads, np, part, need, (size_t)PA_NOALLOC_SCRATCH_BYTES);
      return PA_ERR_WORKSPACE;
    }
  }

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
  p.num_partitions = pa::num_partitions(max_context_len, part);
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
    if (pa::plan_work(host_context_lens, num_seqs, max_context_len, part, &items, &merge_rows,
                      &waves))
      return launch_checked(what, [&] {
        return pa::launch_decode(p, num_seqs, head_dim, block_size, dtype, &items, &merge_rows,
                                 waves, static_cast<hipStream_t>(stream));
      });
  }
  // Grid launch: 4-wave workgroups when no row is longer than 256 tokens, 8
  // otherwise (long rows keep the 8-wave form whatever the partition size).
  constexpr int kGridShortTokens = 256;
  const int grid_waves = max_context_len <= kGridShortTokens ? 4 : 8;
  return launch_checked(what, [&] {
    return pa::launch_decode(p, num_seqs, head_dim, block_size, dtype, nullptr, nullptr,
                             grid_waves, static_cast<hipStream_t>(stream));
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

int pa_decode_noalloc(void *out, const void *q, const void *k_pool, const void *v_pool,
                      const int32_t *block_tables, const int32_t *context_lens, int num_seqs,
                      int num_heads, int head_dim, int block_size, int num_blocks,
                      int max_blocks_per_seq, int max_context_len, float scale, int dtype,
                      int partition_size, const int32_t *host_context_lens, void *stream) {
  return decode_impl("pa_decode_noalloc", out, q, nullptr, nullptr, k_pool, v_pool,
                     block_tables, context_lens, nullptr, num_seqs, num_heads, head_dim,
                     block_size, num_blocks, max_blocks_per_seq, max_context_len, scale, dtype,
                     partition_size, host_context_lens, nullptr, 0, stream, true);
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
