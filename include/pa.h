/*
 * pa.h -- paged decode attention for AMD Instinct MI355X (gfx950).
 *
 * A C ABI over three HIP kernel families: single-query decode attention over
 * a KV cache stored in fixed-size blocks at scattered physical locations
 * (PagedAttention), the per-step write of new tokens' K/V into their slots,
 * and the block-granular copy-on-write copy.  Source: Kwon et al., "Efficient
 * Memory Management for Large Language Model Serving with PagedAttention"
 * (2023), as summarised on three web pages:
 *   [wywy]  wywy.jp reading notes,
 *   [zhai]  zhaifeiyue.github.io structured summary,
 *   [rice]  ricepunchb.github.io "KV Cache Optimization" notes.
 *
 * Conventions for every entry point
 * ---------------------------------
 *  - Every pointer argument is device memory owned by the caller (except
 *    `stream`, a hipStream_t; the returns of pa_status_string and
 *    pa_last_error; and the pools of pa_swap_blocks, which may also be
 *    pinned host memory).  The
 *    kernel entry points allocate nothing and free nothing.  Their only
 *    state between calls is a per-thread error description (pa_last_error)
 *    and, for pa_decode_noalloc alone, a static device array per GPU and its
 *    device address, looked up once per GPU.  They are thread-safe
 *    (pa_decode_noalloc calls that overlap on one GPU race on its array).
 *    The host block manager of pa_manager.h owns the host memory of each
 *    manager object, from pa_manager_create to pa_manager_destroy.
 *  - Work is enqueued asynchronously on `stream` (NULL = the default stream);
 *    no call synchronises.  Buffers must stay valid until the work completes.
 *  - Element type codes: PA_F16 (IEEE binary16) or PA_F32.  Query, pools,
 *    keys, values and output of one call share the element type; attention
 *    arithmetic is fp32.
 *  - KV pool layout (both pools): [num_blocks][num_heads][block_size][head_dim]
 *    row-major, so one (block, head) tile is block_size*head_dim contiguous
 *    elements and one block, all heads, is num_heads*block_size*head_dim
 *    contiguous elements.  K and V live in separate pools addressed by one
 *    block table ([wywy] Keyword "PagedAttention": K and V in separate blocks).
 *  - Token t (0-based) of sequence b lives in logical block t / block_size at
 *    offset t % block_size; its physical block is block_tables[b][t /
 *    block_size] ([rice] 3.2 "address translation": block index, block
 *    offset, physical address; [wywy] Keyword "Block table").
 *  - Floating-point arrays must be 16-byte aligned.
 *  - Return value: PA_OK (0) or a negative PA_ERR_* code.  On any error other
 *    than PA_ERR_HIP nothing was enqueued.  Only scalars and pointers are
 *    validated on the host; device array contents (table entries, slots,
 *    copy pairs, context lengths) are preconditions.  Kernels skip table
 *    entries, slots and copy pairs that fall outside the pool rather than
 *    access memory out of bounds (a decode row that meets such an entry is
 *    written as NaN), and clamp context lengths to [0, max_context_len].
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define PA_OK 0
#define PA_ERR_NULL (-1)        /* a required pointer is NULL */
#define PA_ERR_SHAPE (-2)       /* a size is out of range, or a pointer misaligned */
#define PA_ERR_UNSUPPORTED (-3) /* head_dim, block_size or dtype not compiled in */
#define PA_ERR_WORKSPACE (-4)   /* workspace missing or smaller than required */
#define PA_ERR_HIP (-5)         /* the HIP runtime rejected a launch */

/* Element types. */
#define PA_F16 0
#define PA_F32 1

/* Supported sizes: head_dim in {64, 128}; block_size in {8, 16, 32, 64}. */

/* Partition length used when pa_decode is given partition_size == 0:
 * PA_DEFAULT_PARTITION tokens, or PA_LONG_PARTITION when max_context_len
 * exceeds PA_LONG_CONTEXT. */
#define PA_DEFAULT_PARTITION 1024
#define PA_LONG_PARTITION 4096
#define PA_LONG_CONTEXT 8192

/*
 * Bytes of workspace pa_decode needs for this batch shape:
 * ceil(max_context_len / P) partitions per (sequence, head), where P is the
 * partition length (partition_size, or the default above when 0).  Returns
 * 0 when every context fits in one partition (no workspace needed) and
 * (size_t)-1 for invalid arguments.
 */
size_t pa_decode_workspace_bytes(int num_seqs, int num_heads, int head_dim,
                                 int max_context_len, int partition_size);

/*
 * The partition length pa_decode uses for these arguments: partition_size
 * when it is non-zero; else, with host_context_lens (HOST memory, may be
 * NULL), the length it plans from them within workspace_bytes; else the
 * default above.  A caller that wants the planner's free choice sizes the
 * workspace with pa_decode_workspace_bytes(..., 256).  Returns a negative
 * PA_ERR_* code for invalid arguments.
 */
int pa_decode_partition_size(const int32_t *host_context_lens, int num_seqs, int num_heads,
                             int head_dim, int max_context_len, int partition_size,
                             size_t workspace_bytes);

/*
 * Single-query paged decode attention ([zhai] "method" paragraph, the
 * block-wise equation for A_ij and o_i; [rice] 3.3: per-block scores, the
 * softmax completed by a final reduction; [wywy] WHERE: the kernel fetches
 * each needed block separately).
 *
 * For every sequence b < num_seqs and head h < num_heads, with
 * n = context_lens[b]:
 *     s_t      = scale * dot(q[b][h][:], K[phys(b,t)][h][t % B][:]),  t < n
 *     out[b][h][:] = sum_t softmax(s)_t * V[phys(b,t)][h][t % B][:]
 * where phys(b,t) = block_tables[b][t / B].  Slots of the last block at
 * offsets >= the filled count are not read into the result (they may hold
 * anything, NaN included).  n == 0 gives a zero row.
 *
 *   out            [num_seqs][num_heads][head_dim], element type dtype (written)
 *   q              [num_seqs][num_heads][head_dim], dtype
 *   k_pool, v_pool [num_blocks][num_heads][block_size][head_dim], dtype
 *   block_tables   int32 [num_seqs][max_blocks_per_seq]; entries below
 *                  ceil(n / block_size) must lie in [0, num_blocks); later
 *                  entries are never read
 *   context_lens   int32 [num_seqs], each in [0, max_context_len]
 *   max_context_len host-side bound on context_lens, at most
 *                  max_blocks_per_seq * block_size; sizes the launch grid, so
 *                  the host never reads device data
 *   scale          multiplier of the dot products (usually 1/sqrt(head_dim))
 *   partition_size tokens per context partition, a multiple of 16 in
 *                  [16, 65536], or 0 for the default above.  Contexts longer
 *                  than one partition are split across workgroups and merged
 *                  exactly (max/sum rescaling).
 *   host_context_lens optional HOST copy of context_lens (NULL: none).  The
 *                  step's scheduler has the lengths on the host anyway
 *                  ([wywy] WHERE: the central KV cache manager tracks each
 *                  sequence and sends the per-step inputs to the workers).
 *                  With it, the library launches exactly the non-empty
 *                  (sequence, partition) work items, largest first, and
 *                  merges only the sequences that span several partitions
 *                  (up to 960 items; beyond that, and without it, one
 *                  workgroup per (head, sequence, partition) is launched
 *                  and empty ones leave at once).  When the mean item is
 *                  shorter than 192 tokens, those workgroups have 4 waves
 *                  instead of 8; the result then
 *                  differs from the unplanned launch's by fp32 rounding
 *                  order, otherwise it is the same bit for bit.  Each entry must be at
 *                  least the device value it copies (equal for the best
 *                  schedule); the device values still decide every result.
 *   workspace      device scratch of at least pa_decode_workspace_bytes(...)
 *                  bytes (256-byte aligned), or NULL when that is 0: the
 *                  per-partition partial results (max, sum, unnormalised
 *                  output) of rows longer than one partition.  Contents on
 *                  entry are ignored; concurrent calls must not share one
 *                  workspace.
 *
 * Launches one kernel, plus a small merge kernel when some row spans several
 * partitions.  Workgroups own (head, sequence, partition); rows that fit one
 * partition are finished by the first kernel.
 */
int pa_decode(void *out, const void *q, const void *k_pool, const void *v_pool,
              const int32_t *block_tables, const int32_t *context_lens,
              int num_seqs, int num_heads, int head_dim, int block_size,
              int num_blocks, int max_blocks_per_seq, int max_context_len,
              float scale, int dtype, int partition_size,
              const int32_t *host_context_lens,
              void *workspace, size_t workspace_bytes, void *stream);

/*
 * Size of the static device scratch that pa_decode_noalloc uses: one array
 * of this many bytes on each GPU the library runs on, held until the
 * process ends.
 */
#define PA_NOALLOC_SCRATCH_BYTES (16u << 20)

/*
 * pa_decode for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * same arguments as pa_decode minus the workspace, and the same result, bit
 * for bit, as pa_decode with those arguments and a workspace of
 * PA_NOALLOC_SCRATCH_BYTES.  The partial results of rows that span several
 * partitions go to a static device array of PA_NOALLOC_SCRATCH_BYTES per
 * GPU instead of a caller's workspace.  The call allocates nothing (no
 * hipMalloc, no host heap); its first call on a device looks up the
 * array's address there (hipGetSymbolAddress), and later calls reuse it.
 *
 * A batch whose partial results need more than PA_NOALLOC_SCRATCH_BYTES
 * (num_seqs * num_heads * partitions * (head_dim + 2) * 4 bytes, each part
 * 256-byte aligned; at most 32263 (sequence, head, partition) rows at
 * head_dim 128, 63550 at head_dim 64) returns PA_ERR_WORKSPACE before any launch, with the sizes
 * in pa_last_error; with host_context_lens and partition_size 0 the planner
 * picks a partition length that fits when one exists.  Every call on a GPU
 * shares that GPU's array: calls that overlap in time on one GPU (on
 * different streams, or from different threads) race and must be ordered
 * by the caller.  The array's contents from an earlier call do not matter.
 */
int pa_decode_noalloc(void *out, const void *q, const void *k_pool, const void *v_pool,
                      const int32_t *block_tables, const int32_t *context_lens,
                      int num_seqs, int num_heads, int head_dim, int block_size,
                      int num_blocks, int max_blocks_per_seq, int max_context_len,
                      float scale, int dtype, int partition_size,
                      const int32_t *host_context_lens, void *stream);

/*
 * Store each new token's K and V rows, all heads, in its slot ([wywy]
 * Keyword "autoregressive generation phase": each step creates K/V only for
 * the new token; [zhai] "KV Cache Manager": a new block is taken only when
 * the previous one is full).  For token i with slot = slot_mapping[i] >= 0:
 *     K[slot / B][h][slot % B][:] = key[i][h][:]   for every head h
 *     V[slot / B][h][slot % B][:] = value[i][h][:]
 * Bit copies.  A negative slot skips the token (padding).  Slots must be
 * distinct (two tokens into one slot race) and below num_blocks * block_size.
 *
 *   key, value    [num_tokens][num_heads][head_dim], dtype
 *   k_pool, v_pool pools as for pa_decode (written)
 *   slot_mapping  int64 [num_tokens], slot = physical_block * block_size + offset
 */
int pa_write_kv(const void *key, const void *value, void *k_pool, void *v_pool,
                const int64_t *slot_mapping, int num_tokens, int num_heads,
                int head_dim, int block_size, int num_blocks, int dtype,
                void *stream);

/*
 * Block-granular copy-on-write copy ([wywy] WHERE, parallel sampling: on a
 * write to a block whose reference count exceeds 1, a new block is allocated
 * and the block engine copies the old block's contents into it; [zhai]
 * memory-management table, "Copy-on-Write": one block per copy).  For each
 * pair i, the whole block src = block_mapping[2i] (every head, every offset)
 * is copied onto dst = block_mapping[2i+1], in both pools.  Bit copies.  One
 * source may feed several destinations; destinations must be distinct and
 * must not appear as sources.
 *
 *   k_pool, v_pool pools as for pa_decode (read and written)
 *   block_mapping int64 [num_pairs][2] (src, dst), device memory
 */
int pa_copy_blocks(void *k_pool, void *v_pool, const int64_t *block_mapping,
                   int num_pairs, int num_heads, int head_dim, int block_size,
                   int num_blocks, int dtype, void *stream);

/*
 * One decoding step fused: store every sequence's new token and attend over
 * the context that includes it.  The same result, bit for bit, as
 * pa_write_kv(new_key, new_value, k_pool, v_pool, slot_mapping, num_seqs,
 * ...) followed by pa_decode(out, q, ...): each step creates K/V for the
 * new token only and stores it at the next free position of the sequence's
 * last block (the wywy.jp notes, Keyword "autoregressive generation phase"
 * and "KV cache manager"), and the query of that step attends over the
 * whole context, the new token included.  One launch instead of two, and
 * the new rows are read once, from new_key / new_value.
 *
 * new_key, new_value: [num_seqs][num_heads][head_dim], 16-byte aligned;
 * slot_mapping: int64 [num_seqs], the slot (block * block_size + offset) of
 * sequence b's new token, which must be the position context_lens[b] - 1
 * under its block table (a slot outside the pool is not written, as in
 * pa_write_kv; the attention still uses the new row for that position).
 * Every other argument, the workspace and the errors are those of
 * pa_decode.  No other sequence of the call may read the new token's slot
 * (copy-on-write guarantees it: the block written is private).
 */
int pa_decode_append(void *out, const void *q, const void *new_key, const void *new_value,
                     void *k_pool, void *v_pool, const int32_t *block_tables,
                     const int32_t *context_lens, const int64_t *slot_mapping, int num_seqs,
                     int num_heads, int head_dim, int block_size, int num_blocks,
                     int max_blocks_per_seq, int max_context_len, float scale, int dtype,
                     int partition_size, const int32_t *host_context_lens, void *workspace,
                     size_t workspace_bytes, void *stream);

/*
 * Paged prefill attention (the prompt phase).  Source: the PagedAttention
 * pages -- the wywy.jp notes, Keyword "prompt phase" (all prompt tokens are
 * known, so they are processed together, matrix-matrix) and WHERE, shared
 * prefix (a cached prefix's KV is reused; only the request's own tokens are
 * computed); the zhaifeiyue.github.io summary, method paragraph, block-wise
 * attention equation, with each query's context cut at its own position.
 *
 *   sequence b holds n_b = context_lens[b] tokens in the pools (their K/V
 *   already written, e.g. by pa_write_kv); its last m_b = query_start[b+1]
 *   - query_start[b] tokens are queries, rows query_start[b] ..
 *   query_start[b+1]-1 of q and out.  Query i sits at position
 *   p = n_b - m_b + i and
 *     out[row][h][:] = sum_{t<=p} softmax_t(scale * q[row][h] . K_t[h]) V_t[h]
 *   with K_t / V_t read through block_tables as in pa_decode.
 *
 * q, out: [num_query_rows][num_heads][head_dim] fp16, 16-byte aligned.
 * query_start: int32 [num_seqs + 1], non-decreasing from 0.  Pools, tables
 * and context_lens as in pa_decode.  max_context_len (>= every context
 * length; context lengths above it are clamped to it; at most
 * max_blocks_per_seq * block_size) and max_query_len (>= every m_b, at most
 * max_context_len) are host-side bounds that size the grid.
 * Only PA_F16 (PA_ERR_UNSUPPORTED otherwise); head_dim 64 or 128; block_size
 * 8, 16, 32 or 64.  The products run on MFMA with fp32 accumulation and an
 * fp32 softmax.  Each query element is multiplied by scale * log2(e) in
 * fp32 and rounded to fp16 once, before the products (a relative error of
 * at most 2^-11 per element; |scale * q| must stay below 45000, or the
 * rows turn inf/NaN); the attention weights are rounded to fp16 for the
 * product with V.
 *
 * host_query_start (optional, host memory, num_seqs + 1 entries) is a host
 * copy of query_start: with it the library launches only the query tiles
 * that exist, when there are at most 960 of them, grouped by sequence
 * (sequences in descending order of their heaviest tile, each sequence's
 * tiles heaviest first; a tile's weight is the keys its last query sees);
 * host_context_lens (optional, host memory) then refines that order.  Without them, or with more tiles, the
 * grid covers every (head, tile < max_query_len / 128, sequence) and empty
 * tiles exit at once.  A sequence's device query count must not exceed its
 * host one.  Results do not depend on the launch form.
 *
 * A sequence whose m_b exceeds its (clamped) context, or whose rows fall
 * outside [0, num_query_rows), gets NaN rows (those in range); a table entry
 * outside the pool makes NaN every row that attends to its keys.  Rows past
 * max_query_len of a sequence are not written.  Asynchronous on `stream`.
 *
 * workspace (optional, device memory, 16-byte aligned, caller-owned;
 * workspace_bytes long, see pa_prefill_workspace_bytes) lets the listed
 * launch split the key range of its heaviest query tiles across several
 * workgroups when those tiles alone would set the launch's length (a few
 * long prompts, or a long cached prefix, on a mostly idle GPU).  The
 * chunks write partial softmax states (max, sum, unnormalised output) to
 * the workspace and a second kernel merges them.  Split results equal the
 * unsplit ones up to fp32 rounding of the merge.  Without a workspace (NULL
 * or fewer than two slots) nothing is split.  The workspace must not be in
 * use by another call at the same time.
 */
int pa_prefill(void *out, const void *q, const void *k_pool, const void *v_pool,
               const int32_t *block_tables, const int32_t *context_lens,
               const int32_t *query_start, int num_seqs, int num_query_rows, int num_heads,
               int head_dim, int block_size, int num_blocks, int max_blocks_per_seq,
               int max_context_len, int max_query_len, float scale, int dtype,
               const int32_t *host_query_start, const int32_t *host_context_lens,
               void *workspace, size_t workspace_bytes, void *stream);

/*
 * Bytes of a pa_prefill workspace with room for `slots` partial results
 * (one per key chunk of a split query tile, all heads):
 * slots * num_heads * 128 * (head_dim * 4 + 8).  0 for invalid arguments
 * (num_heads <= 0, head_dim not 64 or 128, slots <= 0).
 */
size_t pa_prefill_workspace_bytes(int num_heads, int head_dim, int slots);

/*
 * Swapping: copy whole blocks between two pool pairs, typically the device
 * pools and pinned host pools (swap out: device -> host; swap in: host ->
 * device).  Source: the PagedAttention pages -- the wywy.jp notes, Keyword
 * "Swapping" and "All-or-nothing eviction" and Overview, scheduling and
 * preemption (every KV block of an evicted sequence is copied from GPU to
 * CPU memory, and back whole when it resumes; the CPU swap space never
 * needs more blocks than the GPU pool holds); the zhaifeiyue.github.io
 * summary, "Scheduling & Preemption" table, row "Swap".
 *
 *   for each i: block block_mapping[2i] of (src_k, src_v) is copied onto
 *   block block_mapping[2i+1] of (dst_k, dst_v), K and V, bit for bit.
 *
 * Pools: [src_num_blocks] (resp. [dst_num_blocks]) x [num_heads][block_size]
 * [head_dim] of `dtype`, 16-byte aligned; both pairs have the same block
 * shape.  Blocks move as bytes, so any positive geometry is accepted whose
 * block span (num_heads * block_size * head_dim * element bytes) is a
 * multiple of 16 bytes (PA_ERR_SHAPE otherwise).  Each of dst_k, dst_v, src_k, src_v and block_mapping (int64
 * [num_pairs][2]) must be device memory or pinned host memory (hipHostMalloc,
 * or torch's pin_memory) that the GPU reaches at the same address: the
 * kernel moves the bytes itself, over PCIe for the host side, in one launch
 * for any number of blocks.  Anything else -- pageable host memory, managed
 * memory -- returns PA_ERR_UNSUPPORTED before any launch (pa_last_error
 * names the pointer).  Destinations must be distinct and must not overlap
 * any source; a pair outside either pool is skipped.  Asynchronous on
 * `stream`: host memory written by a swap out is complete once the stream
 * has been synchronised.
 */
int pa_swap_blocks(void *dst_k, void *dst_v, const void *src_k, const void *src_v,
                   const int64_t *block_mapping, int num_pairs, int num_heads, int head_dim,
                   int block_size, int src_num_blocks, int dst_num_blocks, int dtype,
                   void *stream);

/* Static, NUL-terminated description of a status code. */
const char *pa_status_string(int status);

/*
 * Describes the last HIP runtime error this library saw on the calling
 * thread: the error of a launch that returned PA_ERR_HIP (HIP's error name
 * and text), or an error an earlier HIP call on the thread had left pending,
 * which a launch clears before it starts (hipGetLastError reports the last
 * failure of any call on the thread, so the status read after a launch would
 * otherwise not be the launch's own).  "" when there was none.  The string
 * belongs to the library, stays valid until the thread's next call into it,
 * and is not cleared by reading it.
 */
const char *pa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
