/*
 * pa_manager.h -- host-side KV block manager for the paged decode kernels.
 *
 * Keeps, for one pool of physical KV blocks, which blocks are free, how many
 * logical blocks (of all sequences) reference each one, and each sequence's
 * block list and length.  It decides where each new token goes and when a
 * block must be copied first, and builds the block tables, context lengths,
 * slot mapping and copy pairs that pa_copy_blocks, pa_write_kv and
 * pa_decode (pa.h) consume.  Source: the PagedAttention pages
 * ([wywy] wywy.jp notes; [zhai] zhaifeiyue.github.io summary; [rice]
 * ricepunchb.github.io notes):
 *   - a KV cache manager maps each request's logical blocks to physical
 *     blocks and records filled positions ([wywy] Keyword "KV cache
 *     manager");
 *   - a new block is allocated only when the previous one is full ([zhai]
 *     "KV Cache Manager" paragraph, memory table "Allocate");
 *   - each physical block has a reference count; a block is freed when its
 *     count reaches 0 ([wywy] Keyword "Reference count", WHERE beam search);
 *   - parallel samples share the prompt's blocks; a write into a block whose
 *     count exceeds 1 allocates a new block, copies the old one into it and
 *     decrements the old count ([wywy] WHERE parallel-sampling example;
 *     [zhai] memory table "Copy-on-Write"; [rice] 5.1);
 *   - when blocks run out, a preempted sequence group is evicted all or
 *     nothing; with swapping every one of its blocks goes to CPU memory and
 *     comes back whole when it resumes; the CPU swap space never needs more
 *     blocks than the GPU pool ([wywy] Keyword "Swapping", "All-or-nothing
 *     eviction", Overview, scheduling and preemption; [zhai] "Scheduling &
 *     Preemption" table, row "Swap").
 *
 * Host memory only; no GPU call is made.  A manager is not thread-safe:
 * one thread at a time per manager.  Sequences are named by caller-chosen
 * int64 ids.  Every function returns PA_OK (0) or a negative code:
 * PA_ERR_NULL, PA_ERR_SHAPE (bad argument), PA_ERR_NO_SEQUENCE (unknown
 * id), PA_ERR_EXISTS (id in use), PA_ERR_NO_BLOCKS (not enough free
 * blocks: nothing was changed), PA_ERR_SWAPPED (the sequence is swapped
 * out: only pa_manager_swap_in, pa_manager_free and the queries accept it).
 */
#ifndef PA_MANAGER_H
#define PA_MANAGER_H

#include <stdint.h>

#include "pa.h"

#ifdef __cplusplus
extern "C" {
#endif

#define PA_ERR_NO_SEQUENCE (-6)
#define PA_ERR_EXISTS (-7)
#define PA_ERR_NO_BLOCKS (-8)
#define PA_ERR_SWAPPED (-9)

typedef struct pa_manager pa_manager;

/*
 * A manager for GPU blocks 0 .. num_blocks-1 of block_size tokens, and a
 * CPU swap space of num_host_blocks blocks (0: no swapping).  alloc_order
 * (optional, num_blocks distinct ids) is the order in which free GPU blocks
 * are handed out at first (NULL: ascending); freed blocks are handed out
 * again before never-used ones, most recently freed first (host blocks
 * likewise, ascending at first).  Returns NULL on bad arguments or host
 * allocation failure.
 */
pa_manager *pa_manager_create(int num_blocks, int block_size, int num_host_blocks,
                              const int32_t *alloc_order);
void pa_manager_destroy(pa_manager *m);

/* A new, empty sequence. */
int pa_manager_add(pa_manager *m, int64_t seq);

/*
 * Child shares every block of parent (each count + 1) and has its length:
 * parallel samples or beam candidates forked from one prompt.
 */
int pa_manager_fork(pa_manager *m, int64_t parent, int64_t child);

/*
 * Reserve the slot of the next token of each of n resident sequences, in
 * order (PA_ERR_SWAPPED if one is swapped out).
 * For sequence seqs[i]: if its last block is full (or it has none) a fresh
 * block is appended; else if that block is shared (count > 1) a fresh block
 * replaces it, the old count drops by one, and (old, fresh) is reported as
 * a copy pair that must be executed (pa_copy_blocks) before the write.
 * slots[i] = physical block * block_size + position.  Copy pairs go to
 * copy_pairs ([2 * max_pairs] int64, src then dst) and their number to
 * *num_pairs.  All or nothing: if the free blocks cannot cover every
 * sequence, nothing changes and PA_ERR_NO_BLOCKS is returned (PA_ERR_SHAPE
 * when max_pairs is too small for the copies).  A sequence listed twice
 * gets two consecutive positions.
 */
int pa_manager_append(pa_manager *m, const int64_t *seqs, int n, int64_t *slots,
                      int64_t *copy_pairs, int max_pairs, int *num_pairs);

/* Drop a sequence: each of its blocks' counts - 1; blocks at 0 become free
 * (host blocks if it is swapped out). */
int pa_manager_free(pa_manager *m, int64_t seq);

/*
 * Swap out a group of n distinct resident sequences (a request's samples):
 * every distinct GPU block they reference gets a host block -- a block the
 * group shares is moved once and stays shared -- and the group's references
 * on the GPU blocks are dropped (a block also held by a sequence outside the
 * group stays on the GPU for it).  The (gpu block, host block) pairs go to
 * pairs ([2 * max_pairs] int64) and their number to *num_pairs; the caller
 * copies them with pa_swap_blocks (device pools -> host pools) before the
 * freed GPU blocks are written again.  All or nothing: PA_ERR_NO_BLOCKS if
 * the host pool is short, PA_ERR_SHAPE if max_pairs is too small or an id is
 * listed twice, PA_ERR_SWAPPED if one is already out.
 */
int pa_manager_swap_out(pa_manager *m, const int64_t *seqs, int n, int64_t *pairs,
                        int max_pairs, int *num_pairs);

/*
 * The reverse: every distinct host block of the n swapped-out sequences gets
 * a GPU block; pairs are (host block, gpu block) for pa_swap_blocks (host
 * pools -> device pools).  All or nothing: PA_ERR_NO_BLOCKS if the GPU pool
 * is short; PA_ERR_SHAPE if a sequence is not swapped out, is listed twice,
 * or max_pairs is too small.
 */
int pa_manager_swap_in(pa_manager *m, const int64_t *seqs, int n, int64_t *pairs,
                       int max_pairs, int *num_pairs);

/*
 * Block tables and context lengths of n resident sequences, for pa_decode:
 * tables [n][max_blocks] (entries past a sequence's blocks = -1),
 * context_lens [n].  PA_ERR_SHAPE if a sequence has more than max_blocks
 * blocks; PA_ERR_SWAPPED if one is swapped out.
 */
int pa_manager_tables(const pa_manager *m, const int64_t *seqs, int n, int32_t *tables,
                      int max_blocks, int32_t *context_lens);

/* Queries. */
int pa_manager_num_free(const pa_manager *m);
int pa_manager_num_free_host(const pa_manager *m);
int pa_manager_is_swapped(const pa_manager *m, int64_t seq);  /* 1, 0, or < 0 */
int pa_manager_num_sequences(const pa_manager *m);
int pa_manager_refcount(const pa_manager *m, int block);  /* < 0: bad block */
int pa_manager_length(const pa_manager *m, int64_t seq);   /* tokens, or < 0 */

/*
 * Internal consistency, on both pools: every count equals the number of
 * logical blocks referencing the block; the free lists hold exactly the
 * blocks at count 0, once each; every sequence holds ceil(length /
 * block_size) blocks.
 * PA_OK or PA_ERR_SHAPE.
 */
int pa_manager_check(const pa_manager *m);

#ifdef __cplusplus
}
#endif

#endif /* PA_MANAGER_H */
