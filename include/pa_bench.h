/*
 * pa_bench.h -- reference read kernels for measurement (libpa_bench.so).
 *
 * Not part of the attention library: these two kernels give the ceilings
 * that the paged decode's HBM rate is read against.  The pages' decode is a
 * matrix-vector product that is bound by memory reads (the wywy.jp notes,
 * Keyword "autoregressive generation phase"); these kernels read the same
 * bytes with no arithmetic and no per-item structure.
 *
 * Every pointer is device memory owned by the caller; work is enqueued on
 * `stream` (a hipStream_t, NULL = default) and nothing synchronises.
 * Return value: 0, -1 (a NULL pointer), -2 (a size or alignment out of
 * range), -5 (the HIP runtime rejected the launch).
 */
#ifndef PA_BENCH_H
#define PA_BENCH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Read `bytes` (a multiple of 16) of the 16-byte aligned buffer `buf` once,
 * with `grid` workgroups of 256 threads striding over tiles of 4 * unroll
 * KiB (16-byte non-temporal loads, `unroll` per thread in flight; unroll is
 * 1, 2, 4 or 8, else -2).  sink: device uint32 [grid], written only in the
 * practically impossible case that the folded words equal a fixed constant
 * (it keeps the loads alive).
 */
int pa_bench_stream_read(const void *buf, size_t bytes, int grid, int unroll, void *sink,
                         void *stream);

/*
 * Read num_pieces pieces of piece_bytes (a multiple of 16) from each of the
 * two pools (k_pool and v_pool, pool_bytes each, 16-byte aligned): piece i
 * starts at byte offsets[i] (int64, device memory) of both.  One wave reads
 * one piece of each pool; a piece outside the pools is skipped.  With the
 * paged decode's (block, head) tiles as pieces -- offset (phys * num_heads
 * + h) * block_size * head_dim * element bytes -- this is the decode's
 * gather with nothing else.  sink: device uint32 [ceil(num_pieces / 4)],
 * as above.
 */
int pa_bench_gather_read(const void *k_pool, const void *v_pool, size_t pool_bytes,
                         const int64_t *offsets, int num_pieces, int piece_bytes, void *sink,
                         void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_BENCH_H */
