/*
 * Paged decode attention: plain fp64 CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the tests, the smoke check and the benchmark's CPU
 * baseline use it.  It shares no source, header, table or helper with the
 * HIP library: its own binary16 decoder, its own index arithmetic, its own
 * constants.
 *
 * What it computes (Kwon et al., "Efficient Memory Management for Large
 * Language Model Serving with PagedAttention", as summarised on the three
 * pages):
 *
 *  - decode: for one query token per (sequence, head), the block-wise attention
 *    of the zhaifeiyue.github.io summary, "method" paragraph, equation for
 *    A_ij and o_i: scores of the query against the keys of every KV block j,
 *    a softmax whose denominator runs over all blocks of the context, and the
 *    output o = sum_j V_j A_ij^T.  Keys and values live in separate block
 *    pools (wywy.jp notes, Keyword "PagedAttention"); a per-sequence block
 *    table maps logical block j to a physical block (wywy.jp, Keyword "Block
 *    table"; ricepunchb.github.io notes, section 3.2 "address translation":
 *    block index, block offset, physical address).
 *  - write_kv: each decoding step stores the new token's K and V at the next
 *    free position of the sequence's last block (wywy.jp, Keyword
 *    "autoregressive generation phase" and "KV cache manager"; zhaifeiyue,
 *    "KV Cache Manager" paragraph and memory-management table, "Allocate").
 *  - copy_blocks: block-granular copy-on-write, the block engine copying one
 *    physical block's contents into a newly allocated one (wywy.jp, WHERE,
 *    parallel-sampling example with physical blocks 1 and 3; zhaifeiyue,
 *    memory-management table, "Copy-on-Write"; ricepunchb section 5.1).
 *  - prefill: the prompt phase, where every prompt token is known and all of
 *    them are processed together (wywy.jp Keyword "prompt phase"; the shared
 *    prefix of WHERE, whose cached KV is reused so that only the
 *    request-specific tokens are computed).  The queries of a sequence are
 *    the last tokens of its context; the query at position p attends
 *    causally to tokens 0..p, that is, it is the decode above over the
 *    context truncated to p + 1 tokens.
 *  - swap_blocks: swapping, the recovery that moves every KV block of an
 *    evicted sequence from GPU memory to CPU memory and back whole when it
 *    resumes (wywy.jp, Keyword "Swapping" and "All-or-nothing eviction",
 *    Overview, scheduling and preemption; zhaifeiyue, "Scheduling &
 *    Preemption" table, row "Swap"): each listed block of one pool pair is
 *    copied onto a block of another pool pair of the same shape per block.
 *
 * Readings taken where the pages are silent or garbled:
 *  - token t (0-based) of a sequence lives in logical block t div B at offset
 *    t mod B; the physical block is block_tables[b][t div B];
 *  - slots at offset >= the filled count of the last block are not part of
 *    the context (they may hold anything, NaN included);
 *  - the scale in the exponent is the caller's fp32 `scale`, widened exactly;
 *  - the softmax subtracts the maximum score first (an exact identity in real
 *    arithmetic); sums run in ascending logical token order;
 *  - a context of length 0 gives a zero output;
 *  - pool layout is [num_blocks][num_heads][block_size][head_dim], row-major,
 *    K and V in two separate pools indexed by the same table.
 *
 * Parity pins (checked by the CPU tests): exhaustive binary16 decoding,
 * dense softmax attention from a library routine after gathering, a literal
 * 40-digit evaluation of the block-wise equation, closed forms (one token,
 * zero query, equal keys, two tokens, weights summing to one), invariance
 * under re-placement, block size and shared-versus-copied prefixes, the
 * pages' copy-on-write example and sharing diagram, an append-process
 * simulation of the manager for the address translation, and for the swap a
 * round trip that leaves the decode unchanged, whole-block slices and its
 * reduction to copy_blocks within one pool.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Element type codes understood by the oracle (the same numbering as the
 * library's public header, restated here so that the two share no file). */
#define ORC_F16 0
#define ORC_F32 1

#define ORC_OK 0
#define ORC_BAD_ARG -1
#define ORC_BAD_TABLE -2
#define ORC_BAD_SLOT -3
#define ORC_BAD_PAIRS -4

/* IEEE-754 binary16 -> double: sign bit, 5 exponent bits (bias 15), 10
 * fraction bits; exponent 0 is subnormal (fraction * 2^-24), exponent 31 is
 * infinity or NaN. */
double oracle_half_to_double(uint16_t h)
{
    const int sign = (h >> 15) & 1;
    const int expo = (h >> 10) & 0x1f;
    const int frac = h & 0x3ff;
    double v;
    if (expo == 0)
        v = ldexp((double)frac, -24);
    else if (expo == 31)
        v = frac ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + frac), expo - 25);
    return sign ? -v : v;
}

void oracle_half_to_double_array(const uint16_t *src, double *dst, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        dst[i] = oracle_half_to_double(src[i]);
}

static int elem_bytes(int dtype)
{
    if (dtype == ORC_F16)
        return 2;
    if (dtype == ORC_F32)
        return 4;
    return 0;
}

/* Element `idx` of an array of the given type, widened exactly to double. */
static double load_elem(const void *base, int dtype, int64_t idx)
{
    if (dtype == ORC_F16) {
        uint16_t bits;
        memcpy(&bits, (const char *)base + idx * 2, 2);
        return oracle_half_to_double(bits);
    }
    float f;
    memcpy(&f, (const char *)base + idx * 4, 4);
    return (double)f;
}

/* Index of element (block, head, offset, dim) in a [NB][H][B][D] pool. */
static int64_t pool_index(int64_t block, int head, int offset, int dim,
                          int H, int B, int D)
{
    return ((block * H + head) * (int64_t)B + offset) * D + dim;
}

/*
 * Decode for one (sequence b, head h): out[D] (double), and optionally the
 * normalised attention weights of the ctx tokens in weights[0..ctx).
 * Returns ORC_OK or ORC_BAD_TABLE.
 */
static int decode_one(double *out, double *weights,
                      const void *q, const void *k_pool, const void *v_pool,
                      const int32_t *block_tables, const int32_t *context_lens,
                      int b, int h, int H, int D, int B, int NB, int MB,
                      double scale, int dtype)
{
    const int n = context_lens[b];
    for (int d = 0; d < D; ++d)
        out[d] = 0.0;
    if (n <= 0)
        return ORC_OK;

    const int nblk = (n + B - 1) / B;
    if (nblk > MB)
        return ORC_BAD_TABLE;

    double *qv = (double *)malloc(sizeof(double) * (size_t)D);
    double *s = (double *)malloc(sizeof(double) * (size_t)n);
    int64_t *phys = (int64_t *)malloc(sizeof(int64_t) * (size_t)nblk);
    if (!qv || !s || !phys) {
        free(qv);
        free(s);
        free(phys);
        return ORC_BAD_ARG;
    }
    for (int d = 0; d < D; ++d)
        qv[d] = load_elem(q, dtype, ((int64_t)b * H + h) * D + d);

    /* Address translation: logical block j -> physical block. */
    for (int j = 0; j < nblk; ++j) {
        const int32_t p = block_tables[(int64_t)b * MB + j];
        if (p < 0 || p >= NB) {
            free(qv);
            free(s);
            free(phys);
            for (int d = 0; d < D; ++d)
                out[d] = NAN;
            return ORC_BAD_TABLE;
        }
        phys[j] = p;
    }

    /* Scores, block by block: the row A_ij before normalisation.  Only the
     * filled positions of each block take part. */
    for (int j = 0; j < nblk; ++j) {
        const int filled = (n - j * B < B) ? (n - j * B) : B;
        for (int o = 0; o < filled; ++o) {
            double dot = 0.0;
            for (int d = 0; d < D; ++d)
                dot += qv[d] * load_elem(k_pool, dtype, pool_index(phys[j], h, o, d, H, B, D));
            s[j * B + o] = scale * dot;
        }
    }

    /* Softmax over every token of every block: max first, then the
     * denominator summed in ascending token order. */
    double m = s[0];
    for (int t = 1; t < n; ++t)
        if (s[t] > m)
            m = s[t];
    double z = 0.0;
    for (int t = 0; t < n; ++t)
        z += exp(s[t] - m);

    /* o = sum_j V_j A_ij^T, ascending token order. */
    for (int j = 0; j < nblk; ++j) {
        const int filled = (n - j * B < B) ? (n - j * B) : B;
        for (int o = 0; o < filled; ++o) {
            const double w = exp(s[j * B + o] - m) / z;
            if (weights)
                weights[j * B + o] = w;
            for (int d = 0; d < D; ++d)
                out[d] += w * load_elem(v_pool, dtype, pool_index(phys[j], h, o, d, H, B, D));
        }
    }
    free(qv);
    free(s);
    free(phys);
    return ORC_OK;
}

/*
 * out: double [N][H][D].  pairs: optional list of (b, h) int32 pairs to
 * compute (num_pairs of them); NULL computes every (b, h).  weights:
 * optional double [N][H][weights_stride]; row (b, h) receives the ctx[b]
 * normalised weights.  threads: OpenMP threads (<= 0: library default).
 * Returns ORC_OK or the first error code met.
 */
int oracle_decode(double *out, const void *q, const void *k_pool, const void *v_pool,
                  const int32_t *block_tables, const int32_t *context_lens,
                  int N, int H, int D, int B, int NB, int MB, float scale, int dtype,
                  const int32_t *pairs, int num_pairs,
                  double *weights, int weights_stride, int threads)
{
    if (!out || !q || !k_pool || !v_pool || !block_tables || !context_lens)
        return ORC_BAD_ARG;
    if (N < 0 || H <= 0 || D <= 0 || B <= 0 || NB < 0 || MB < 0 || !elem_bytes(dtype))
        return ORC_BAD_ARG;
    const int total = pairs ? num_pairs : N * H;
    int status = ORC_OK;
#ifdef _OPENMP
    if (threads <= 0)
        threads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(threads)
#endif
    for (int i = 0; i < total; ++i) {
        const int b = pairs ? pairs[2 * i] : i / H;
        const int h = pairs ? pairs[2 * i + 1] : i % H;
        if (b < 0 || b >= N || h < 0 || h >= H) {
#ifdef _OPENMP
#pragma omp critical
#endif
            status = ORC_BAD_ARG;
            continue;
        }
        double *w = weights ? weights + ((int64_t)b * H + h) * weights_stride : NULL;
        if (w && context_lens[b] > weights_stride) {
#ifdef _OPENMP
#pragma omp critical
#endif
            status = ORC_BAD_ARG;
            continue;
        }
        const int rc = decode_one(out + ((int64_t)b * H + h) * D, w, q, k_pool, v_pool,
                                  block_tables, context_lens, b, h, H, D, B, NB, MB,
                                  (double)scale, dtype);
        if (rc != ORC_OK) {
#ifdef _OPENMP
#pragma omp critical
#endif
            status = rc;
        }
    }
    return status;
}

/*
 * Prefill: sequence b has context_lens[b] = n tokens in the pools, of which
 * the last m = query_start[b+1] - query_start[b] are queries, in rows
 * query_start[b] .. query_start[b+1]-1 of q and out ([T][H][D]).  Query i
 * of the chunk is the token at position p = n - m + i; its output is the
 * attention of its q row over tokens 0..p of the sequence.  query_start must
 * start at 0, not decrease, and give every sequence m <= n.
 */
int oracle_prefill(double *out, const void *q, const void *k_pool, const void *v_pool,
                   const int32_t *block_tables, const int32_t *context_lens,
                   const int32_t *query_start, int N, int H, int D, int B, int NB, int MB,
                   float scale, int dtype, int threads)
{
    if (!out || !q || !k_pool || !v_pool || !block_tables || !context_lens || !query_start)
        return ORC_BAD_ARG;
    if (N < 0 || H <= 0 || D <= 0 || B <= 0 || NB < 0 || MB < 0 || !elem_bytes(dtype))
        return ORC_BAD_ARG;
    if (query_start[0] != 0)
        return ORC_BAD_ARG;
    for (int b = 0; b < N; ++b) {
        const int m = query_start[b + 1] - query_start[b];
        if (m < 0 || m > context_lens[b])
            return ORC_BAD_ARG;
    }
    const int T = query_start[N];
    int status = ORC_OK;
#ifdef _OPENMP
    if (threads <= 0)
        threads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 4) num_threads(threads)
#endif
    for (int64_t i = 0; i < (int64_t)T * H; ++i) {
        const int row = (int)(i / H), h = (int)(i % H);
        int b = 0;
        while (query_start[b + 1] <= row)
            ++b;
        const int n = context_lens[b];
        const int m = query_start[b + 1] - query_start[b];
        const int32_t visible = n - m + (row - query_start[b]) + 1;   /* tokens 0..p */
        const int rc = decode_one(out + ((int64_t)row * H + h) * D, NULL,
                                  (const char *)q + (int64_t)row * H * D * elem_bytes(dtype),
                                  k_pool, v_pool, block_tables + (int64_t)b * MB, &visible,
                                  0, h, H, D, B, NB, MB, (double)scale, dtype);
        if (rc != ORC_OK) {
#ifdef _OPENMP
#pragma omp critical
#endif
            status = rc;
        }
    }
    return status;
}

int oracle_threads_available(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Store token i's key and value rows (all heads) at physical block
 * slot div B, offset slot mod B of the two pools.  A negative slot skips the
 * token.  Slots must be distinct and below NB*B.  Byte copies: the stored
 * bits equal the input bits.
 */
int oracle_write_kv(const void *key, const void *value, void *k_pool, void *v_pool,
                    const int64_t *slot_mapping, int num_tokens,
                    int H, int D, int B, int NB, int dtype)
{
    const int es = elem_bytes(dtype);
    if (!key || !value || !k_pool || !v_pool || !slot_mapping || num_tokens < 0 || !es)
        return ORC_BAD_ARG;
    if (H <= 0 || D <= 0 || B <= 0 || NB < 0)
        return ORC_BAD_ARG;
    for (int i = 0; i < num_tokens; ++i) {
        const int64_t si = slot_mapping[i];
        if (si < 0)
            continue;
        if (si >= (int64_t)NB * B)
            return ORC_BAD_SLOT;
        for (int k = 0; k < i; ++k)
            if (slot_mapping[k] == si)
                return ORC_BAD_SLOT;
    }
    const size_t row = (size_t)D * es;
    for (int i = 0; i < num_tokens; ++i) {
        const int64_t slot = slot_mapping[i];
        if (slot < 0)
            continue;
        const int64_t block = slot / B;
        const int offset = (int)(slot % B);
        for (int h = 0; h < H; ++h) {
            const int64_t src = ((int64_t)i * H + h) * D;
            const int64_t dst = pool_index(block, h, offset, 0, H, B, D);
            memcpy((char *)k_pool + dst * es, (const char *)key + src * es, row);
            memcpy((char *)v_pool + dst * es, (const char *)value + src * es, row);
        }
    }
    return ORC_OK;
}

/*
 * For each (src, dst) pair copy all of physical block src (every head, every
 * offset) onto block dst, in both pools.  Destinations must be distinct and
 * must not also appear as sources; one source may feed many destinations.
 */
int oracle_copy_blocks(void *k_pool, void *v_pool, const int64_t *block_mapping,
                       int num_pairs, int H, int D, int B, int NB, int dtype)
{
    const int es = elem_bytes(dtype);
    if (!k_pool || !v_pool || (num_pairs > 0 && !block_mapping) || num_pairs < 0 || !es)
        return ORC_BAD_ARG;
    for (int i = 0; i < num_pairs; ++i) {
        const int64_t src = block_mapping[2 * i], dst = block_mapping[2 * i + 1];
        if (src < 0 || src >= NB || dst < 0 || dst >= NB)
            return ORC_BAD_PAIRS;
        for (int k = 0; k < num_pairs; ++k) {
            if (k != i && block_mapping[2 * k + 1] == dst)
                return ORC_BAD_PAIRS;
            if (block_mapping[2 * k] == dst)
                return ORC_BAD_PAIRS;
        }
    }
    const size_t block_bytes = (size_t)H * B * D * es;
    for (int i = 0; i < num_pairs; ++i) {
        const int64_t src = block_mapping[2 * i], dst = block_mapping[2 * i + 1];
        memcpy((char *)k_pool + dst * block_bytes, (const char *)k_pool + src * block_bytes, block_bytes);
        memcpy((char *)v_pool + dst * block_bytes, (const char *)v_pool + src * block_bytes, block_bytes);
    }
    return ORC_OK;
}

/*
 * For each (src, dst) pair copy every element (head, offset, dim) of block
 * src of the source pools onto block dst of the destination pools, K and V.
 * The two pool pairs may hold different numbers of blocks (src_NB, dst_NB)
 * and must not overlap.  Destinations must be distinct; a source may be
 * listed more than once.
 */
int oracle_swap_blocks(void *dst_k, void *dst_v, const void *src_k, const void *src_v,
                       const int64_t *block_mapping, int num_pairs, int H, int D, int B,
                       int src_NB, int dst_NB, int dtype)
{
    const int es = elem_bytes(dtype);
    if (!dst_k || !dst_v || !src_k || !src_v || (num_pairs > 0 && !block_mapping) ||
        num_pairs < 0 || !es)
        return ORC_BAD_ARG;
    for (int i = 0; i < num_pairs; ++i) {
        const int64_t src = block_mapping[2 * i], dst = block_mapping[2 * i + 1];
        if (src < 0 || src >= src_NB || dst < 0 || dst >= dst_NB)
            return ORC_BAD_PAIRS;
        for (int k = 0; k < i; ++k)
            if (block_mapping[2 * k + 1] == dst)
                return ORC_BAD_PAIRS;
    }
    for (int i = 0; i < num_pairs; ++i) {
        const int64_t src = block_mapping[2 * i], dst = block_mapping[2 * i + 1];
        for (int h = 0; h < H; ++h)
            for (int o = 0; o < B; ++o)
                for (int d = 0; d < D; ++d) {
                    const int64_t from = pool_index(src, h, o, d, H, B, D);
                    const int64_t to = pool_index(dst, h, o, d, H, B, D);
                    memcpy((char *)dst_k + to * es, (const char *)src_k + from * es, es);
                    memcpy((char *)dst_v + to * es, (const char *)src_v + from * es, es);
                }
    }
    return ORC_OK;
}
