/*
 * CPU check of the oracle (oracle/oracle.c) under the address and
 * undefined-behaviour sanitizers, built with gcc by tests/test_sanitizers.py
 * (without OpenMP, so every loop runs on one thread under the checkers).
 * Every entry point runs on seeded random shapes, fp16 and fp32, including
 * empty contexts, ragged last blocks, NaN in unused slots, subsets of rows,
 * weights, and each error path (entries outside the pool, repeated slots,
 * conflicting copy pairs, malformed query ranges).  Beside memory safety it
 * checks two closed forms on every decode: a context of one token returns
 * that token's V row exactly, and the weights of every row sum to 1.
 * Exits 0 when everything holds.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_decode(double *out, const void *q, const void *k_pool, const void *v_pool,
                  const int32_t *block_tables, const int32_t *context_lens, int N, int H, int D,
                  int B, int NB, int MB, float scale, int dtype, const int32_t *pairs,
                  int num_pairs, double *weights, int weights_stride, int threads);
int oracle_prefill(double *out, const void *q, const void *k_pool, const void *v_pool,
                   const int32_t *block_tables, const int32_t *context_lens,
                   const int32_t *query_start, int N, int H, int D, int B, int NB, int MB,
                   float scale, int dtype, int threads);
int oracle_write_kv(const void *key, const void *value, void *k_pool, void *v_pool,
                    const int64_t *slot_mapping, int num_tokens, int H, int D, int B, int NB,
                    int dtype);
int oracle_copy_blocks(void *k_pool, void *v_pool, const int64_t *block_mapping, int num_pairs,
                       int H, int D, int B, int NB, int dtype);
int oracle_swap_blocks(void *dst_k, void *dst_v, const void *src_k, const void *src_v,
                       const int64_t *block_mapping, int num_pairs, int H, int D, int B,
                       int src_NB, int dst_NB, int dtype);
void oracle_half_to_double_array(const uint16_t *src, double *dst, int64_t n);

static uint64_t g_state = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64(void)
{ /* xorshift64* */
    g_state ^= g_state >> 12;
    g_state ^= g_state << 25;
    g_state ^= g_state >> 27;
    return g_state * 2685821657736338717ull;
}
static int uni(int lo, int hi) { return lo + (int)(next_u64() % (uint64_t)(hi - lo + 1)); }
static double unit(void) { return (double)(next_u64() >> 11) * (1.0 / 9007199254740992.0); }

static int g_checks = 0;
#define CHECK(cond, msg)                                                            \
    do {                                                                            \
        ++g_checks;                                                                 \
        if (!(cond)) {                                                              \
            fprintf(stderr, "FAIL %s:%d: %s (%s)\n", __FILE__, __LINE__, #cond, msg); \
            exit(1);                                                                \
        }                                                                           \
    } while (0)

/* A random finite value in the element type, or NaN. */
static void put(void *base, int dtype, size_t i, double v)
{
    if (dtype == 1) {
        ((float *)base)[i] = (float)v;
    } else {
        /* a binary16 pattern: random sign, exponent 10..20 (about 2^-5..2^5), fraction */
        uint16_t h;
        if (isnan(v)) h = 0x7e00;
        else h = (uint16_t)(((v < 0) << 15) | (uni(10, 20) << 10) | uni(0, 1023));
        ((uint16_t *)base)[i] = h;
    }
}

static int es_of(int dtype) { return dtype == 1 ? 4 : 2; }

static void check_half(void)
{
    uint16_t *h = malloc(65536 * sizeof *h);
    double *d = malloc(65536 * sizeof *d);
    for (int i = 0; i < 65536; ++i) h[i] = (uint16_t)i;
    oracle_half_to_double_array(h, d, 65536);
    CHECK(d[0x3c00] == 1.0 && d[0xbc00] == -1.0 && d[0x0001] == ldexp(1.0, -24) &&
              isinf(d[0x7c00]) && isnan(d[0x7e00]) && d[0x7bff] == 65504.0,
          "binary16 landmarks");
    free(h);
    free(d);
}

static void check_decode_and_friends(int iter)
{
    const int dtype = uni(0, 1), es = es_of(dtype);
    const int H = uni(1, 3), D = uni(1, 2) * 32, B = 1 << uni(0, 5);
    const int N = uni(1, 6), MB = uni(1, 6), NB = N * MB + uni(1, 5);
    const size_t row = (size_t)D, tile = (size_t)B * D, blk = (size_t)H * tile;
    char *k = malloc((size_t)NB * blk * es), *v = malloc((size_t)NB * blk * es);
    char *q = malloc((size_t)N * H * D * es);
    int32_t *tables = malloc(sizeof(int32_t) * N * MB), *ctx = malloc(sizeof(int32_t) * N);
    double *out = malloc(sizeof(double) * N * H * D);
    double *w = malloc(sizeof(double) * N * H * MB * B);
    int *perm = malloc(sizeof(int) * NB);
    for (int i = 0; i < NB; ++i) perm[i] = i;
    for (int i = NB - 1; i > 0; --i) {
        const int j = uni(0, i), t = perm[i];
        perm[i] = perm[j];
        perm[j] = t;
    }
    for (size_t i = 0; i < (size_t)NB * blk; ++i) {
        put(k, dtype, i, NAN);
        put(v, dtype, i, NAN);
    }
    for (size_t i = 0; i < (size_t)N * H * D; ++i) put(q, dtype, i, unit() - 0.5);
    int cursor = 0;
    for (int b = 0; b < N; ++b) {
        ctx[b] = uni(0, 3) == 0 ? uni(0, 1) : uni(1, MB * B);
        const int nb = (ctx[b] + B - 1) / B;
        for (int j = 0; j < MB; ++j) tables[b * MB + j] = j < nb ? perm[cursor + j] : -1;
        for (int t = 0; t < ctx[b]; ++t) {
            const int p = tables[b * MB + t / B];
            for (int h = 0; h < H; ++h)
                for (int d = 0; d < D; ++d) {
                    const size_t i = (size_t)p * blk + h * tile + (size_t)(t % B) * row + d;
                    put(k, dtype, i, unit() - 0.5);
                    put(v, dtype, i, unit() - 0.5);
                }
        }
        cursor += nb;
    }
    const float scale = 1.0f / sqrtf((float)D);
    int rc = oracle_decode(out, q, k, v, tables, ctx, N, H, D, B, NB, MB, scale, dtype, NULL, 0,
                           w, MB * B, 0);
    CHECK(rc == 0, "decode");
    for (int b = 0; b < N; ++b)
        for (int h = 0; h < H; ++h) {
            const double *o = out + ((size_t)b * H + h) * D;
            if (ctx[b] == 0) {
                for (int d = 0; d < D; ++d) CHECK(o[d] == 0.0, "empty context gives zeros");
                continue;
            }
            double s = 0;
            for (int t = 0; t < ctx[b]; ++t) s += w[((size_t)b * H + h) * MB * B + t];
            CHECK(fabs(s - 1.0) < 1e-12, "weights sum to 1");
            for (int d = 0; d < D; ++d) CHECK(isfinite(o[d]), "NaN in unused slots leaked");
            if (ctx[b] == 1) {
                const size_t i0 = (size_t)tables[b * MB] * blk + h * tile;
                double vv[1];
                for (int d = 0; d < D; ++d) {
                    if (dtype == 1) vv[0] = ((float *)v)[i0 + d];
                    else oracle_half_to_double_array((uint16_t *)v + i0 + d, vv, 1);
                    CHECK(o[d] == vv[0], "one token returns its V row");
                }
            }
        }
    /* a subset of (b, h) rows */
    int32_t pr[2] = {N - 1, H - 1};
    rc = oracle_decode(out, q, k, v, tables, ctx, N, H, D, B, NB, MB, scale, dtype, pr, 1, NULL,
                       0, 1);
    CHECK(rc == 0, "decode of a subset");
    /* an entry outside the pool is an error, not a read */
    for (int b = 0; b < N; ++b)
        if (ctx[b] > 0) {
            const int32_t keep = tables[b * MB];
            tables[b * MB] = NB + uni(0, 3);
            CHECK(oracle_decode(out, q, k, v, tables, ctx, N, H, D, B, NB, MB, scale, dtype,
                                NULL, 0, NULL, 0, 1) != 0,
                  "table entry outside the pool");
            tables[b * MB] = keep;
            break;
        }

    /* prefill: each sequence's last m tokens are queries */
    int32_t *qs = malloc(sizeof(int32_t) * (N + 1));
    qs[0] = 0;
    for (int b = 0; b < N; ++b) qs[b + 1] = qs[b] + (ctx[b] ? uni(0, ctx[b]) : 0);
    const int T = qs[N];
    if (dtype == 0 && T > 0) {
        char *pq = malloc((size_t)T * H * D * es);
        double *po = malloc(sizeof(double) * T * H * D);
        for (size_t i = 0; i < (size_t)T * H * D; ++i) put(pq, dtype, i, unit() - 0.5);
        rc = oracle_prefill(po, pq, k, v, tables, ctx, qs, N, H, D, B, NB, MB, scale, dtype, 1);
        CHECK(rc == 0, "prefill");
        for (size_t i = 0; i < (size_t)T * H * D; ++i) CHECK(isfinite(po[i]), "prefill finite");
        int32_t saved = qs[1];
        qs[1] = qs[0] + ctx[0] + 1; /* more queries than context: refused before any read */
        rc = oracle_prefill(po, pq, k, v, tables, ctx, qs, N, H, D, B, NB, MB, scale, dtype, 1);
        CHECK(rc != 0, "malformed query range rejected");
        qs[1] = saved;
        free(pq);
        free(po);
    }
    free(qs);

    /* write: distinct slots, some skipped; a repeated slot is refused */
    const int T2 = uni(1, 8);
    char *key = malloc((size_t)T2 * H * D * es), *val = malloc((size_t)T2 * H * D * es);
    int64_t *slots = malloc(sizeof(int64_t) * T2);
    for (size_t i = 0; i < (size_t)T2 * H * D; ++i) {
        put(key, dtype, i, unit());
        put(val, dtype, i, unit());
    }
    for (int i = 0; i < T2; ++i) slots[i] = (i % 3 == 2) ? -1 : (int64_t)i * 7 % ((int64_t)NB * B);
    int distinct = 1;
    for (int i = 0; i < T2; ++i)
        for (int j = 0; j < i; ++j)
            if (slots[i] >= 0 && slots[i] == slots[j]) distinct = 0;
    rc = oracle_write_kv(key, val, k, v, slots, T2, H, D, B, NB, dtype);
    CHECK(distinct ? rc == 0 : rc != 0, "write");
    if (T2 >= 2) {
        slots[0] = 0;
        slots[1] = 0;
        CHECK(oracle_write_kv(key, val, k, v, slots, T2, H, D, B, NB, dtype) != 0,
              "repeated slot refused");
    }
    slots[0] = (int64_t)NB * B;
    CHECK(oracle_write_kv(key, val, k, v, slots, 1, H, D, B, NB, dtype) != 0,
          "slot outside the pool refused");

    /* copy: one source to several destinations; conflicts refused */
    if (NB >= 4) {
        int64_t pairs[4] = {0, 1, 0, 2};
        rc = oracle_copy_blocks(k, v, pairs, 2, H, D, B, NB, dtype);
        CHECK(rc == 0, "copy");
        CHECK(memcmp(k, k + blk * es, blk * es) == 0, "copied block equals its source");
        int64_t bad[4] = {0, 1, 1, 2}; /* a destination that is also a source */
        CHECK(oracle_copy_blocks(k, v, bad, 2, H, D, B, NB, dtype) != 0, "conflict refused");
        int64_t out_of[2] = {0, NB};
        CHECK(oracle_copy_blocks(k, v, out_of, 1, H, D, B, NB, dtype) != 0, "outside refused");
    }

    /* swap into another pool and back */
    const int NB2 = uni(NB, NB + 3);
    char *hk = malloc((size_t)NB2 * blk * es), *hv = malloc((size_t)NB2 * blk * es);
    memset(hk, 0, (size_t)NB2 * blk * es);
    memset(hv, 0, (size_t)NB2 * blk * es);
    int64_t *sp = malloc(sizeof(int64_t) * 2 * NB);
    for (int i = 0; i < NB; ++i) {
        sp[2 * i] = i;
        sp[2 * i + 1] = NB2 - 1 - i;
    }
    CHECK(oracle_swap_blocks(hk, hv, k, v, sp, NB, H, D, B, NB, NB2, dtype) == 0, "swap out");
    for (int i = 0; i < NB; ++i)
        CHECK(memcmp(hk + (size_t)(NB2 - 1 - i) * blk * es, k + (size_t)i * blk * es,
                     blk * es) == 0,
              "swapped block");
    (void)iter;
    free(sp);
    free(hk);
    free(hv);
    free(key);
    free(val);
    free(slots);
    free(k);
    free(v);
    free(q);
    free(tables);
    free(ctx);
    free(out);
    free(w);
    free(perm);
}

int main(int argc, char **argv)
{
    if (argc > 1) g_state ^= strtoull(argv[1], NULL, 10) * 0x9E3779B97F4A7C15ull;
    check_half();
    for (int i = 0; i < 400; ++i) check_decode_and_friends(i);
    printf("oracle_check ok: %d checks\n", g_checks);
    return 0;
}
