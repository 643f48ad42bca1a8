// Paged prefill attention (the prompt phase) on MFMA.
//
// Every prompt token is known in the prompt phase, so all of them are
// processed at once and the work is matrix-matrix (the wywy.jp notes on
// PagedAttention, Keyword "prompt phase"); a cached shared prefix is reused
// and only the request's own tokens are computed (same notes, WHERE, shared
// prefix).  Sequence b holds n tokens in the paged pools; its last m are
// queries (rows query_start[b] .. query_start[b+1]-1 of q and out), and the
// query at position p attends to tokens 0..p through the block table (the
// block-wise equation of the zhaifeiyue.github.io summary, method paragraph,
// with the context cut at the query's own position).
//
// One workgroup = one (head, sequence, tile of 128 queries); 4 waves of 32
// queries each.  The waves share each staged K/V tile; a wave skips the
// products of tiles past its last query and, holding no query, all of them.  Per 32-key tile, on v_mfma_f32_32x32x16_f16:
//   * S^T = K Q^T: key rows are the A operand, the wave's 32 query rows the
//     B operand (kept in registers for the whole loop).  The contraction
//     over head_dim runs in a permuted order both operands share (lane
//     group g takes the half [g*D/2, (g+1)*D/2)), so each lane reads one
//     contiguous half row.
//   * In the accumulator layout every lane holds 16 scores of one query
//     (its column): the online softmax needs one exchange (lanes l, l ^ 32)
//     per tile and rescaling the output is a per-lane multiply.
//   * O^T += V^T P^T: P^T is the B operand straight from the score
//     registers (converted to fp16, no shuffle); the key order this implies
//     is matched by the A operand, V^T, read from LDS.
// A tile whose keys all precede the workgroup's last query and whose table
// entries all lie in the pool (every tile but the last, normally) is
// fetched from uniform row bases: its one to four table entries are scalar
// loads, and each thread adds an offset fixed for the whole loop.  Other
// tiles take the checked fetch, which reads each key's table entry (from an
// LDS copy of the workgroup's entries when it fits) and stages keys past
// the last query as zeros and rows of bad entries as NaN.  K and V tiles go
// through LDS, double-buffered: the next tile's global
// loads are in flight while the current tile's products run, and one
// barrier per tile separates the two buffers.  K is stored row-major with a
// 68-dword row (16-byte reads by 16 lanes hit 64 distinct banks); V is
// stored transposed, written as packed key pairs (32-bit stores) into rows
// of 18 dwords, which keeps both the pair writes and the 8-byte operand
// reads free of bank conflicts.
// Accumulation and the softmax are fp32; P is rounded to fp16 for the
// second product, and the softmax denominator sums those rounded weights
// (v_dot2 against ones, fp32 accumulation), so numerator and denominator
// use the same P.
#include <math.h>

#include "pa_kernels.h"
#include "pa_prefill.h"

namespace pa {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 half16 __attribute__((ext_vector_type(16)));
typedef unsigned uint8v __attribute__((ext_vector_type(8)));
typedef float float16v __attribute__((ext_vector_type(16)));

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kRows = 32;                 // queries per wave
constexpr int kQTile = kWaves * kRows;    // queries per workgroup
constexpr int kKeys = 32;                 // keys per tile
constexpr int kTabCache = 2048;           // block-table entries kept in LDS
constexpr float kSlack = 8.f;             // lazy-rescale slack, log2 units

template <int D>
struct Lds {
  static constexpr int kRowK = D + 8;             // halves per K row (68 dwords at D = 128)
  static constexpr int kRowV = kKeys + 4;         // halves per V^T row (18 dwords)
  static constexpr int kK = kKeys * kRowK;        // halves per K buffer
  static constexpr int kV = D * kRowV;            // halves per V^T buffer
  // one tile: K chunks (16 bytes of one key row) and V units (8 head-dim
  // values of a key pair); per thread, rounded up (the last round guarded)
  static constexpr int kKUnits = kKeys * (D / 8);                // 512 at D = 128
  static constexpr int kVUnits = (kKeys / 2) * (D / 8);          // 256 at D = 128
  static constexpr int kKChunks = (kKUnits + kThreads - 1) / kThreads;
  static constexpr int kVPairs = (kVUnits + kThreads - 1) / kThreads;
};

typedef _Float16 half2v __attribute__((ext_vector_type(2)));

// Lanes l and l ^ 32 combined.  v_permlane32_swap trades the upper half of
// its first operand with the lower half of its second; applied to two
// copies of x it leaves x[l] and x[l ^ 32] in every lane, one in each
// register.  Written as inline assembly because this compiler's builtin for
// the instruction hands back the first register twice.  The s_nop gives the
// two wait states a permlane swap needs after a VALU write of its operands.
__device__ inline void swap_halves(unsigned &a, unsigned &b) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ inline float half_max(float x) {
  unsigned a = __builtin_bit_cast(unsigned, x), b = a;
  swap_halves(a, b);
  return fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
}
__device__ inline float half_sum(float x) {
  unsigned a = __builtin_bit_cast(unsigned, x), b = a;
  swap_halves(a, b);
  return __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
}

__device__ inline half8 load_half8(const _Float16 *p) {
  return *reinterpret_cast<const half8 *>(p);
}

template <int D, int B>
struct TileLoads {
  half8 k[Lds<D>::kKChunks];
  half8 v[Lds<D>::kVPairs][2];
  bool kok[Lds<D>::kKChunks], kbad[Lds<D>::kKChunks];
  bool vok[Lds<D>::kVPairs][2];
  bool all_ok;   // every key this wave loads comes from the pool (uniform per wave)
};

// Global -> registers for keys t0 .. t0+31; keys at or past `end` (the
// workgroup's last query position + 1) are not read and stage as zeros, and
// a key whose table entry lies outside the pool stages as NaN (K) / zero
// (V).  Straight-line code: every table entry is read first, then every
// row load is issued (from the pool's first row where the key is not
// read, so that no load is conditional), so the loads overlap each other
// and the current tile's products.  The table entry comes from the
// workgroup's LDS copy when the whole row fits there (kLdsTable), else from
// global memory; the two are separate instantiations, since a pointer that
// could be either becomes a flat load whose wait also drains every global
// load in flight.
template <int D, int B, bool kLdsTable>
__device__ inline void fetch_tile(const PrefillParams &p, const int32_t *table,
                                  const __attribute__((address_space(3))) int32_t *tab, int h,
                                  int end, int t0, TileLoads<D, B> &r) {
  const _Float16 *kh = static_cast<const _Float16 *>(p.k_pool);
  const _Float16 *vh = static_cast<const _Float16 *>(p.v_pool);
  constexpr int NK = Lds<D>::kKChunks, NV = Lds<D>::kVPairs;
  int kt[NK], kd[NK], vt[NV][2], vd[NV];
  int32_t kphys[NK], vphys[NV][2];
#pragma unroll
  for (int u = 0; u < NK; ++u) {
    const int chunk = threadIdx.x + u * kThreads;   // d-chunk fastest: coalesced rows
    kt[u] = chunk < Lds<D>::kKUnits ? t0 + chunk / (D / 8) : end;
    kd[u] = (chunk % (D / 8)) * 8;
    const int j = kt[u] < end ? kt[u] / B : 0;
    kphys[u] = kLdsTable ? tab[j] : table[j];
  }
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    const int unit = threadIdx.x + u * kThreads;    // key pair fastest
    vd[u] = (unit / (kKeys / 2)) * 8;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      vt[u][s] = unit < Lds<D>::kVUnits ? t0 + 2 * (unit % (kKeys / 2)) + s : end;
      const int j = vt[u][s] < end ? vt[u][s] / B : 0;
      vphys[u][s] = kLdsTable ? tab[j] : table[j];
    }
  }
  bool all = true;
  // Element offset of a row: phys * (H B D) + (h B + t % B) D + d0, one
  // 64-bit multiply-add; keys not read point at the pool's first row.
  const uint32_t block_elems = (uint32_t)p.num_heads * B * D;
  const uint32_t head_elems = (uint32_t)h * B * D;
#pragma unroll
  for (int u = 0; u < NK; ++u) {
    const bool in = kt[u] < end;
    const bool ok = in && kphys[u] >= 0 && kphys[u] < p.num_blocks;
    r.kok[u] = ok;
    r.kbad[u] = in && !ok;
    all = all && ok;
    const uint32_t phys = ok ? (uint32_t)kphys[u] : 0u;
    const uint32_t within = ok ? head_elems + (uint32_t)(kt[u] % B) * D : 0u;
    r.k[u] = load_half8(kh + ((uint64_t)phys * block_elems + within + kd[u]));
  }
#pragma unroll
  for (int u = 0; u < NV; ++u)
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const bool ok = vt[u][s] < end && vphys[u][s] >= 0 && vphys[u][s] < p.num_blocks;
      r.vok[u][s] = ok;
      all = all && ok;
      const uint32_t phys = ok ? (uint32_t)vphys[u][s] : 0u;
      const uint32_t within = ok ? head_elems + (uint32_t)(vt[u][s] % B) * D : 0u;
      r.v[u][s] = load_half8(vh + ((uint64_t)phys * block_elems + within + vd[u]));
    }
  r.all_ok = __ballot(!all) == 0;   // uniform per wave
}

// Fast fetch, for a tile whose 32 keys all precede `end` and whose table
// entries all lie inside the pool (the common case; the caller checks both
// on uniform values).  The tile covers kTB consecutive table entries (one
// entry for B >= 32); their row bases are uniform, so every load is a
// scalar base plus a per-thread offset that does not change over the loop.
template <int D, int B>
struct FastFetch {
  static constexpr int kTB = B >= kKeys ? 1 : kKeys / B;   // table entries per tile
  static constexpr int kKPerRound = kThreads / (D / 8);     // keys one K chunk round covers
  // K chunk round u covers keys kk0 + u * kKPerRound; with kKPerRound <= B
  // its table entry is the same for every thread.
  static constexpr bool kKUniform = kKPerRound <= B;
  // Per thread, fixed over the loop: byte offsets inside a block (head,
  // row, head-dim chunk) of the first K chunk and of the first key of the V
  // pair (the second key is the next row), and their table entries.
  uint32_t koff, voff;
  int klb, vlb;
};

template <int D, int B>
__device__ inline FastFetch<D, B> fast_fetch_setup(int h) {
  FastFetch<D, B> f;
  const uint32_t head_bytes = (uint32_t)h * B * D * 2;
  const int kk = threadIdx.x / (D / 8);                       // < kKPerRound
  f.klb = B >= kKeys ? 0 : kk / B;
  f.koff = head_bytes + (uint32_t)((kk % B) * D + (threadIdx.x % (D / 8)) * 8) * 2;
  const int unit = threadIdx.x;                               // V units past kVUnits load a
  const int d0 = ((unit / (kKeys / 2)) * 8) % D;              // valid row and are not stored
  const int k0 = 2 * (unit % (kKeys / 2));
  f.vlb = B >= kKeys ? 0 : k0 / B;                            // k0 and k0 + 1 share an entry
  f.voff = head_bytes + (uint32_t)((k0 % B) * D + d0) * 2;
  return f;
}

// Reads the kTB table entries of the tile at t0 (uniform; t0 + kKeys <= end
// guarantees they lie in the row) and says whether the fast fetch applies.
template <int D, int B>
__device__ inline bool fast_tile_ok(const PrefillParams &p,
                                    const __attribute__((address_space(4))) int32_t *ctab,
                                    int end, int t0, int32_t (&phys)[FastFetch<D, B>::kTB]) {
  if (t0 + kKeys > end) return false;
  bool ok = true;
#pragma unroll
  for (int i = 0; i < FastFetch<D, B>::kTB; ++i) {
    phys[i] = ctab[t0 / B + i];
    ok = ok && phys[i] >= 0 && phys[i] < p.num_blocks;
  }
  return ok;
}

template <int D, int B>
__device__ inline void fetch_tile_fast(const PrefillParams &p, const FastFetch<D, B> &f,
                                       const int32_t (&phys)[FastFetch<D, B>::kTB], int t0,
                                       TileLoads<D, B> &r) {
  using F = FastFetch<D, B>;
  constexpr int kTB = F::kTB;
  const uint64_t block_bytes = (uint64_t)p.num_heads * B * D * 2;
  const uint64_t row0 = B > kKeys ? (uint64_t)(t0 % B) * D * 2 : 0;   // tile inside one block
  uint64_t base[kTB];
#pragma unroll
  for (int i = 0; i < kTB; ++i) base[i] = (uint64_t)(uint32_t)phys[i] * block_bytes + row0;
  const char *kp = static_cast<const char *>(p.k_pool);
  const char *vp = static_cast<const char *>(p.v_pool);
#pragma unroll
  for (int u = 0; u < Lds<D>::kKChunks; ++u) {
    uint64_t b;
    if constexpr (F::kKUniform) {
      // entry (u R) / B, row offset (u R) % B, both uniform
      b = base[(u * F::kKPerRound) / B % kTB] + (uint64_t)((u * F::kKPerRound) % B) * D * 2;
    } else {
      // rows repeat every round; the entry moves by R / B per round
      const int lb = f.klb + u * (F::kKPerRound / B);
      b = base[0];
#pragma unroll
      for (int i = 1; i < kTB; ++i) b = lb == i ? base[i] : b;
    }
    r.k[u] = *reinterpret_cast<const half8 *>(kp + b + f.koff);
  }
#pragma unroll
  for (int u = 0; u < Lds<D>::kVPairs; ++u) {
    uint64_t b = base[0];
#pragma unroll
    for (int i = 1; i < kTB; ++i) b = f.vlb == i ? base[i] : b;
    b += (uint64_t)u * (kThreads / (kKeys / 2)) * 8 * 2;   // next head-dim chunks
#pragma unroll
    for (int s = 0; s < 2; ++s)
      r.v[u][s] = *reinterpret_cast<const half8 *>(vp + b + f.voff + s * D * 2);
  }
  r.all_ok = true;
}

// Registers -> LDS buffers (K row-major, V transposed as key pairs).
template <int D, int B>
__device__ inline void store_tile(const TileLoads<D, B> &r, _Float16 *ks, _Float16 *vs) {
#pragma unroll
  for (int u = 0; u < Lds<D>::kKChunks; ++u) {
    const int chunk = threadIdx.x + u * kThreads;
    if (chunk < Lds<D>::kKUnits) {
      const int key = chunk / (D / 8), d0 = (chunk % (D / 8)) * 8;
      half8 v = r.k[u];
      if (!r.all_ok) {
        if (!r.kok[u]) v = half8{};
        if (r.kbad[u]) v = half8{} + (_Float16)NAN;   // NaN for every query that sees it
      }
      *reinterpret_cast<half8 *>(ks + key * Lds<D>::kRowK + d0) = v;
    }
  }
#pragma unroll
  for (int u = 0; u < Lds<D>::kVPairs; ++u) {
    const int unit = threadIdx.x + u * kThreads;
    if (unit < Lds<D>::kVUnits) {
      const int kp = unit % (kKeys / 2), d0 = (unit / (kKeys / 2)) * 8;
      // word e = (key 2kp, key 2kp+1) at head-dim d0 + e
      half8 v0 = r.v[u][0], v1 = r.v[u][1];
      if (!r.all_ok) {
        if (!r.vok[u][0]) v0 = half8{};
        if (!r.vok[u][1]) v1 = half8{};
      }
      const half16 z = __builtin_shufflevector(v0, v1, 0, 8, 1, 9, 2, 10, 3, 11,
                                               4, 12, 5, 13, 6, 14, 7, 15);
      const uint8v words = __builtin_bit_cast(uint8v, z);
      unsigned *col = reinterpret_cast<unsigned *>(vs + d0 * Lds<D>::kRowV + 2 * kp);
#pragma unroll
      for (int e = 0; e < 8; ++e) col[e * (Lds<D>::kRowV / 2)] = words[e];
    }
  }
}

template <int D, int B, bool kLdsTable>
__device__ void prefill_item(const PrefillParams &p, int h, int b, int qt, _Float16 *lds,
                             __attribute__((address_space(3))) int32_t *tab) {
  using L = Lds<D>;
  const int q0 = p.query_start[b];
  const int m = p.query_start[b + 1] - q0;
  const int n = min(max(p.context_lens[b], 0), p.max_context_len);
  if (qt * kQTile >= m) return;
  const bool bad_seq = m < 0 || m > n || q0 < 0 || q0 + m > p.num_query_rows;

  const int w = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int c = lane & 31;                 // this lane's query column / key row
  const int g = lane >> 5;                 // lane group
  const int r = qt * kQTile + w * kRows + c;         // query index in the chunk
  const bool q_ok = r < m && !bad_seq;
  const int pos = n - m + r;                         // its position in the sequence
  const int last = min(m, (qt + 1) * kQTile) - 1;
  const int kv_end = bad_seq ? 0 : n - m + last + 1; // keys the workgroup needs
  const int wave_pos0 = n - m + qt * kQTile + w * kRows;   // the wave's first query position
  // The wave's products are skipped when it holds no query of the chunk,
  // and for key tiles past its last query (it still stages tiles and meets
  // every barrier).
  const bool wave_active = qt * kQTile + w * kRows < m && !bad_seq;
  const int wave_last = n - m + min(m, qt * kQTile + (w + 1) * kRows) - 1;
  const int32_t *table = p.block_tables + (int64_t)b * p.max_blocks_per_seq;

  constexpr int kSteps = D / 16;
  half8 qb[kSteps];
  {
    const _Float16 *row = static_cast<const _Float16 *>(p.q) +
                          ((int64_t)(q0 + r) * p.num_heads + h) * D + g * (D / 2);
#pragma unroll
    for (int j = 0; j < kSteps; ++j) qb[j] = q_ok ? load_half8(row + 8 * j) : half8{};
  }

  float16v acc_o[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t) acc_o[t] = float16v{};
  float m_run = -INFINITY, l_run = 0.f;

  // The table entries the workgroup needs, once, into LDS.
  if (kLdsTable) {
    const int nblk = (kv_end + B - 1) / B;      // at most kTabCache here
    for (int j = threadIdx.x; j < nblk; j += kThreads) tab[j] = table[j];
  }
  // Drain the query and table loads here, once: memory counters retire in
  // order, so a wait for the query fragments inside the loop would also
  // wait for the next tile's loads issued just before it.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  const FastFetch<D, B> ff = fast_fetch_setup<D, B>(h);
  const auto *ctab = (const __attribute__((address_space(4))) int32_t *)table;
  // One tile of K/V rows into registers: the fast fetch when the tile lies
  // before kv_end with every table entry in the pool, else the checked one.
  auto fetch = [&](int t, TileLoads<D, B> &r) {
    int32_t phys[FastFetch<D, B>::kTB];
    if (fast_tile_ok<D, B>(p, ctab, kv_end, t, phys))
      fetch_tile_fast<D, B>(p, ff, phys, t, r);
    else
      fetch_tile<D, B, kLdsTable>(p, table, tab, h, kv_end, t, r);
  };

  TileLoads<D, B> next;
  if (kv_end > 0) {
    fetch(0, next);
    store_tile<D, B>(next, lds, lds + L::kK);
  }
  __syncthreads();

  int buf = 0;
  for (int t0 = 0; t0 < kv_end; t0 += kKeys) {
    const bool more = t0 + kKeys < kv_end;
    if (more) fetch(t0 + kKeys, next);
    const _Float16 *ks = lds + buf * (L::kK + L::kV);
    const _Float16 *vs = ks + L::kK;

    if (wave_active && t0 <= wave_last) {
    // S^T = K Q^T.  A operand: key row c, head-dim half g.
    float16v s = {};
    {
      const _Float16 *krow = ks + c * L::kRowK + g * (D / 2);
#pragma unroll
      for (int j = 0; j < kSteps; ++j)
        s = __builtin_amdgcn_mfma_f32_32x32x16_f16(load_half8(krow + 8 * j), qb[j], s, 0, 0, 0);
    }

    // Online softmax for this lane's query over the tile's visible keys.
    // The maximum is taken on raw scores (the scale is positive) and the
    // scale is folded into the exponent: p = 2^(s * scale_log2 - m).
    // Tiles wholly at or below every query of the wave skip the mask.
    if (t0 + kKeys - 1 > wave_pos0) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = t0 + (i / 4) * 8 + g * 4 + (i % 4);
        if (key > pos) s[i] = -INFINITY;
      }
    }
    float tile_max = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) tile_max = fmaxf(tile_max, s[i]);
    tile_max = half_max(tile_max) * p.scale_log2;
    // Lazy rescaling: the reference m_run moves only when this tile's max
    // exceeds it by more than kSlack (log2 units); otherwise the weights of
    // the tile are at most 2^kSlack, well inside fp16 and fp32.  Numerator
    // and denominator share the reference, so the result is the same
    // softmax; the output is rescaled only when some query's reference moves.
    const bool bump = tile_max > m_run + kSlack;
    const float m_new = bump ? tile_max : m_run;
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = bump ? __builtin_amdgcn_exp2f(m_run - m_use) : 1.f;
    half8 pb[2];
#pragma unroll
    for (int i = 0; i < 16; ++i)
      pb[i / 8][i % 8] = (_Float16)__builtin_amdgcn_exp2f(fmaf(s[i], p.scale_log2, -m_use));
    // The denominator sums the fp16 weights the second product uses.
    float psum = 0.f;
    const half2v one = {(_Float16)1.f, (_Float16)1.f};
#pragma unroll
    for (int i = 0; i < 8; ++i)
      psum = __builtin_amdgcn_fdot2(half2v{pb[i / 4][2 * (i % 4)], pb[i / 4][2 * (i % 4) + 1]}, one,
                                    psum, false);
    psum = half_sum(psum);
    l_run = l_run * alpha + psum;
    m_run = m_new;

    // O^T += V^T P^T.  k-step jj covers keys 16jj .. 16jj+15 in the order
    // the score registers hold them: slots 0..3 -> keys 16jj + 4g + e,
    // slots 4..7 -> keys 16jj + 8 + 4g + (e - 4).
    if (__ballot(bump)) {   // some query's reference moved
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) acc_o[dt] *= alpha;
    }
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      const _Float16 *vrow = vs + (dt * 32 + c) * L::kRowV;
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const half4 lo = *reinterpret_cast<const half4 *>(vrow + 16 * jj + 4 * g);
        const half4 hi = *reinterpret_cast<const half4 *>(vrow + 16 * jj + 8 + 4 * g);
        const half8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        acc_o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pb[jj], acc_o[dt], 0, 0, 0);
      }
    }
    }   // wave_active

    if (more) {
      _Float16 *nk = lds + (buf ^ 1) * (L::kK + L::kV);
      store_tile<D, B>(next, nk, nk + L::kK);
    }
    __syncthreads();
    buf ^= 1;
  }

  if (r >= m || q0 + r >= p.num_query_rows || r < 0) return;
  // Lane holds O^T[d][query c] for d = 32 dt + 8 (i/4) + 4 g + (i%4).
  const float inv = (bad_seq || !(l_run > 0.f)) ? NAN : 1.f / l_run;
  _Float16 *orow = static_cast<_Float16 *>(p.out) + ((int64_t)(q0 + r) * p.num_heads + h) * D;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      half4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = (_Float16)(acc_o[dt][i4 * 4 + e] * inv);
      *reinterpret_cast<half4 *>(orow + dt * 32 + i4 * 8 + g * 4) = o;
    }
}

template <int D>
constexpr int lds_halves() {
  return 2 * (Lds<D>::kK + Lds<D>::kV);
}

// Dispatch on whether the workgroup's table row fits its LDS copy (uniform
// per workgroup).
template <int D, int B>
__device__ inline void prefill_dispatch(const PrefillParams &p, int h, int b, int qt,
                                        _Float16 *lds,
                                        __attribute__((address_space(3))) int32_t *tab) {
  const int m = p.query_start[b + 1] - p.query_start[b];
  const int n = min(max(p.context_lens[b], 0), p.max_context_len);
  const int last_key = n - m + min(m, (qt + 1) * kQTile);   // kv_end when the chunk is valid
  if ((last_key + B - 1) / B <= kTabCache)
    prefill_item<D, B, true>(p, h, b, qt, lds, tab);
  else
    prefill_item<D, B, false>(p, h, b, qt, lds, tab);
}

// grid (heads, query tiles, sequences); tiles in descending order.
template <int D, int B>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3))) prefill_kernel(const PrefillParams p) {
  __shared__ __attribute__((aligned(16))) _Float16 lds[lds_halves<D>()];
  __shared__ int32_t tab[kTabCache];
  prefill_dispatch<D, B>(p, blockIdx.x, blockIdx.z, (int)gridDim.y - 1 - (int)blockIdx.y, lds,
                         (__attribute__((address_space(3))) int32_t *)tab);
}

// grid (heads, items): items = sequence << 16 | query tile, in the order the
// host planned.
template <int D, int B>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3))) prefill_listed_kernel(const PrefillParams p,
                                                                  const WorkList items) {
  __shared__ __attribute__((aligned(16))) _Float16 lds[lds_halves<D>()];
  __shared__ int32_t tab[kTabCache];
  const uint32_t it = items.item[blockIdx.y];
  prefill_dispatch<D, B>(p, blockIdx.x, (int)(it >> 16), (int)(it & 0xffffu), lds,
                         (__attribute__((address_space(3))) int32_t *)tab);
}

template <int D, int B>
hipError_t launch_db(const PrefillParams &p, int num_seqs, int max_query_len,
                     const WorkList *items, hipStream_t stream) {
  if (items) {
    if (items->count > 0)
      prefill_listed_kernel<D, B>
          <<<dim3(p.num_heads, items->count), kThreads, 0, stream>>>(p, *items);
  } else {
    const dim3 grid(p.num_heads, (max_query_len + kQTile - 1) / kQTile, num_seqs);
    prefill_kernel<D, B><<<grid, kThreads, 0, stream>>>(p);
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const PrefillParams &p, int num_seqs, int block_size, int max_query_len,
                    const WorkList *items, hipStream_t stream) {
  switch (block_size) {
    case 8: return launch_db<D, 8>(p, num_seqs, max_query_len, items, stream);
    case 16: return launch_db<D, 16>(p, num_seqs, max_query_len, items, stream);
    case 32: return launch_db<D, 32>(p, num_seqs, max_query_len, items, stream);
    case 64: return launch_db<D, 64>(p, num_seqs, max_query_len, items, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

int prefill_query_tile() { return kQTile; }

hipError_t launch_prefill(const PrefillParams &p, int num_seqs, int head_dim, int block_size,
                          int max_query_len, const WorkList *items, hipStream_t stream) {
  if (head_dim == 128) return launch_d<128>(p, num_seqs, block_size, max_query_len, items, stream);
  if (head_dim == 64) return launch_d<64>(p, num_seqs, block_size, max_query_len, items, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa
