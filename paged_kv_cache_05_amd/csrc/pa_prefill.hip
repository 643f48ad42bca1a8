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
// queries each; keys in tiles of kKeys.  Per tile, on
// v_mfma_f32_32x32x16_f16:
//   * S^T = K Q^T, one 32-key block at a time: key rows are the A operand,
//     the wave's 32 query rows the B operand (kept in registers for the
//     whole loop, multiplied once by scale * log2 e, so that scores come out
//     in log2 units).  The contraction over head_dim runs in a permuted order
//     both operands share (lane group g takes the half [g*D/2, (g+1)*D/2)).
//   * In the accumulator layout every lane holds 16 scores of one query
//     per key block, and lanes l and l ^ 32 hold the same query.  The online
//     softmax keeps a lazy reference per query: a tile's common path takes
//     the weights against it with no maximum and no lane exchange, and only
//     a weight sum that shows a weight of 2^11 or more sends the tile down a
//     path that moves the reference (a max over the two lanes) and rescales
//     the output, a per-lane multiply.
//   * O^T += V^T P^T: P^T is the B operand straight from the score
//     registers (converted to fp16, no shuffle); V^T, the A operand, comes
//     from the row-major V tile by transposing LDS reads
//     (ds_read_b64_tr_b16), in the key order the score registers imply.
// Staging: K and V tiles are double-buffered in LDS, row-major, each
// 16-byte chunk at a row-dependent XOR position, which keeps the K reads
// and the transposing V reads free of bank conflicts.  Each wave stages a
// quarter of the tile's rows.  When its rows all precede the workgroup's
// last query and their table entries lie in the pool (every tile but the
// last, normally), it loads them straight from the pools into LDS
// (global_load_lds_dwordx4: 16 bytes per lane into consecutive LDS chunks;
// the swizzle is applied by the choice of each lane's source chunk), from a
// scalar row base plus a per-lane offset fixed for the whole loop.
// Otherwise it takes a checked, synchronous fetch through registers that
// stages keys past the last query as zeros and rows of entries outside the
// pool as NaN (K) / zero (V).  The next tile's loads are in flight while
// the current tile's products run; one barrier per tile.
// Accumulation and the softmax are fp32; P is rounded to fp16 for the
// second product, and the softmax denominator sums those rounded weights
// (v_dot2 against ones, fp32 accumulation), so numerator and denominator
// use the same P.
#include <math.h>

#include <type_traits>

#include "pa_kernels.h"
#include "pa_prefill.h"

namespace pa {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef float float16v __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) half8 lds_half8;
typedef __attribute__((address_space(3))) short4v lds_short4v;

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kRows = 32;                 // queries per wave
constexpr int kQTile = kWaves * kRows;    // queries per workgroup
constexpr int kKeys = 32;                 // keys per tile
constexpr int kKeyBlocks = kKeys / 32;    // 32-key blocks per tile
constexpr float kSlack = 8.f;             // lazy-rescale slack, log2 units

template <int D>
struct Geo {
  static constexpr int kChunks = D / 8;                   // 16-byte chunks per row
  static constexpr int kRowBytes = D * 2;
  static constexpr int kTensorBytes = kKeys * kRowBytes;  // K or V of one tile
  static constexpr int kStageBytes = 2 * kTensorBytes;
  static constexpr int kWaveRows = kKeys / kWaves;        // rows each wave stages
  static constexpr int kLoadRows = 64 / kChunks;          // rows one wave-wide load covers
  static constexpr int kLoads = kWaveRows / kLoadRows;    // loads per wave per tensor
  static_assert(kLoads >= 1 && kWaveRows % kLoadRows == 0, "tile geometry");
};

// Chunk c of tile row r sits at chunk position c ^ swz(r).  K: the 16 (D =
// 128) or 8 rows that 16 lanes read at one chunk index spread over all 64
// banks.  V: the 4 rows a half-wave's transposing read covers, 4
// consecutive chunks each, land in 4 disjoint 16-bank ranges.
template <int D>
__device__ __forceinline__ int swz_k(int r) {
  return D == 128 ? (r & 15) : ((r >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int swz_v(int r) {
  return D == 128 ? ((r & 3) << 2) : (((r >> 1) & 1) << 2);
}

// Lanes l and l ^ 32 combined.  v_permlane32_swap trades the upper half of
// its first operand with the lower half of its second; applied to two
// copies of x it leaves x[l] and x[l ^ 32] in every lane, one in each
// register.  Written as inline assembly because this compiler's builtin for
// the instruction hands back the first register twice.  The s_nop gives the
// two wait states a permlane swap needs after a VALU write of its operands.
__device__ inline void swap_halves(unsigned &a, unsigned &b) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
// The maximum of x over lanes l and l ^ 32, in one block with the swap: a
// plain v_max_f32 (NaN inputs are ignored, as fmaxf does), without the
// canonicalising moves the compiler puts on values it did not produce.  The
// second s_nop covers the VALU read of the swapped registers.
__device__ inline float half_max(float x) {
  unsigned a = __builtin_bit_cast(unsigned, x), b = a;
  float r;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %1, %2\n\ts_nop 1\n\tv_max_f32 %0, %1, %2"
               : "=v"(r), "+v"(a), "+v"(b));
  return r;
}
__device__ inline float half_sum(float x) {
  unsigned a = __builtin_bit_cast(unsigned, x), b = a;
  swap_halves(a, b);
  return __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
}

// Per-lane byte offsets, fixed for the whole loop.  Only the first offset
// of each family is kept; the others differ from it in bits the swizzle
// owns alone, so one XOR with a constant gives them (no carries: the
// remaining terms are multiples of 256 bytes):
//   staging load j:   K at gk ^ (j << 6) (the rows of load j are 4 further
//                     on at D = 128, which flips bit 2 of swz_k; D = 64 has
//                     one load), V at gv (swz_v reads row bits 0..1 only);
//   K operand step j: rk ^ (j << 4) (j covers the chunk bits swz_k flips);
//   V^T block dt:     rv ^ (dt << 6) (dt covers chunk bits 2..3).
template <int D>
struct Offsets {
  uint32_t gk, gv;   // staging, inside a block
  uint32_t rk;       // K operand, head-dim step 0
  uint32_t rv;       // V^T operand, head dims 0..31
};

template <int D>
__device__ __forceinline__ uint32_t off_gk(const Offsets<D> &o, int j) {
  return o.gk ^ (uint32_t)(j << 6);
}
template <int D>
__device__ __forceinline__ uint32_t off_rk(const Offsets<D> &o, int j) {
  return o.rk ^ (uint32_t)(j << 4);
}
template <int D>
__device__ __forceinline__ uint32_t off_rv(const Offsets<D> &o, int dt) {
  return o.rv ^ (uint32_t)(dt << 6);
}

// Staging offsets are relative to the head's rows in a block; the head's
// offset is added to the (uniform) block base.
template <int D>
__device__ inline Offsets<D> make_offsets(int w, int lane) {
  using G = Geo<D>;
  static_assert(G::kLoads <= 2, "staging offsets of loads past the second");
  Offsets<D> o;
  const int pos = lane % G::kChunks, sub = lane / G::kChunks;
  const int r = w * G::kWaveRows + sub;   // tile row this lane fills in load 0
  o.gk = sub * G::kRowBytes + ((pos ^ swz_k<D>(r)) * 16);
  o.gv = sub * G::kRowBytes + ((pos ^ swz_v<D>(r)) * 16);
  // K operand: lane (c, g) reads row c (plus 32 per key block; the swizzle
  // repeats every 32 rows), chunk g D/16 + j at step j.
  const int c = lane & 31, g = lane >> 5;
  o.rk = c * G::kRowBytes + (((g * (D / 16)) ^ swz_k<D>(c)) * 16);
  // V^T operand by ds_read_b64_tr_b16: in each 16-lane group, result lane
  // i gets element i % 4 of the 4 values read by lanes i / 4, 4 + i / 4,
  // 8 + i / 4 and 12 + i / 4.  So source lane s of group grp reads key row
  // 4 (grp / 2) + s / 4 (plus the k-step's base; +8 for the operand's
  // upper four keys) at head dims 32 dt + 16 (grp % 2) + 4 (s % 4) .. +3,
  // and result lane l holds head dim 32 dt + l % 32 of keys
  // 16 kk + 8 (e / 4) + 4 (l / 32) + e % 4, the order of the score
  // registers.  Adding 16 kk or 8 rows leaves the swizzle unchanged.
  const int s = lane & 15, grp = lane >> 4;
  const int row = 4 * (grp >> 1) + (s >> 2);
  const int q = 2 * (grp & 1) + ((s & 3) >> 1);
  o.rv = row * G::kRowBytes + ((q ^ swz_v<D>(row)) * 16) + (s & 1) * 8;
  return o;
}

// The table entries of this wave's rows [w kWaveRows, (w+1) kWaveRows) of
// the tile at t0.  Uniform: scalar loads, always issued, with the index
// clamped to the table row (max_blocks_per_seq >= 1), so that no load
// depends on the sequence's lengths; stage_rows uses the entries only when
// the rows all precede kv_end.  Nothing here reads the loaded values, so the
// wait for them falls at their use in stage_rows.
template <int D, int B>
struct TileEntries {
  static constexpr int kEnt = B >= Geo<D>::kWaveRows ? 1 : Geo<D>::kWaveRows / B;
  int32_t phys[kEnt];
};

template <int D, int B>
__device__ inline TileEntries<D, B> tile_entries(const int32_t *table, int max_blocks, int w,
                                                 int t0) {
  using G = Geo<D>;
  TileEntries<D, B> e;
  const int key0 = t0 + w * G::kWaveRows;
  const auto *ctab = (const __attribute__((address_space(4))) int32_t *)table;
#pragma unroll
  for (int i = 0; i < TileEntries<D, B>::kEnt; ++i)
    e.phys[i] = ctab[min(key0 / B + i, max_blocks - 1)];
  return e;
}

// Stages this wave's rows of the tile at t0 into the stage buffer st (K,
// then V), given the rows' entries from tile_entries.  Rows whose entries
// all lie in the pool take direct loads; the others the checked fetch.
// True when the direct loads (2 kLoads of them) are still in flight on
// return; the checked fetch has written its rows before it returns.
template <int D, int B>
__device__ inline bool stage_rows(const PrefillParams &p, const int32_t *table, int h, int w,
                                  int lane, int kv_end, int t0, lds_char *st,
                                  const Offsets<D> &o, const TileEntries<D, B> &ent) {
  using G = Geo<D>;
  const int r0 = w * G::kWaveRows;
  const char *kp = static_cast<const char *>(p.k_pool);
  const char *vp = static_cast<const char *>(p.v_pool);
  const uint64_t block_bytes = (uint64_t)p.num_heads * B * D * 2;
  const uint64_t head_bytes = (uint64_t)h * B * D * 2;
  bool fast = t0 + r0 + G::kWaveRows <= kv_end;   // the entries lie in the table row
#pragma unroll
  for (int i = 0; i < TileEntries<D, B>::kEnt; ++i)
    fast = fast && ent.phys[i] >= 0 && ent.phys[i] < p.num_blocks;
  if (fast) {
#pragma unroll
    for (int j = 0; j < G::kLoads; ++j) {
      // a load's rows share one table entry: it covers kLoadRows <= B
      // aligned rows
      const int rj = r0 + j * G::kLoadRows;
      const int e = B >= G::kWaveRows ? 0 : (j * G::kLoadRows) / B;
      const uint64_t base = (uint64_t)(uint32_t)ent.phys[e] * block_bytes + head_bytes +
                            (uint64_t)((t0 + rj) % B) * G::kRowBytes;
      __builtin_amdgcn_global_load_lds(kp + base + off_gk(o, j), st + rj * G::kRowBytes, 16, 0, 0);
      __builtin_amdgcn_global_load_lds(vp + base + o.gv,
                                       st + G::kTensorBytes + rj * G::kRowBytes, 16, 0, 0);
    }
    return true;
  }
  // Checked fetch: per lane, the same row and chunk as the direct load.
  const int pos = lane % G::kChunks, sub = lane / G::kChunks;
#pragma unroll
  for (int j = 0; j < G::kLoads; ++j) {
    const int rj = r0 + j * G::kLoadRows;
    const int r = rj + sub;
    const int key = t0 + r;
    const bool in = key < kv_end;
    const int32_t ph = in ? table[key / B] : 0;
    const bool ok = in && ph >= 0 && ph < p.num_blocks;
    const uint64_t row =
        ok ? (uint64_t)(uint32_t)ph * block_bytes + head_bytes + (uint64_t)(key % B) * G::kRowBytes
           : 0;
    half8 kx = *reinterpret_cast<const half8 *>(kp + row + (pos ^ swz_k<D>(r)) * 16);
    half8 vx = *reinterpret_cast<const half8 *>(vp + row + (pos ^ swz_v<D>(r)) * 16);
    if (!ok) {
      kx = in ? half8{} + (_Float16)NAN : half8{};   // NaN for every query that sees it
      vx = half8{};
    }
    *reinterpret_cast<lds_half8 *>(st + rj * G::kRowBytes + lane * 16) = kx;
    *reinterpret_cast<lds_half8 *>(st + G::kTensorBytes + rj * G::kRowBytes + lane * 16) = vx;
  }
  return false;
}

// One work item: head h, sequence b, query tile qt.
struct Item {
  int h, b, qt;
  int q0, m, n;        // first query row, query tokens and context of the sequence
  bool empty;          // the tile holds no query of the sequence
  bool bad;            // inconsistent lengths: the tile's rows get NaN
  int kv_end;          // keys the tile needs: 0 .. kv_end - 1
  const int32_t *table;
};

__device__ __forceinline__ Item make_item(const PrefillParams &p, int h, int b, int qt) {
  Item it;
  it.h = h;
  it.b = b;
  it.qt = qt;
  // uniform across the workgroup: kept in scalar registers, so that the
  // tile loop and the branches on these lengths stay uniform
  it.q0 = __builtin_amdgcn_readfirstlane(p.query_start[b]);
  it.m = __builtin_amdgcn_readfirstlane(p.query_start[b + 1]) - it.q0;
  it.n = min(max(__builtin_amdgcn_readfirstlane(p.context_lens[b]), 0), p.max_context_len);
  it.empty = qt * kQTile >= it.m;
  it.bad = it.m < 0 || it.m > it.n || it.q0 < 0 || it.q0 + it.m > p.num_query_rows;
  const int last = min(it.m, (qt + 1) * kQTile) - 1;
  it.kv_end = (it.empty || it.bad) ? 0 : it.n - it.m + last + 1;
  it.table = p.block_tables + (int64_t)b * p.max_blocks_per_seq;
  return it;
}

// The wave's view of an item: lane c of wave w holds query r of the tile,
// at position pos = n - m + r of the sequence (only pos is kept; r follows).
struct WaveRows {
  int pos;           // per lane
  int wave_pos0;     // the wave's first query position
  bool active;       // the wave holds a query of the chunk
  int wave_last;     // the wave's last query position
};

__device__ __forceinline__ WaveRows wave_rows(const Item &it, int w, int c) {
  WaveRows v;
  v.pos = it.n - it.m + it.qt * kQTile + w * kRows + c;
  v.wave_pos0 = it.n - it.m + it.qt * kQTile + w * kRows;
  v.active = it.qt * kQTile + w * kRows < it.m && !it.bad;
  v.wave_last = it.n - it.m + min(it.m, it.qt * kQTile + (w + 1) * kRows) - 1;
  return v;
}

// The lane's query index in the sequence's chunk.
__device__ __forceinline__ int query_row(const Item &it, const WaveRows &v) {
  return v.pos - (it.n - it.m);
}

// The query tile goes through LDS: a wave's 32 query rows sit in the K
// tile's layout (chunk ch of row r at ch ^ swz_k(r)), so the wave reads its
// MFMA fragments with the K operand's offsets.  Waves 0 and 1 use the query
// buffer, waves 2 and 3 the second stage buffer, which holds nothing until
// the first step stages into it.
template <int D>
__device__ __forceinline__ lds_char *q_block(int w, lds_char *ldsq, lds_char *lds1) {
  return (w < 2 ? ldsq : lds1) + (w & 1) * kRows * Geo<D>::kRowBytes;
}

// Loads the wave's query rows straight into its block: each load covers
// kLoadRows whole rows (16 bytes per lane), where lane-per-row reads of the
// fragments would touch 64 rows per load.  Rows outside the chunk (a ragged
// tile, or an item with inconsistent lengths) read query row 0 instead:
// their columns of the products are independent of the others and their
// output rows are never stored.  (B is not used: with D alone as its
// parameter, the host pass of this compiler rejects the direct-to-LDS
// builtin once callers of several block sizes share the function.)
template <int D, int B>
__device__ __forceinline__ void stage_queries(const PrefillParams &p, const Item &it, int w, int lane,
                                        lds_char *qblk) {
  using G = Geo<D>;
  const int pos = lane % G::kChunks, sub = lane / G::kChunks;
  const int r0 = it.qt * kQTile + w * kRows;   // the wave's first query of the chunk
  const char *q = static_cast<const char *>(p.q);
#pragma unroll
  for (int i = 0; i < kRows / G::kLoadRows; ++i) {
    const int rr = i * G::kLoadRows + sub;     // row of the block this lane fills
    const bool ok = r0 + rr < it.m && !it.bad;
    const int64_t row = ok ? (int64_t)it.q0 + r0 + rr : 0;
    const char *src = q + ((row * p.num_heads + it.h) * D) * 2 + ((pos ^ swz_k<D>(rr)) * 16);
    __builtin_amdgcn_global_load_lds(src, qblk + i * G::kLoadRows * G::kRowBytes, 16, 0, 0);
  }
}

// A lane's online-softmax state for its query.  Scores are in log2 units
// (the query fragments carry scale * log2 e).  m is the reference the
// weights are taken against (-inf until the query has seen a key), m_use the
// same but 0 while m is -inf (so that weights of masked keys come out 0,
// never NaN), thr the score above which the reference moves, m + kSlack,
// and l this lane's partial denominator.
struct SoftmaxState {
  float m = -INFINITY, m_use = 0.f, thr = -INFINITY, l = 0.f;
};

// S^T = K Q^T for one staged tile (keys t0 .. t0 + 31), masked: slot i of
// key block kb holds key t0 + 32 kb + 8 (i / 4) + 4 g + i % 4, set to -inf
// when that key lies past the lane's query position, i.e. when its constant
// part 32 kb + 8 (i / 4) + i % 4 exceeds pos - t0 - 4 g.  Tiles wholly at or
// below every query of the wave skip the mask.
template <int D>
__device__ __forceinline__ void tile_scores(const lds_char *ks, const Offsets<D> &o,
                                            const half8 (&qb)[D / 16], float16v (&s)[kKeyBlocks],
                                            int t0, const WaveRows &v, int g) {
  using G = Geo<D>;
  constexpr int kSteps = D / 16;
#pragma unroll
  for (int kb = 0; kb < kKeyBlocks; ++kb) {
    s[kb] = float16v{};
#pragma unroll
    for (int j = 0; j < kSteps; ++j) {
      const half8 a =
          *reinterpret_cast<const lds_half8 *>(ks + off_rk(o, j) + kb * 32 * G::kRowBytes);
      s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, qb[j], s[kb], 0, 0, 0);
    }
  }
  // Schedule: the K operand reads run kAhead steps ahead of the score
  // MFMAs (LDS reads, then one MFMA and one read per step), so that the
  // reads of later steps return under the earlier MFMAs instead of each
  // pair waiting for its own.  Four steps ahead at D = 128 (168 VGPRs, the
  // whole three-waves-per-SIMD budget, no scratch) and three at D = 64,
  // where four (every read at once) measured slower.
  constexpr int kAhead = kSteps >= 8 ? 4 : (kSteps < 3 ? kSteps : 3);
  __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);   // LDS reads
#pragma unroll
  for (int j = 0; j < kSteps - kAhead; ++j) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);      // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, kAhead, 0);
  if (t0 + kKeys - 1 > v.wave_pos0) {
    const int lim = v.pos - t0 - 4 * g;
#pragma unroll
    for (int kb = 0; kb < kKeyBlocks; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (32 * kb + (i / 4) * 8 + (i % 4) > lim) s[kb][i] = -INFINITY;
  }
}

// The lazy step of the online softmax: a query whose tile maximum exceeds
// its reference by more than kSlack takes that maximum as its new
// reference, and its output and denominator are rescaled.  Lanes l and
// l ^ 32 hold the same query and combine their maxima, so both take the
// same step.  kFirst (the wave's first tile of its key range, where every
// query that sees a key of the range sees one): the reference is set, to 0
// when the tile's maximum lies in [kRefLo, kRefHi] (then the largest weight
// is between 2^-8 and 2^11, inside fp16 with full precision, and the common
// path needs no subtraction), else to the maximum.
constexpr float kRefLo = -8.f, kRefHi = 11.f;
template <int D, bool kFirst>
__device__ __forceinline__ void rebase(const float16v (&s)[kKeyBlocks], float16v (&acc_o)[D / 32],
                                       SoftmaxState &sm) {
  float tile_max = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < kKeyBlocks; ++kb)
#pragma unroll
    for (int i = 0; i < 16; ++i) tile_max = fmaxf(tile_max, s[kb][i]);
  tile_max = half_max(tile_max);
  const bool bump = tile_max > sm.thr;
  if (__ballot(bump)) {
    float m_new = tile_max;
    if constexpr (kFirst) m_new = (tile_max >= kRefLo && tile_max <= kRefHi) ? 0.f : tile_max;
    const float alpha = bump ? __builtin_amdgcn_exp2f(sm.m - m_new) : 1.f;
    sm.l *= alpha;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) acc_o[dt] *= alpha;
    if (bump) {
      sm.m = m_new;
      sm.m_use = m_new;
      sm.thr = m_new + kSlack;
    }
  }
}

// Weights 2^(s - m_use) rounded to fp16 (round to nearest even) two at a
// time (kZeroRef: m_use is 0 for every lane, and the subtraction is left
// out; the weights are the same), and their sum over this lane's 16 keys (v_dot2
// against ones, fp32), which is what the denominator adds: numerator and
// denominator use the same rounded weights.  The pair conversion is written
// as plain C, which compiles to one v_cvt_pk_f16_f32: the compiler then
// also puts in the wait state that gfx950 needs between a transcendental
// result (v_exp_f32) and a VALU read of it.  Inline assembly would hide
// that read from it, and a schedule that placed the conversion right after
// its exponential would read the exponential's input.
template <bool kZeroRef>
__device__ __forceinline__ float tile_weights(const float16v (&s)[kKeyBlocks], float m_use,
                                              unsigned (&pw)[kKeyBlocks][8]) {
#pragma unroll
  for (int kb = 0; kb < kKeyBlocks; ++kb)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float e0 = __builtin_amdgcn_exp2f(kZeroRef ? s[kb][2 * i] : s[kb][2 * i] - m_use);
      const float e1 =
          __builtin_amdgcn_exp2f(kZeroRef ? s[kb][2 * i + 1] : s[kb][2 * i + 1] - m_use);
      const half2v h = {(_Float16)e0, (_Float16)e1};
      pw[kb][i] = __builtin_bit_cast(unsigned, h);
    }
  float psum = 0.f;
  const half2v one = {(_Float16)1.f, (_Float16)1.f};
#pragma unroll
  for (int kb = 0; kb < kKeyBlocks; ++kb)
#pragma unroll
    for (int i = 0; i < 8; ++i)
      psum = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2v, pw[kb][i]), one, psum, false);
  return psum;
}

// A lane's weight sum at or above this means one of its 16 weights is at
// least 2^11 (or rounded to inf in fp16): the reference has to move.
constexpr float kOverflowSum = 32768.f;

// The wave's products on one staged tile (keys t0 .. t0 + 31): scores, the
// online softmax update and the output accumulation.  kFirst: the wave's
// first tile of its key range.
template <int D, bool kFirst>
__device__ __forceinline__ void tile_products(const PrefillParams &p, const lds_char *ks,
                                              const Offsets<D> &o, const half8 (&qb)[D / 16],
                                              float16v (&acc_o)[D / 32], SoftmaxState &sm,
                                              int t0, const WaveRows &v, int g) {
  using G = Geo<D>;
  const lds_char *vs = ks + G::kTensorBytes;
  float16v s[kKeyBlocks];
  tile_scores<D>(ks, o, qb, s, t0, v, g);
  // The reference moves lazily (rebase).  On the wave's first tile it is
  // set from the tile's maximum (to 0 when that maximum is in [-8, 11]): a
  // query's visible keys are a prefix of the sequence, so a query that sees
  // any key of the range sees one in its first tile, and the largest weight
  // it has seen is never below 2^-8 from then on.  On later tiles the test runs on the weights, not on a
  // maximum: the common path takes the weights against the current
  // reference, and only when some lane's weight sum shows a weight of 2^11
  // or more (or one beyond fp16, 2^16) are the scores taken again (they are
  // not kept: registers), the reference moved and the weights redone.
  // Weights stay below 2^16, inside fp16 and fp32; numerator and
  // denominator share the reference, so the result is the same softmax.  A
  // NaN score gives a NaN sum, which stays on the common path and reaches
  // the row, as it should.
  if constexpr (kFirst) rebase<D, true>(s, acc_o, sm);
  unsigned pw[kKeyBlocks][8];
  float psum = __ballot(sm.m_use != 0.f) ? tile_weights<false>(s, sm.m_use, pw)
                                         : tile_weights<true>(s, 0.f, pw);
  if (!kFirst && __ballot(psum >= kOverflowSum)) {
    // The clobber makes the scores' LDS reads happen again here: reusing the
    // first reads would keep their 32 registers live across the weights.
    asm volatile("" ::: "memory");
    tile_scores<D>(ks, o, qb, s, t0, v, g);
    rebase<D, false>(s, acc_o, sm);
    psum = tile_weights<false>(s, sm.m_use, pw);
  }
  // Each lane sums its own 16 keys of the tile; lanes l and l ^ 32 hold the
  // same query with the same reference and scale factors, so their sums are
  // added once, after the loop.
  sm.l += psum;
  half8 pb[kKeyBlocks][2];
#pragma unroll
  for (int kb = 0; kb < kKeyBlocks; ++kb)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
      pb[kb][j] = __builtin_bit_cast(
          half8, u32x4{pw[kb][4 * j], pw[kb][4 * j + 1], pw[kb][4 * j + 2], pw[kb][4 * j + 3]});
    }

  // O^T += V^T P^T.  k-step kk covers keys 16 kk .. 16 kk + 15 in the
  // order the score registers hold them: slots 0..3 -> keys
  // 16 kk + 4 g + e, slots 4..7 -> keys 16 kk + 8 + 4 g + (e - 4).
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
    for (int kk = 0; kk < kKeys / 16; ++kk) {
      const lds_char *vrow = vs + off_rv(o, dt) + 16 * kk * G::kRowBytes;
      const short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v *)vrow);
      const short4v hi =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v *)(vrow + 8 * G::kRowBytes));
      const half8 a = __builtin_bit_cast(
          half8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      acc_o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pb[kk / 2][kk % 2], acc_o[dt], 0, 0, 0);
    }
  }
  // Schedule: the Vᵀ reads of two 32-dim blocks first, then each block's
  // two MFMAs followed by the reads of the block two ahead.
  __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);        // LDS reads
#pragma unroll
  for (int dt = 0; dt < D / 32 - 2; ++dt) {
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);      // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
}

// The tile's output rows (rows in range only).  Lane (c, g) holds O^T[d][c]
// for d = 32 dt + 8 (i / 4) + 4 g + (i % 4): 8-byte pieces of 32 rows.  The
// wave normalises them, writes them to its own 32 rows of the (now idle)
// stage buffers, row-major with 16-byte chunk ch of row r at ch ^ (r mod
// kChunks) (so the writes of a chunk index by 32 rows spread over the
// banks, and the reads of whole rows hit each bank once), and reads them
// back as whole rows: each global store then writes 64 / kChunks complete
// rows (16 bytes per lane) instead of 8 bytes in each of 32 rows.
template <int D>
__device__ __forceinline__ void store_rows(const PrefillParams &p, const Item &it, int w,
                                           const float16v (&acc_o)[D / 32], float l_run,
                                           lds_char *lds0, lds_char *lds1) {
  using G = Geo<D>;
  constexpr int kC = G::kChunks;
  static_assert(2 * kRows * G::kRowBytes == G::kStageBytes, "two waves' rows per stage buffer");
  lds_char *wb = (w < 2 ? lds0 : lds1) + (w & 1) * kRows * G::kRowBytes;
  // The lane index is taken afresh (mbcnt) rather than from the value the
  // loop's offsets were built from: reusing those would keep one more
  // register live across the whole tile loop.
  const int lane_now = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  const int c = lane_now & 31, g = lane_now >> 5;
  const float inv = (it.bad || !(l_run > 0.f)) ? NAN : 1.f / l_run;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      half4 o4;
#pragma unroll
      for (int e = 0; e < 4; ++e) o4[e] = (_Float16)(acc_o[dt][i4 * 4 + e] * inv);
      const int pos = (4 * dt + i4) ^ (c % kC);
      *reinterpret_cast<__attribute__((address_space(3))) half4 *>(wb + c * G::kRowBytes +
                                                                   pos * 16 + 8 * g) = o4;
    }
  // This wave reads back only what it wrote itself; the wait and the
  // clobber keep the reads behind the writes.
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  constexpr int kRowsPerStore = 64 / kC;
  const int sub = lane_now / kC, ch = lane_now % kC;
  const int r0 = it.qt * kQTile + w * kRows;   // the wave's first query row
#pragma unroll
  for (int k = 0; k < kRows / kRowsPerStore; ++k) {
    const int row = k * kRowsPerStore + sub;
    const half8 x =
        *reinterpret_cast<const lds_half8 *>(wb + row * G::kRowBytes + ((ch ^ (row % kC)) * 16));
    const int r = r0 + row;
    if (r < it.m && it.q0 + r < p.num_query_rows && it.q0 + r >= 0)
      *reinterpret_cast<half8 *>(static_cast<_Float16 *>(p.out) +
                                 ((int64_t)(it.q0 + r) * p.num_heads + it.h) * D + ch * 8) = x;
  }
}

// With nchunks > 1 the workgroup covers key chunk `chunk` of the tile's
// keys (an equal share of its 32-key tiles) and writes that chunk's partial
// result to slot `slot` for the merge pass.
template <int D, int B>
__device__ void prefill_item(const PrefillParams &p, int h, int b, int qt, lds_char *lds0,
                             lds_char *lds1, lds_char *ldsq, int chunk = 0, int nchunks = 1,
                             int slot = 0) {
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // The entries of keys 0..31 (the first tile of every range that starts at
  // key 0) are loaded beside the sequence's lengths, not after them.
  const TileEntries<D, B> ent0 =
      tile_entries<D, B>(p.block_tables + (int64_t)b * p.max_blocks_per_seq,
                         p.max_blocks_per_seq, w, 0);
  const Item it = make_item(p, h, b, qt);
  // An empty use keeps the entries' loads here, in flight with the lengths'
  // loads and waited for with them, instead of sunk to their use.
#pragma unroll
  for (int i = 0; i < TileEntries<D, B>::kEnt; ++i) asm volatile("" ::"s"(ent0.phys[i]));
  // The same for the pointers the staging needs (kernel arguments).
  asm volatile("" ::"s"(p.q), "s"(p.k_pool), "s"(p.v_pool));
  if (it.empty) return;
  const int lane = threadIdx.x & 63;
  const int c = lane & 31;                 // this lane's query column / key row
  const int g = lane >> 5;                 // lane group
  // The wave's products are skipped when it holds no query of the chunk,
  // and for key tiles past its last query (it still stages its rows and
  // meets every barrier).
  const WaveRows v = wave_rows(it, w, c);
  const Offsets<D> o = make_offsets<D>(w, lane);

  lds_char *qblk = q_block<D>(w, ldsq, lds1);
  stage_queries<D, B>(p, it, w, lane, qblk);
  float16v acc_o[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t) acc_o[t] = float16v{};
  SoftmaxState sm;

  // This workgroup's keys [k_lo, k_hi): all of them, or one chunk.
  const int ntiles = (it.kv_end + kKeys - 1) / kKeys;
  const int k_lo = (int)((int64_t)ntiles * chunk / nchunks) * kKeys;
  const int k_hi = min(it.kv_end, (int)((int64_t)ntiles * (chunk + 1) / nchunks) * kKeys);
  bool tile0_in_flight = false;
  if (k_lo < k_hi)
    tile0_in_flight = stage_rows<D, B>(p, it.table, h, w, lane, it.kv_end, k_lo, lds0, o,
                     k_lo == 0 ? ent0
                               : tile_entries<D, B>(it.table, p.max_blocks_per_seq, w, k_lo));
  // The next tile's entries are loaded one step ahead, so that their wait
  // falls under the product's LDS waits instead of before the staging.
  TileEntries<D, B> ent = tile_entries<D, B>(it.table, p.max_blocks_per_seq, w, k_lo + kKeys);
  // This wave's query rows are in LDS once no more than the first tile's
  // direct loads are in flight (loads retire in order); the query scaling
  // then runs under those.  vmcnt in bits 3:0; expcnt 6:4 and lgkmcnt 11:8
  // at their maxima (no wait).
  if (tile0_in_flight)
    __builtin_amdgcn_s_waitcnt(0xf70 | (2 * Geo<D>::kLoads));
  else
    __builtin_amdgcn_s_waitcnt(0xf70);
  // The wave reads only the query rows it loaded itself, so its own wait
  // covers them; the barrier (whose fences wait for the first tile) then
  // also keeps every wave's first staging into the second buffer behind
  // waves 2 and 3 reading their rows there.
  half8 qb[D / 16];
#pragma unroll
  for (int j = 0; j < D / 16; ++j) qb[j] = *reinterpret_cast<const lds_half8 *>(qblk + off_rk(o, j));
  // Scores in log2 units: each query element times scale * log2 e, in fp32,
  // rounded to fp16 once (a relative error of at most 2^-11 per element).
#pragma unroll
  for (int j = 0; j < D / 16; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) qb[j][e] = (_Float16)((float)qb[j][e] * p.scale_log2);
  __syncthreads();

  // One tile: stage the next one into the other buffer, run the products on
  // this one, then wait for this wave's loads and meet the others.  The two
  // buffers alternate by template argument, so every LDS offset is an
  // immediate.  The first tile of the range is peeled off the loop: it sets
  // each query's softmax reference (tile_products<D, true>).
  auto step = [&](auto stage, auto first, int t0) {
    constexpr int kS = decltype(stage)::value;
    lds_char *cur = kS ? lds1 : lds0;
    if (t0 + kKeys < k_hi)
      stage_rows<D, B>(p, it.table, h, w, lane, it.kv_end, t0 + kKeys, kS ? lds0 : lds1, o, ent);
    ent = tile_entries<D, B>(it.table, p.max_blocks_per_seq, w, t0 + 2 * kKeys);
    if (v.active && t0 <= v.wave_last)
      tile_products<D, decltype(first)::value>(p, cur, o, qb, acc_o, sm, t0, v, g);
    __builtin_amdgcn_s_waitcnt(0);   // this wave's direct loads have reached LDS
    __syncthreads();
  };
  if (k_lo < k_hi) step(std::integral_constant<int, 0>{}, std::true_type{}, k_lo);
  for (int t0 = k_lo + kKeys; t0 < k_hi; t0 += 2 * kKeys) {
    step(std::integral_constant<int, 1>{}, std::false_type{}, t0);
    if (t0 + kKeys >= k_hi) break;
    step(std::integral_constant<int, 0>{}, std::false_type{}, t0 + kKeys);
  }
  const float l_run = half_sum(sm.l);   // the two lanes' partial denominators

  if (nchunks > 1) {
    const int r = query_row(it, v);
    if (r >= it.m || it.q0 + r >= p.num_query_rows || it.q0 + r < 0) return;
    // Partial result: the unnormalised output and (m, l) of this chunk,
    // for the merge pass; an empty chunk leaves m = -inf, l = 0, O = 0.
    const size_t prow = ((size_t)slot * p.num_heads + h) * kQTile + w * kRows + c;
    float *po = p.part_o + prow * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4)
        *reinterpret_cast<float4 *>(po + dt * 32 + i4 * 8 + g * 4) =
            make_float4(acc_o[dt][i4 * 4], acc_o[dt][i4 * 4 + 1], acc_o[dt][i4 * 4 + 2],
                        acc_o[dt][i4 * 4 + 3]);
    if (g == 0) p.part_ml[prow] = make_float2(sm.m, l_run);
    return;
  }
  store_rows<D>(p, it, w, acc_o, l_run, lds0, lds1);
}

// Waves per SIMD the register budget is set for (168 VGPRs).  Two stages of
// 32-key tiles take 32 KB of LDS at D = 128.  64-key tiles (two waves per
// SIMD) measured 5-12% slower.
template <int D>
constexpr int waves_per_eu() {
  return 3;
}

// grid (heads, query tiles, sequences); tiles in descending order.
template <int D, int B>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(waves_per_eu<D>())))
prefill_kernel(const PrefillParams p) {
  __shared__ __attribute__((aligned(1024))) char lds0[Geo<D>::kStageBytes];
  __shared__ __attribute__((aligned(1024))) char lds1[Geo<D>::kStageBytes];
  __shared__ __attribute__((aligned(1024))) char ldsq[Geo<D>::kStageBytes];
  prefill_item<D, B>(p, blockIdx.x, blockIdx.z, (int)gridDim.y - 1 - (int)blockIdx.y,
                     (lds_char *)lds0, (lds_char *)lds1, (lds_char *)ldsq);
}

// grid (heads, items): items = sequence << 16 | query tile, in the order the
// host planned.
template <int D, int B>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(waves_per_eu<D>())))
prefill_listed_kernel(const PrefillParams p, const WorkList items) {
  __shared__ __attribute__((aligned(1024))) char lds0[Geo<D>::kStageBytes];
  __shared__ __attribute__((aligned(1024))) char lds1[Geo<D>::kStageBytes];
  __shared__ __attribute__((aligned(1024))) char ldsq[Geo<D>::kStageBytes];
  const uint32_t it = items.item[blockIdx.y];
  prefill_item<D, B>(p, blockIdx.x, (int)(it >> 16), (int)(it & 0xffffu), (lds_char *)lds0,
                     (lds_char *)lds1, (lds_char *)ldsq);
}

// grid (heads, split list entries): one key chunk of one query tile each.
template <int D, int B>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(waves_per_eu<D>())))
prefill_split_kernel(const PrefillParams p, const SplitList items) {
  __shared__ __attribute__((aligned(1024))) char lds0[Geo<D>::kStageBytes];
  __shared__ __attribute__((aligned(1024))) char lds1[Geo<D>::kStageBytes];
  __shared__ __attribute__((aligned(1024))) char ldsq[Geo<D>::kStageBytes];
  const uint32_t it = items.item[blockIdx.y], part = items.part[blockIdx.y];
  prefill_item<D, B>(p, blockIdx.x, (int)(it >> 16), (int)(it & 0xffffu), (lds_char *)lds0,
                     (lds_char *)lds1, (lds_char *)ldsq, (int)((part >> 4) & 15u),
                     (int)(part & 15u) + 1, (int)(part >> 8));
}

// Merge of a split tile's chunks: grid (heads, split tiles, row groups),
// 256 threads.  D / 4 lanes cover one query row with 16-byte loads, so a
// wave reads whole rows per instruction and each workgroup takes 256 / (D /
// 4) rows.  Every chunk's state and partial row are loaded before any
// arithmetic (one memory round trip per workgroup), then combined by the
// usual rescaling: with M the largest running max,
//   out = sum_c 2^(m_c - M) O_c / sum_c 2^(m_c - M) l_c.
// Rows and invalid sequences follow the unsplit epilogue.
constexpr int kMergeThreads = 256;
template <int D>
constexpr int merge_rows() {
  return kMergeThreads / (D / 4);
}
template <int D>
__global__ void __launch_bounds__(kMergeThreads) prefill_merge_kernel(const PrefillParams p,
                                                                       const SplitList merges) {
  constexpr int kLanesPerRow = D / 4;
  static_assert(kQTile % merge_rows<D>() == 0, "row groups");
  const int h = blockIdx.x;
  const uint32_t it = merges.item[blockIdx.y], part = merges.part[blockIdx.y];
  const int b = (int)(it >> 16), qt = (int)(it & 0xffffu);
  const int slot0 = (int)(part >> 8), nc = (int)(part & 15u) + 1;
  const int q0 = p.query_start[b];
  const int m = p.query_start[b + 1] - q0;
  const int n = min(max(p.context_lens[b], 0), p.max_context_len);
  const bool bad_seq = m < 0 || m > n || q0 < 0 || q0 + m > p.num_query_rows;
  const int d = (threadIdx.x % kLanesPerRow) * 4;
  const int row = blockIdx.z * merge_rows<D>() + threadIdx.x / kLanesPerRow;
  const int r = qt * kQTile + row;
  if (r >= m || q0 + r >= p.num_query_rows || q0 + r < 0) return;
  float2 ml[kMaxChunks];
  float4 v[kMaxChunks];
#pragma unroll
  for (int i = 0; i < kMaxChunks; ++i) {
    if (i < nc) {
      const size_t prow = ((size_t)(slot0 + i) * p.num_heads + h) * kQTile + row;
      ml[i] = p.part_ml[prow];
      v[i] = *reinterpret_cast<const float4 *>(p.part_o + prow * D + d);
    }
  }
  float M = -INFINITY;
#pragma unroll
  for (int i = 0; i < kMaxChunks; ++i)
    if (i < nc) M = fmaxf(M, ml[i].x);
  float L = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int i = 0; i < kMaxChunks; ++i) {
    if (i < nc) {
      const float wgt = ml[i].x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ml[i].x - M);
      L += wgt * ml[i].y;
      acc.x += wgt * v[i].x;
      acc.y += wgt * v[i].y;
      acc.z += wgt * v[i].z;
      acc.w += wgt * v[i].w;
    }
  }
  const float inv = (bad_seq || !(L > 0.f)) ? NAN : 1.f / L;
  half4 o4;
  o4[0] = (_Float16)(acc.x * inv);
  o4[1] = (_Float16)(acc.y * inv);
  o4[2] = (_Float16)(acc.z * inv);
  o4[3] = (_Float16)(acc.w * inv);
  *reinterpret_cast<half4 *>(static_cast<_Float16 *>(p.out) +
                             ((int64_t)(q0 + r) * p.num_heads + h) * D + d) = o4;
}

template <int D, int B>
hipError_t launch_db(const PrefillParams &p, int num_seqs, int max_query_len,
                     const WorkList *items, const SplitList *split, const SplitList *merges,
                     hipStream_t stream) {
  if (split) {
    if (split->count > 0)
      prefill_split_kernel<D, B>
          <<<dim3(p.num_heads, split->count), kThreads, 0, stream>>>(p, *split);
    if (merges && merges->count > 0)
      prefill_merge_kernel<D><<<dim3(p.num_heads, merges->count, kQTile / merge_rows<D>()),
                                kMergeThreads, 0, stream>>>(p, *merges);
    return hipGetLastError();
  }
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
                    const WorkList *items, const SplitList *split, const SplitList *merges,
                    hipStream_t stream) {
  switch (block_size) {
    case 8: return launch_db<D, 8>(p, num_seqs, max_query_len, items, split, merges, stream);
    case 16: return launch_db<D, 16>(p, num_seqs, max_query_len, items, split, merges, stream);
    case 32: return launch_db<D, 32>(p, num_seqs, max_query_len, items, split, merges, stream);
    case 64: return launch_db<D, 64>(p, num_seqs, max_query_len, items, split, merges, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

int prefill_query_tile() { return kQTile; }
int prefill_key_tile() { return kKeys; }

size_t prefill_slot_bytes(int num_heads, int head_dim) {
  return (size_t)num_heads * kQTile * ((size_t)head_dim * sizeof(float) + sizeof(float2));
}

// 168 VGPRs per wave: three waves per SIMD, so three 4-wave workgroups per
// CU (their 32 KB of LDS each fits as well).
int prefill_groups_per_cu() { return 3; }

hipError_t launch_prefill(const PrefillParams &p, int num_seqs, int head_dim, int block_size,
                          int max_query_len, const WorkList *items, const SplitList *split,
                          const SplitList *merges, hipStream_t stream) {
  if (head_dim == 128)
    return launch_d<128>(p, num_seqs, block_size, max_query_len, items, split, merges, stream);
  if (head_dim == 64)
    return launch_d<64>(p, num_seqs, block_size, max_query_len, items, split, merges, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa
