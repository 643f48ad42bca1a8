// Paged single-query decode attention for gfx950 (CDNA 4).
//
// Computes, for every (sequence b, head h), attention of the one query token
// over the sequence's cached keys and values, which sit in fixed-size blocks
// scattered through two pools (K and V) and are found through the
// sequence's block table: the block-wise form of attention in the
// zhaifeiyue.github.io summary of Kwon et al. (PagedAttention), "method"
// paragraph, equation for A_ij and o_i, completed "by a final reduction" as
// ricepunchb.github.io section 3.3 puts it.
//
// Design (MI355X: wave64, 16-byte vector loads, DPP, HBM-bound):
//  * One workgroup of W waves per (head, sequence, context partition).  A
//    partition is `partition_size` tokens; each wave takes every W-th
//    16-token tile of it.
//  * A token row of K or V (head_dim elements) is read as 16-byte chunks by
//    a group of lanes: at fp16/head_dim 128 one row is 256 bytes = 16 lanes,
//    so one wave load covers 4 consecutive tokens and a 16-token tile is 4
//    loads of K and 4 of V, each 1 KiB contiguous inside one block.
//  * The physical block of a tile comes from one load of the block table
//    entry (block index = token / B, offset = token % B): a scalar load for
//    tiles fetched while another is in flight (its wait leaves their loads
//    in flight), a vector load for a wave's first and ragged tiles, which
//    have nothing else in flight.  Translation costs one load per tile.
//  * With a fused append the new token is read from its input rows, and
//    extra writer workgroups in the same launch store those rows at their
//    slots; no workgroup of the launch reads them there.
//  * q.k per token: v_dot2 (fp16 pairs into fp32) on the lane's chunk, then a
//    DPP row reduction over the lanes of the token (quad_perm, half-mirror,
//    mirror).  Every lane of the row ends up holding the token's score.
//  * Online softmax in base 2 (scale * log2 e folded into one multiply).
//    Each lane row keeps its own running max / sum / accumulator for the
//    tokens it sees (tokens congruent to it modulo the row count), so the hot
//    loop has no cross-row traffic.  At the end the rows of a wave are folded
//    by a lane butterfly and the waves merged through LDS, both with the
//    usual max/sum rescaling.
//  * Masking of the ragged last tile is a select on scores and values, never
//    a multiply by zero, so whatever sits in unused slots (NaN included)
//    cannot reach the result.
//  * A row whose context fits one partition is finished in the first pass.
//    Longer rows are split across workgroups; each writes (max, sum,
//    unnormalised output) to the workspace and a second, small kernel merges
//    them with max/sum rescaling.  (Merging inside the first kernel would
//    need device-scope release/acquire fences, which on this multi-L2 part
//    write back and invalidate the L2 per workgroup.)
//  * No MFMA: one query row per (sequence, head) makes q.K and p.V
//    matrix-vector products, about one flop per byte moved.
#include <math.h>

#include <type_traits>

#include "pa_kernels.h"

namespace pa {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
// Integers in the constant address space (read-only for the kernel's life).
typedef const __attribute__((address_space(4))) int32_t ConstI32;
typedef const __attribute__((address_space(4))) int64_t ConstI64;

// 16-byte chunks each writer thread of a fused append copies (its loads are
// issued together, then its stores).
constexpr int kWriterChunks = 4;

union Chunk {  // one 16-byte vector load
  uint4 u;
  uint32_t w[4];
};

template <typename T, int D>
struct Geometry {
  static constexpr int kElemBytes = sizeof(T);
  static constexpr int kPerChunk = 16 / kElemBytes;     // elements per 16-byte chunk
  static constexpr int kChunksPerRow = D / kPerChunk;   // chunks per token row
  static constexpr int kLanesPerToken = kChunksPerRow < 16 ? kChunksPerRow : 16;
  static constexpr int kChunksPerLane = kChunksPerRow / kLanesPerToken;
  static constexpr int kTokensPerGroup = 64 / kLanesPerToken;  // tokens per wave load
  static constexpr int kTile = 16;                              // tokens per wave step
  static constexpr int kGroups = kTile / kTokensPerGroup;
  static constexpr int kAcc = kChunksPerLane * kPerChunk;     // output elements per lane
  static_assert(kLanesPerToken == 8 || kLanesPerToken == 16, "row reduction covers 8 or 16 lanes");
};

template <int kCtrl>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), kCtrl,
                                                            0xF, 0xF, true));
}

// Sum over each aligned group of kLanes (8 or 16) lanes; every lane of the
// group receives the total.
template <int kLanes>
__device__ __forceinline__ float row_sum(float v) {
  v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]: pairs
  v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]: quads
  v += dpp<0x141>(v);  // row_half_mirror: eights
  if constexpr (kLanes == 16) v += dpp<0x140>(v);  // row_mirror: sixteens
  return v;
}

__device__ __forceinline__ Chunk load_chunk(const char *p) {
  Chunk c;
  c.u = *reinterpret_cast<const uint4 *>(p);
  return c;
}

// K/V rows that only one workgroup reads are streamed with non-temporal
// loads, which keep them from displacing reusable lines (block tables, q,
// shared blocks) in the caches.
__device__ __forceinline__ Chunk load_stream(const char *p) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
  Chunk c;
  c.w[0] = x.x;
  c.w[1] = x.y;
  c.w[2] = x.z;
  c.w[3] = x.w;
  return c;
}

// K/V load of one 16-byte chunk: streamed (non-temporal), or with the
// default policy that keeps the line in the caches for another reader.
template <bool kKeep>
__device__ __forceinline__ Chunk load_kv(const char *p) {
  if constexpr (kKeep) return load_chunk(p);
  else return load_stream(p);
}

__device__ __forceinline__ float dot_chunk(const Chunk &q, const Chunk &k, float acc, _Float16) {
#pragma unroll
  for (int j = 0; j < 4; ++j)
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, q.w[j]),
                                 __builtin_bit_cast(half2_t, k.w[j]), acc, false);
  return acc;
}

__device__ __forceinline__ float dot_chunk(const Chunk &q, const Chunk &k, float acc, float) {
#pragma unroll
  for (int j = 0; j < 4; ++j)
    acc = __builtin_fmaf(__builtin_bit_cast(float, q.w[j]), __builtin_bit_cast(float, k.w[j]), acc);
  return acc;
}

__device__ __forceinline__ void axpy_chunk(float *acc, float p, const Chunk &v, _Float16) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const half2_t h = __builtin_bit_cast(half2_t, v.w[j]);
    acc[2 * j] = __builtin_fmaf(p, (float)h.x, acc[2 * j]);
    acc[2 * j + 1] = __builtin_fmaf(p, (float)h.y, acc[2 * j + 1]);
  }
}

__device__ __forceinline__ void axpy_chunk(float *acc, float p, const Chunk &v, float) {
#pragma unroll
  for (int j = 0; j < 4; ++j)
    acc[j] = __builtin_fmaf(p, __builtin_bit_cast(float, v.w[j]), acc[j]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <typename T, int D>
struct Tile {
  using G = Geometry<T, D>;
  Chunk k[G::kGroups][G::kChunksPerLane];
  Chunk v[G::kGroups][G::kChunksPerLane];
};

// Per-lane-row softmax state.
template <int kAcc>
struct RowState {
  float m, l;
  float acc[kAcc];
};

// LDS of one workgroup: one softmax state per wave, merged at the end.
template <typename T, int D, int W>
struct ItemShared {
  static constexpr int kStates = W;
  float m[kStates];
  float l[kStates];
  float o[kStates][D];
};

// Table entries of a wave's first 16-token tile (one per block the tile
// spans), loaded before the context length is known.
template <int B>
struct FirstEntries {
  static constexpr int kCount = B >= 16 ? 1 : 16 / B;
  int32_t e[kCount];
};

// This lane's chunk(s) of the query row (b, h).
template <typename T, int D>
__device__ __forceinline__ void load_q(const DecodeParams &p, int b, int h,
                                       Chunk (&qc)[Geometry<T, D>::kChunksPerLane]) {
  using G = Geometry<T, D>;
  const int col = (threadIdx.x & 63) % G::kLanesPerToken;
  const char *qp =
      reinterpret_cast<const char *>(p.q) + ((size_t)b * p.num_heads + h) * D * sizeof(T);
#pragma unroll
  for (int k = 0; k < G::kChunksPerLane; ++k)
    qc[k] = load_chunk(qp + (col + k * G::kLanesPerToken) * 16);
}

// One work item: sequence b, head h, context partition `part` (tokens
// [part * P, min(ctx, (part + 1) * P)), non-empty), ctx already clamped.
// Called by every thread of the workgroup (it synchronises inside).  Writes
// the output row when the row has a single partition, else this partition's
// (max, sum, unnormalised output) for the merge pass.
template <typename T, int D, int B, int W, bool kKeep>
__device__ __forceinline__ void process_item(const DecodeParams &p, ItemShared<T, D, W> &sh,
                                             int b, int h, int part, int ctx, bool append,
                                             const FirstEntries<B> &first,
                                             const Chunk (&qc)[Geometry<T, D>::kChunksPerLane]) {
  using G = Geometry<T, D>;
  constexpr int kStates = ItemShared<T, D, W>::kStates;
  constexpr int kLPT = G::kLanesPerToken;
  constexpr int kTPG = G::kTokensPerGroup;
  const int H = p.num_heads;
  const size_t row = (size_t)b * H + h;
  T *out_row = reinterpret_cast<T *>(p.out) + row * D;
  const int P = p.partition_size;
  const int tok0 = part * P;
  const int tok_end = min(ctx, tok0 + P);
  const int n_parts = (ctx + P - 1) / P;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane % kLPT;   // which 16-byte chunk(s) of a token row
  const int trow = lane / kLPT;  // which token of a 4- or 8-token group


  // Two views of the sequence's table row.  Inside the tile loop entries are
  // read through the constant address space: the kernel never writes the
  // tables, and a constant load at a wave-uniform address becomes a scalar
  // load whose wait (lgkmcnt) leaves the prefetched K/V loads in flight,
  // where a vector load would need vmcnt(0), which retires in order.  A
  // wave's first tile and the ragged tile have nothing else in flight, and
  // there the vector path's shorter latency wins.
  const int32_t *table = p.block_tables + (size_t)b * p.max_blocks_per_seq;
  const ConstI32 *table_s = (const ConstI32 *)table;
  const size_t block_bytes = (size_t)H * B * D * sizeof(T);
  const size_t lane_off = ((size_t)h * B + trow) * D * sizeof(T) + (size_t)col * 16;
  const char *kbase = reinterpret_cast<const char *>(p.k_pool) + lane_off;
  const char *vbase = reinterpret_cast<const char *>(p.v_pool) + lane_off;
  const unsigned num_blocks = (unsigned)p.num_blocks;
  bool bad = false;
  // Fused append: the token at position ctx - 1 comes from the new rows,
  // not from the pool, which the same launch is writing it to.
  const int last = ctx - 1;
  const char *nk = append ? reinterpret_cast<const char *>(p.new_key) + row * D * sizeof(T)
                          : nullptr;
  const char *nv = append ? reinterpret_cast<const char *>(p.new_value) + row * D * sizeof(T)
                          : nullptr;

  // Load the 16-token tile starting at logical token ts.  With kCheck,
  // groups at or past tok_end are not loaded (their table entries may not
  // exist); full tiles skip the check.  kScalar picks the table view;
  // kFirst takes the entries from `first` (the wave's first tile).
  auto fetch = [&](Tile<T, D> &tile, int ts, auto check_tag, auto scalar_tag,
                   auto first_tag) {
    constexpr bool kCheck = decltype(check_tag)::value;
    constexpr bool kScalar = decltype(scalar_tag)::value;
    constexpr bool kFirst = decltype(first_tag)::value;
#pragma unroll
    for (int g = 0; g < G::kGroups; ++g) {
      const int gs = ts + g * kTPG;
      int lb, off;
      if constexpr (B >= 16) {
        lb = ts / B;
        off = ts % B + g * kTPG;
      } else {
        lb = gs / B;
        off = gs % B;
      }
      if (!kCheck || gs < tok_end) {
        const int phys = kFirst ? first.e[B >= 16 ? 0 : (g * kTPG) / B]
                                : (kScalar ? table_s[lb] : table[lb]);
        const bool ok = (unsigned)phys < num_blocks;
        bad |= !ok;
        const size_t boff = (size_t)(ok ? phys : 0) * block_bytes + (size_t)off * D * sizeof(T);
        // The lanes of the appended token read its new rows instead: one
        // load per chunk either way, so no second write to the tile
        // registers is pending when the tile is consumed.
        const bool fresh = append && gs + trow == last;
#pragma unroll
        for (int k = 0; k < G::kChunksPerLane; ++k) {
          const char *ka = kbase + boff + k * kLPT * 16;
          const char *va = vbase + boff + k * kLPT * 16;
          if (fresh) {
            ka = nk + (col + k * kLPT) * 16;
            va = nv + (col + k * kLPT) * 16;
          }
          tile.k[g][k] = load_kv<kKeep>(ka);
          tile.v[g][k] = load_kv<kKeep>(va);
        }
      } else {
#pragma unroll
        for (int k = 0; k < G::kChunksPerLane; ++k) {
          tile.k[g][k].u = make_uint4(0, 0, 0, 0);
          tile.v[g][k].u = make_uint4(0, 0, 0, 0);
        }
      }
    }
  };

  RowState<G::kAcc> st;
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int i = 0; i < G::kAcc; ++i) st.acc[i] = 0.f;

  // Fold one tile into the row state.  kMask: the tile may hold tokens at or
  // past tok_end, which are excluded by select.
  auto consume = [&](Tile<T, D> &tile, int ts, auto mask_tag) {
    // No contraction here: fused into the exponent, score * scale - max
    // would skip the rounding of the product, and the best token's weight
    // would be 2^(that rounding error) instead of exactly 1.
#pragma clang fp contract(off)
    constexpr bool kMask = decltype(mask_tag)::value;
    float s[G::kGroups];
#pragma unroll
    for (int g = 0; g < G::kGroups; ++g) {
      float d = 0.f;
#pragma unroll
      for (int k = 0; k < G::kChunksPerLane; ++k) d = dot_chunk(qc[k], tile.k[g][k], d, T());
      s[g] = row_sum<kLPT>(d) * p.scale_log2;
    }
    if constexpr (kMask) {
#pragma unroll
      for (int g = 0; g < G::kGroups; ++g) {
        const bool valid = ts + g * kTPG + trow < tok_end;
        s[g] = valid ? s[g] : -INFINITY;
#pragma unroll
        for (int k = 0; k < G::kChunksPerLane; ++k)
#pragma unroll
          for (int j = 0; j < 4; ++j) tile.v[g][k].w[j] = valid ? tile.v[g][k].w[j] : 0u;
      }
    }
    float mx = st.m;
#pragma unroll
    for (int g = 0; g < G::kGroups; ++g) mx = fmaxf(mx, s[g]);
    // A row that has seen no valid token keeps m = -inf; use 0 as the
    // reference so that no -inf - -inf appears.
    const float mu = (kMask && mx == -INFINITY) ? 0.f : mx;
    const float alpha = fast_exp2(st.m - mu);
    st.l *= alpha;
#pragma unroll
    for (int i = 0; i < G::kAcc; ++i) st.acc[i] *= alpha;
#pragma unroll
    for (int g = 0; g < G::kGroups; ++g) {
      const float pg = fast_exp2(s[g] - mu);
      st.l += pg;
#pragma unroll
      for (int k = 0; k < G::kChunksPerLane; ++k)
        axpy_chunk(st.acc + k * G::kPerChunk, pg, tile.v[g][k], T());
    }
    st.m = mx;
  };

  const int span = tok_end - tok0;
  const int nfull = span / G::kTile;
  {
    // Full tiles of this wave: t = wave, wave + W, ...  Two tile buffers in
    // ping-pong; each step issues the next tile's loads before consuming the
    // current one, and the issue is unconditional inside each branch so the
    // wait before a consume covers only that tile's loads.
    const int iters = nfull > wave ? (nfull - wave + W - 1) / W : 0;
    Tile<T, D> ta, tb;
    auto tile_start = [&](int n) { return tok0 + (wave + n * W) * G::kTile; };
    if (iters > 0) fetch(ta, tile_start(0), std::false_type(), std::false_type(), std::true_type());
    int n = 0;
    for (; n + 2 < iters; n += 2) {
      fetch(tb, tile_start(n + 1), std::false_type(), std::true_type(), std::false_type());
      __builtin_amdgcn_sched_barrier(0);  // keep the next tile's loads first
      consume(ta, tile_start(n), std::false_type());
      fetch(ta, tile_start(n + 2), std::false_type(), std::true_type(), std::false_type());
      __builtin_amdgcn_sched_barrier(0);
      consume(tb, tile_start(n + 1), std::false_type());
    }
    if (n + 1 < iters) {
      fetch(tb, tile_start(n + 1), std::false_type(), std::true_type(), std::false_type());
      __builtin_amdgcn_sched_barrier(0);
      consume(ta, tile_start(n), std::false_type());
      consume(tb, tile_start(n + 1), std::false_type());
    } else if (n < iters) {
      consume(ta, tile_start(n), std::false_type());
    }
    // Ragged last tile.
    if (nfull * G::kTile < span && wave == nfull % W) {
      const int ts = tok0 + nfull * G::kTile;
      fetch(ta, ts, std::true_type(), std::false_type(), std::false_type());
      consume(ta, ts, std::true_type());
    }
  }
  if (bad) st.l = NAN;  // a table entry outside the pool poisons the row

  // Fold the wave's lane rows together (butterfly over the row bits of the
  // lane index): every lane ends with the wave's state for its chunk(s).
#pragma unroll
  for (int off = kLPT; off < 64; off <<= 1) {
    const float m2 = __shfl_xor(st.m, off);
    const float l2 = __shfl_xor(st.l, off);
    const float mn = fmaxf(st.m, m2);
    const float a = st.m == -INFINITY ? 0.f : fast_exp2(st.m - mn);
    const float a2 = m2 == -INFINITY ? 0.f : fast_exp2(m2 - mn);
    st.l = st.l * a + l2 * a2;
#pragma unroll
    for (int i = 0; i < G::kAcc; ++i) {
      const float o2 = __shfl_xor(st.acc[i], off);
      st.acc[i] = st.acc[i] * a + o2 * a2;
    }
    st.m = mn;
  }
  // Merge the W wave states of this workgroup.
  if (trow == 0) {
    if (col == 0) {
      sh.m[wave] = st.m;
      sh.l[wave] = st.l;
    }
#pragma unroll
    for (int k = 0; k < G::kChunksPerLane; ++k)
#pragma unroll
      for (int i = 0; i < G::kPerChunk; ++i)
        sh.o[wave][(col + k * kLPT) * G::kPerChunk + i] = st.acc[k * G::kPerChunk + i];
  }
  __syncthreads();

  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < kStates; ++s) M = fmaxf(M, sh.m[s]);
  float lsum = 0.f;
#pragma unroll
  for (int s = 0; s < kStates; ++s) {
    const float ms = sh.m[s];
    lsum += (ms == -INFINITY ? 0.f : fast_exp2(ms - M)) * sh.l[s];
  }

  if (n_parts == 1) {
    for (int d = threadIdx.x; d < D; d += 64 * W) {
      float o = 0.f;
#pragma unroll
      for (int s = 0; s < kStates; ++s) {
        const float ms = sh.m[s];
        o += (ms == -INFINITY ? 0.f : fast_exp2(ms - M)) * sh.o[s][d];
      }
      out_row[d] = T(o / lsum);
    }
    return;
  }

  // Several partitions: publish this one's partial result for the merge pass.
  const int NP = p.num_partitions;
  float *po = p.part_o + (row * NP + part) * D;
  for (int d = threadIdx.x; d < D; d += 64 * W) {
    float o = 0.f;
#pragma unroll
    for (int s = 0; s < kStates; ++s) {
      const float ms = sh.m[s];
      o += (ms == -INFINITY ? 0.f : fast_exp2(ms - M)) * sh.o[s][d];
    }
    po[d] = o;
  }
  if (threadIdx.x == 0) p.part_ml[row * NP + part] = make_float2(M, lsum);
}

// Fused append in the grid launch: the extra column of workgroups (head
// index num_heads) copies sequence b's new K and V rows of every head to the
// token's slot (a slot outside the pool is skipped, as pa_write_kv does).
// No workgroup of the launch reads that slot: the attention takes the new
// token from its input rows.  Each pass loads its chunks, then stores them.
template <typename T, int D, int B, int W>
__device__ __forceinline__ void write_seq_rows(const DecodeParams &p, int b) {
  constexpr int kC = D * (int)sizeof(T) / 16;  // 16-byte chunks per row
  constexpr int kThreads = 64 * W;
  const int64_t slot = ((const ConstI64 *)p.slot_mapping)[b];
  if (slot < 0 || slot >= (int64_t)p.num_blocks * B) return;
  const size_t blk = (size_t)(slot / B), off = (size_t)(slot % B);
  const int total = 2 * p.num_heads * kC;
  for (int base = 0; base < total; base += kThreads * kWriterChunks) {
    uint4 data[kWriterChunks];
    uint4 *dst[kWriterChunks];
#pragma unroll
    for (int i = 0; i < kWriterChunks; ++i) {
      const int c = base + (int)threadIdx.x + i * kThreads;
      dst[i] = nullptr;
      data[i] = make_uint4(0, 0, 0, 0);
      if (c < total) {
        const int h = c / (2 * kC);
        const int e = c % (2 * kC);
        const bool is_k = e < kC;
        const int ch = is_k ? e : e - kC;
        const size_t src = ((size_t)b * p.num_heads + h) * kC + ch;
        const size_t at = ((blk * p.num_heads + h) * B + off) * kC + ch;
        data[i] = reinterpret_cast<const uint4 *>(is_k ? p.new_key : p.new_value)[src];
        dst[i] = reinterpret_cast<uint4 *>(const_cast<void *>(is_k ? p.k_pool : p.v_pool)) + at;
      }
    }
#pragma unroll
    for (int i = 0; i < kWriterChunks; ++i)
      if (dst[i]) *dst[i] = data[i];
  }
}

// Fused append in the listed launch: workgroups past the list copy the new
// tokens' K and V rows of head h, sequences [first, first + count), to their
// slots (slots outside the pool are skipped, as pa_write_kv does).  No
// workgroup of the launch reads those slots: the attention takes the new
// token from its input rows.
template <typename T, int D, int B, int W>
__device__ __forceinline__ void write_new_rows(const DecodeParams &p, int h, int first,
                                               int count) {
  constexpr int kC = D * (int)sizeof(T) / 16;  // 16-byte chunks per row
  constexpr int kThreads = 64 * W;
  // Three phases (slots, rows, stores), so each phase's loads are in flight
  // together: two memory latencies per writer, not two per chunk.
  int64_t slot[kWriterChunks];
#pragma unroll
  for (int i = 0; i < kWriterChunks; ++i) {
    const int c = (int)threadIdx.x + i * kThreads;
    slot[i] = c < count * 2 * kC ? p.slot_mapping[first + c / (2 * kC)] : -1;
  }
  uint4 data[kWriterChunks];
  uint4 *dst[kWriterChunks];
#pragma unroll
  for (int i = 0; i < kWriterChunks; ++i) {
    const int c = (int)threadIdx.x + i * kThreads;
    dst[i] = nullptr;
    data[i] = make_uint4(0, 0, 0, 0);
    if (slot[i] >= 0 && slot[i] < (int64_t)p.num_blocks * B) {
      const int b = first + c / (2 * kC);
      const int e = c % (2 * kC);
      const bool is_k = e < kC;
      const int ch = is_k ? e : e - kC;
      const size_t src = ((size_t)b * p.num_heads + h) * kC + ch;
      const size_t at =
          (((size_t)(slot[i] / B) * p.num_heads + h) * B + (size_t)(slot[i] % B)) * kC + ch;
      data[i] = reinterpret_cast<const uint4 *>(is_k ? p.new_key : p.new_value)[src];
      dst[i] = reinterpret_cast<uint4 *>(const_cast<void *>(is_k ? p.k_pool : p.v_pool)) + at;
    }
  }
#pragma unroll
  for (int i = 0; i < kWriterChunks; ++i)
    if (dst[i]) *dst[i] = data[i];
}

// Sequences whose new rows one writer workgroup copies.
template <typename T, int D, int W>
constexpr int writer_seqs() {
  return kWriterChunks * 64 * W / (2 * D * (int)sizeof(T) / 16);
}

// Workgroup for head h of sequence b, partition `part`: clamps the context
// from the device array, writes a zero row for an empty context (partition
// 0 only) and leaves at once when the partition holds no token.  With a
// fused append the launch's writer workgroups store the new rows.
template <typename T, int D, int B, int W>
__device__ __forceinline__ void decode_one(const DecodeParams &p, ItemShared<T, D, W> &sh, int h,
                                           int b, int part) {
  // Everything the first K/V loads need but the context length follows
  // from (b, part): the two entries that pick the load policy and this
  // wave's first-tile entries are loaded beside the context length, all as
  // scalar loads (the kernel never writes these arrays) issued before the
  // first wait, so the first K/V loads wait for one round trip instead of
  // three.  The loads are unconditional, at indices clamped into the table
  // rows; an entry read at a clamped index is never used: a tile that
  // exists lies inside the row, and the next row's entry only counts when
  // there is a next row.
  const ConstI32 *row_s = (const ConstI32 *)(p.block_tables + (size_t)b * p.max_blocks_per_seq);
  const int last_lb = p.max_blocks_per_seq - 1;
  const int lb0 = min(part * p.partition_size / B, last_lb);
  const bool has_next = b + 1 < p.num_seqs;
  const int32_t e_here = row_s[lb0];
  const int32_t e_next = row_s[(has_next ? p.max_blocks_per_seq : 0) + lb0];
  FirstEntries<B> first;
  {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lb = (part * p.partition_size + wave * 16) / B;
#pragma unroll
    for (int i = 0; i < FirstEntries<B>::kCount; ++i) first.e[i] = row_s[min(lb + i, last_lb)];
  }
  // The query row's chunks are loaded here too: they need only (b, h).
  Chunk qc[Geometry<T, D>::kChunksPerLane];
  load_q<T, D>(p, b, h, qc);
  int ctx = ((const ConstI32 *)p.context_lens)[b];
  // Keeps the entry loads above the branches below (the compiler would
  // otherwise sink them past the context checks, one round trip later).
  asm volatile("" ::"s"(e_here), "s"(e_next));
#pragma unroll
  for (int i = 0; i < FirstEntries<B>::kCount; ++i) asm volatile("" ::"s"(first.e[i]));
  ctx = ctx < 0 ? 0 : (ctx > p.max_context_len ? p.max_context_len : ctx);
  // A partition whose first block the next sequence of the batch maps at the
  // same logical index is read again by that sequence's workgroups: parallel
  // samples share their prompt's blocks and sit next to each other in the
  // batch, and with the head as the grid's fastest index their workgroups for
  // one head run on the same XCD.  Such an item loads its K/V with the
  // default, cache-retaining policy; every other item streams them
  // non-temporally.  The next row's entry is only compared, never used as an
  // address.
  const bool keep = has_next && e_next == e_here;
  // With a fused append the item that owns the last token (partition 0 for
  // an empty context) reads it from the new rows; no item of the launch
  // reads that slot.
  const int n_parts = (ctx + p.partition_size - 1) / p.partition_size;
  const bool append = p.new_key != nullptr && part == (n_parts > 0 ? n_parts - 1 : 0);
  if (ctx == 0) {
    if (part == 0) {
      T *out_row = reinterpret_cast<T *>(p.out) + ((size_t)b * p.num_heads + h) * D;
      for (int d = threadIdx.x; d < D; d += 64 * W) out_row[d] = T(0);
    }
    return;
  }
  if (part * p.partition_size >= ctx) return;
  if (keep)
    process_item<T, D, B, W, true>(p, sh, b, h, part, ctx, append, first, qc);
  else
    process_item<T, D, B, W, false>(p, sh, b, h, part, ctx, append, first, qc);
}

// One workgroup per (head, sequence, partition); the hardware dispatcher
// hands slots to workgroups as earlier ones finish.  The partition index is
// the slowest grid dimension, counted down: the last partitions, which
// exist only for the longest sequences, are dispatched first and partition
// 0 (every row, including the short ones) last, so the work that trails
// the launch is the smallest.  With a fused append the grid has
// ceil(num_seqs / num_heads) more rows after the sequences: in the
// last-dispatched slice, workgroup (x, num_seqs + r) stores the new rows of
// sequence r * num_heads + x (write_seq_rows), so the writers are the last
// workgroups of the launch and their scattered stores do not interleave
// with the decode's reads; in the other slices those rows leave at once.
// Waves per SIMD the decode kernels are compiled for: fp16 tiles fit 5 at
// B < 16 (at most 96 VGPRs) and 4 otherwise (128); fp32 is left to the
// compiler.
template <typename T, int B>
constexpr int decode_waves_per_eu() {
  return sizeof(T) == 2 ? (B < 16 ? 5 : 4) : 1;
}

template <typename T, int D, int B, int W>
__global__ void __launch_bounds__(64 * W)
    __attribute__((amdgpu_waves_per_eu(decode_waves_per_eu<T, B>())))
    decode_kernel(const DecodeParams p) {
  __shared__ ItemShared<T, D, W> sh;
  if ((int)blockIdx.y >= p.num_seqs) {
    if (blockIdx.z == gridDim.z - 1) {
      const int b = ((int)blockIdx.y - p.num_seqs) * p.num_heads + (int)blockIdx.x;
      if (b < p.num_seqs) write_seq_rows<T, D, B, W>(p, b);
    }
    return;
  }
  decode_one<T, D, B, W>(p, sh, blockIdx.x, blockIdx.y, p.num_partitions - 1 - (int)blockIdx.z);
}

// Workgroups own (head, listed item): the host listed the non-empty
// (sequence, partition) items, longest first, so no workgroup is empty and
// the smallest items trail the launch.  With a fused append, the rows past
// the list are writers (write_new_rows), which fill the launch's tail.
template <typename T, int D, int B, int W>
__global__ void __launch_bounds__(64 * W)
    __attribute__((amdgpu_waves_per_eu(decode_waves_per_eu<T, B>())))
    decode_listed_kernel(const DecodeParams p,
                                                                const WorkList items) {
  __shared__ ItemShared<T, D, W> sh;
  const int y = blockIdx.y;
  if (y >= items.count) {
    constexpr int S = writer_seqs<T, D, W>();
    const int first = (y - items.count) * S;
    write_new_rows<T, D, B, W>(p, blockIdx.x, first, min(S, p.num_seqs - first));
    return;
  }
  const uint32_t it = items.item[y];
  decode_one<T, D, B, W>(p, sh, blockIdx.x, (int)(it >> 16), (int)(it & 0xffffu));
}

// Second pass, rows with several partitions only: out = sum_p w_p o_p /
// sum_p w_p l_p with w_p = 2^(m_p - max_p m_p).  One workgroup of head_dim
// threads per (head, sequence); the partition results come from the first
// pass, made visible by the kernel boundary.
template <typename T, int D>
__device__ __forceinline__ void merge_one(const DecodeParams &p, int h, int b) {
  const size_t row = (size_t)b * p.num_heads + h;
  int ctx = p.context_lens[b];
  ctx = ctx < 0 ? 0 : (ctx > p.max_context_len ? p.max_context_len : ctx);
  const int P = p.partition_size;
  const int n_parts = (ctx + P - 1) / P;
  if (n_parts <= 1) return;  // written by the first pass
  const int NP = p.num_partitions;
  const float2 *ml = p.part_ml + row * NP;
  float gM = -INFINITY;
  for (int q = 0; q < n_parts; ++q) gM = fmaxf(gM, ml[q].x);
  const float *po = p.part_o + row * NP * D;
  const int d = threadIdx.x;
  float num = 0.f, den = 0.f;
  for (int q = 0; q < n_parts; ++q) {
    const float2 mlq = ml[q];
    const float w = mlq.x == -INFINITY ? 0.f : fast_exp2(mlq.x - gM);
    num += w * po[(size_t)q * D + d];
    den += w * mlq.y;
  }
  reinterpret_cast<T *>(p.out)[row * D + d] = T(num / den);
}

template <typename T, int D>
__global__ void __launch_bounds__(D) merge_kernel(const DecodeParams p) {
  merge_one<T, D>(p, blockIdx.x, blockIdx.y);
}

template <typename T, int D>
__global__ void __launch_bounds__(D) merge_listed_kernel(const DecodeParams p,
                                                          const WorkList rows) {
  merge_one<T, D>(p, blockIdx.x, (int)rows.item[blockIdx.y]);
}

// Waves per workgroup: 8 (4 and 16 measured slower on the lognormal batch).
// Both launches also have a 4-wave form for short rows, where 8 waves leave
// most of them one tile or none: the listed launch when its items average
// under 12 tiles, the grid launch when no row is longer than 256 tokens (the
// host's bound on every row).
constexpr int kDecodeWaves = 8;

struct Lists {
  const WorkList *items, *merge_rows;
  int waves;
};

template <typename T, int D, int B, int W>
void launch_listed(const DecodeParams &p, Lists l, hipStream_t stream) {
  constexpr int S = writer_seqs<T, D, W>();
  const int writers = p.new_key != nullptr ? (p.num_seqs + S - 1) / S : 0;
  decode_listed_kernel<T, D, B, W>
      <<<dim3(p.num_heads, l.items->count + writers), 64 * W, 0, stream>>>(p, *l.items);
}

template <typename T, int D, int B>
hipError_t launch_typed(const DecodeParams &p, int num_seqs, Lists l, hipStream_t stream) {
  constexpr int W = kDecodeWaves;
  if (l.items) {
    if (l.items->count > 0 || (p.new_key != nullptr && num_seqs > 0)) {
      if (l.waves == 4) launch_listed<T, D, B, 4>(p, l, stream);
      else launch_listed<T, D, B, 8>(p, l, stream);
    }
    if (p.num_partitions > 1 && l.merge_rows && l.merge_rows->count > 0)
      merge_listed_kernel<T, D>
          <<<dim3(p.num_heads, l.merge_rows->count), D, 0, stream>>>(p, *l.merge_rows);
    return hipGetLastError();
  }
  const int writer_rows = p.new_key != nullptr ? (num_seqs + p.num_heads - 1) / p.num_heads : 0;
  const dim3 grid(p.num_heads, num_seqs + writer_rows, p.num_partitions);
  if (l.waves == 4) decode_kernel<T, D, B, 4><<<grid, 64 * 4, 0, stream>>>(p);
  else decode_kernel<T, D, B, W><<<grid, 64 * W, 0, stream>>>(p);
  if (p.num_partitions > 1)
    merge_kernel<T, D><<<dim3(p.num_heads, num_seqs), D, 0, stream>>>(p);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_block(const DecodeParams &p, int num_seqs, int block_size, Lists l,
                        hipStream_t s) {
  switch (block_size) {
    case 8: return launch_typed<T, D, 8>(p, num_seqs, l, s);
    case 16: return launch_typed<T, D, 16>(p, num_seqs, l, s);
    case 32: return launch_typed<T, D, 32>(p, num_seqs, l, s);
    case 64: return launch_typed<T, D, 64>(p, num_seqs, l, s);
  }
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t launch_dim(const DecodeParams &p, int num_seqs, int head_dim, int block_size,
                      Lists l, hipStream_t s) {
  switch (head_dim) {
    case 64: return launch_block<T, 64>(p, num_seqs, block_size, l, s);
    case 128: return launch_block<T, 128>(p, num_seqs, block_size, l, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode(const DecodeParams &p, int num_seqs, int head_dim, int block_size,
                         int dtype, const WorkList *items, const WorkList *merge_rows,
                         int waves, hipStream_t stream) {
  const Lists l{items, merge_rows, waves};
  if (dtype == 0) return launch_dim<_Float16>(p, num_seqs, head_dim, block_size, l, stream);
  if (dtype == 1) return launch_dim<float>(p, num_seqs, head_dim, block_size, l, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa
