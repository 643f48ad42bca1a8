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
// queries each.  Per 32-key tile, on v_mfma_f32_32x32x16_f16:
//   * S^T = K Q^T: the key rows are the A operand, read straight from the
//     pool (16-byte loads along head_dim), the wave's 32 query rows the B
//     operand.  The contraction over head_dim runs in a permuted order that
//     both operands share (lane group g takes the half [g*D/2, (g+1)*D/2)),
//     so that each lane reads one contiguous half row.
//   * In the accumulator layout every lane holds 16 scores of one query
//     (its column), so the online softmax needs one exchange (lanes l and
//     l ^ 32) per tile, and rescaling the output is a per-lane multiply.
//   * O^T += V^T P^T: P^T is the B operand straight from the score
//     registers (converted to fp16, no shuffle); the key order that layout
//     implies is matched by the A operand, V^T, read from LDS, where the
//     workgroup stages each V tile transposed.
// Accumulation and the softmax are fp32; P is rounded to fp16 for the
// second product.
#include <math.h>

#include "pa_kernels.h"

namespace pa {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float float16v __attribute__((ext_vector_type(16)));

constexpr int kWaves = 4;
constexpr int kRows = 32;                 // queries per wave
constexpr int kQTile = kWaves * kRows;    // queries per workgroup
constexpr int kKeys = 32;                 // keys per tile
constexpr int kVtStride = kKeys + 8;      // LDS row of V^T (halves), padded

__device__ inline half8 load_half8(const _Float16 *p) {
  return *reinterpret_cast<const half8 *>(p);
}

template <int D, int B>
__global__ void __launch_bounds__(kWaves * 64)
prefill_kernel(const PrefillParams p) {
  __shared__ _Float16 vt[D * kVtStride];

  const int h = blockIdx.x;
  const int b = blockIdx.z;
  const int qt = (int)gridDim.y - 1 - (int)blockIdx.y;   // longest tiles first
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
  // keys the workgroup needs: up to its last query's position
  const int last = min(m, (qt + 1) * kQTile) - 1;
  const int kv_end = bad_seq ? 0 : n - m + last + 1;

  const _Float16 *qh = static_cast<const _Float16 *>(p.q);
  const _Float16 *kh = static_cast<const _Float16 *>(p.k_pool);
  const _Float16 *vh = static_cast<const _Float16 *>(p.v_pool);
  const int32_t *table = p.block_tables + (int64_t)b * p.max_blocks_per_seq;

  // B operand of S^T: q row r, head-dim half g, in 16-element k-steps.
  constexpr int kSteps = D / 16;
  half8 qb[kSteps];
  {
    const _Float16 *row = qh + ((int64_t)(q0 + r) * p.num_heads + h) * D + g * (D / 2);
#pragma unroll
    for (int j = 0; j < kSteps; ++j) qb[j] = q_ok ? load_half8(row + 8 * j) : half8{};
  }

  float16v acc_o[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t) acc_o[t] = float16v{};
  float m_run = -INFINITY, l_run = 0.f;

  for (int t0 = 0; t0 < kv_end; t0 += kKeys) {
    // Stage V^T of keys t0 .. t0+31 into LDS (zeros past the context).
    __syncthreads();
    for (int chunk = threadIdx.x; chunk < kKeys * (D / 8); chunk += kWaves * 64) {
      const int key = chunk / (D / 8);
      const int d0 = (chunk % (D / 8)) * 8;
      const int t = t0 + key;
      half8 v = {};
      if (t < n) {
        const int32_t phys = table[t / B];
        if (phys >= 0 && phys < p.num_blocks)
          v = load_half8(vh + (((int64_t)phys * p.num_heads + h) * B + t % B) * D + d0);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) vt[(d0 + e) * kVtStride + key] = v[e];
    }

    // S^T = K Q^T.  Lane row c holds key t0 + c.
    float16v s = {};
    {
      const int t = t0 + c;
      const _Float16 *krow = nullptr;
      bool poison = false;
      if (t < n) {
        const int32_t phys = table[t / B];
        if (phys >= 0 && phys < p.num_blocks)
          krow = kh + (((int64_t)phys * p.num_heads + h) * B + t % B) * D + g * (D / 2);
        else
          poison = true;   // a table entry outside the pool: NaN for whoever sees it
      }
#pragma unroll
      for (int j = 0; j < kSteps; ++j) {
        half8 a = {};
        if (krow) a = load_half8(krow + 8 * j);
        if (poison) a = half8{} + (_Float16)NAN;
        s = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, qb[j], s, 0, 0, 0);
      }
    }

    // Online softmax for this lane's query over the tile's valid keys.
    float tile_max = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = t0 + (i / 4) * 8 + g * 4 + (i % 4);
      const float x = s[i] * p.scale_log2;
      s[i] = key <= pos ? x : -INFINITY;
      tile_max = fmaxf(tile_max, s[i]);
    }
    tile_max = fmaxf(tile_max, __shfl_xor(tile_max, 32));
    const float m_new = fmaxf(m_run, tile_max);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    float psum = 0.f;
    half8 pb[2];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float e = __builtin_amdgcn_exp2f(s[i] - m_use);
      psum += e;
      pb[i / 8][i % 8] = (_Float16)e;
    }
    psum += __shfl_xor(psum, 32);
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int t = 0; t < D / 32; ++t) acc_o[t] *= alpha;

    __syncthreads();   // V^T staged
    // O^T += V^T P^T.  k-step jj covers keys 16jj .. 16jj+15 in the order
    // the score registers hold them: slots e = 0..3 -> keys 16jj + 4g + e,
    // slots 4..7 -> keys 16jj + 8 + 4g + (e - 4).
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      const _Float16 *vrow = vt + (dt * 32 + c) * kVtStride;
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const half4 lo = *reinterpret_cast<const half4 *>(vrow + 16 * jj + 4 * g);
        const half4 hi = *reinterpret_cast<const half4 *>(vrow + 16 * jj + 8 + 4 * g);
        const half8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        acc_o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pb[jj], acc_o[dt], 0, 0, 0);
      }
    }
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
hipError_t launch_prefill_d(const PrefillParams &p, int num_seqs, int block_size,
                            int max_query_len, hipStream_t stream) {
  const dim3 grid(p.num_heads, (max_query_len + kQTile - 1) / kQTile, num_seqs);
  switch (block_size) {
    case 8: prefill_kernel<D, 8><<<grid, kWaves * 64, 0, stream>>>(p); break;
    case 16: prefill_kernel<D, 16><<<grid, kWaves * 64, 0, stream>>>(p); break;
    case 32: prefill_kernel<D, 32><<<grid, kWaves * 64, 0, stream>>>(p); break;
    case 64: prefill_kernel<D, 64><<<grid, kWaves * 64, 0, stream>>>(p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

int prefill_query_tile() { return kQTile; }

hipError_t launch_prefill(const PrefillParams &p, int num_seqs, int head_dim, int block_size,
                          int max_query_len, hipStream_t stream) {
  if (head_dim == 128) return launch_prefill_d<128>(p, num_seqs, block_size, max_query_len, stream);
  if (head_dim == 64) return launch_prefill_d<64>(p, num_seqs, block_size, max_query_len, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa
