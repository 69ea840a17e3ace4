// Device helpers of the log-sum-exp combine (ChunkKV page, section 4.1,
// Algorithm 1 step 3, with every attention row normalised over all T keys as
// in Kara eq. (1)).
//
// Row r of a KV head has per-span statistics (m_s, l_s) with
// l_s = sum over the span of 2^((x - m_s) * scale).  Then
//   M_r = max_s m_s,   L_r = sum_s 2^((m_s - M_r) * scale) * l_s,
// and the weight of span s for row r is 2^((m_s - M_r) * scale) / L_r.
#pragma once

#include "chunkkv_internal.h"

namespace ckv {

// Merge of two partial (max, sum) pairs of one row.  Commutative bit for bit
// (fmaxf and the two-term sum are), so a butterfly gives every lane the same
// result.
__device__ __forceinline__ void lse_merge(float& m, float& l, float m2, float l2, float scale) {
  const float M = fmaxf(m, m2);
  if (M == -INFINITY) return;
  l = l * __builtin_amdgcn_exp2f((m - M) * scale) + l2 * __builtin_amdgcn_exp2f((m2 - M) * scale);
  m = M;
}

// Threads that share one row in rows_lse: as many as fit with every row in
// one pass (a power of two, 1 to 8).
__host__ __device__ inline int lse_tpr(int R, int nthreads) {
  int t = 8;
  while (t > 1 && t * R > nthreads) t >>= 1;
  return t;
}

// (M_r, L_r) of every row r < R from the n_span statistics (row stride 1,
// span stride R_pad) into lse[r]: tpr = lse_tpr(R, NTHREADS) consecutive
// threads share a row, thread `sub` merging spans sub, sub + tpr, ... in
// order (loads issued kUnr at a time, so a row of a few dozen spans costs one
// or two memory round trips), then a butterfly over the tpr threads.  The
// result depends only on R, NTHREADS and the statistics.
template <int NTHREADS>
__device__ __forceinline__ void rows_lse(const float2* st, int nspan, int R, int64_t R_pad, float scale,
                                         float2* lse) {
  constexpr int kUnr = 16;
  const int tpr = lse_tpr(R, NTHREADS);
  const int sub = threadIdx.x % tpr;
  for (int r = threadIdx.x / tpr; r < R; r += NTHREADS / tpr) {
    float m = -INFINITY, l = 0.0f;
    for (int s0 = sub; s0 < nspan; s0 += tpr * kUnr) {
      float2 ml[kUnr];
#pragma unroll
      for (int u = 0; u < kUnr; ++u) {
        const int s = s0 + u * tpr;
        ml[u] = s < nspan ? st[s * R_pad + r] : make_float2(-INFINITY, 0.0f);
      }
#pragma unroll
      for (int u = 0; u < kUnr; ++u) lse_merge(m, l, ml[u].x, ml[u].y, scale);
    }
    for (int o = 1; o < tpr; o <<= 1) {
      const float m2 = __shfl_xor(m, o, 64), l2 = __shfl_xor(l, o, 64);
      lse_merge(m, l, m2, l2, scale);
    }
    if (sub == 0) lse[r] = make_float2(m, l);
  }
}

__device__ __forceinline__ float span_weight(float m_span, float2 lse, float scale) {
  return __builtin_amdgcn_exp2f((m_span - lse.x) * scale) / lse.y;
}

// Threads that share one chunk's dot product: R_pad/4 row quads, at most a
// wave (a power of two dividing 64).
#ifndef CKV_COMBINE_QUADS
#define CKV_COMBINE_QUADS 4
#endif
#ifndef CKV_COMBINE_INFLIGHT
#define CKV_COMBINE_INFLIGHT 8
#endif
// Threads sharing a chunk: each takes about CKV_COMBINE_QUADS row quads (8
// threads for 128 rows, 32 for 512), a power of two of at most a wave.
__host__ __device__ inline int combine_tpc(int R_pad) {
  int t = 1;
  while (t < 64 && t * CKV_COMBINE_QUADS < R_pad / 4) t <<= 1;
  return t;
}

// Row quads per thread (power of two >= R_pad/4 / tpc).
__host__ __device__ inline int combine_qpt(int R_pad) {
  const int tpc = combine_tpc(R_pad);
  int q = 1;
  while (q * tpc < R_pad / 4) q <<= 1;
  return q;
}

// Chunk scores S[j] = sum_r U[j][r] * wts[j / span_chunks - s_lo][r] for the
// chunks j in [j_lo, j_hi) of one (layer, sequence, head): U rows are
// u_row_words(R_pad, PACKED) words (padding rows carry weight 0), wts holds
// R_pad weights per span starting at span s_lo.  Groups of tpc consecutive
// threads share a chunk; thread `sub` sums its row quads q = sub + k*tpc
// (k < QPT, 16 bytes of fp32 or 12 bytes of packed partials each) in order,
// then a fixed butterfly over the group, so the result depends on neither
// the workgroup size nor the unrolling.  All loads of an iteration (8 quads
// per thread) are issued before any arithmetic.
template <int NTHREADS, int QPT, bool PACKED>
__device__ __forceinline__ void combine_chunks(const float* U, const float* wts, int j_lo, int j_hi,
                                               int s_lo, int span_chunks, int R_pad, float* S) {
  constexpr int kUnr = QPT >= CKV_COMBINE_INFLIGHT ? 1 : CKV_COMBINE_INFLIGHT / QPT;
  const int tpc = combine_tpc(R_pad);
  const int groups = NTHREADS / tpc;
  const int g = threadIdx.x / tpc, sub = threadIdx.x % tpc;
  const int q4 = R_pad / 4;
  const int64_t row_words = u_row_words(R_pad, PACKED);
  for (int j0 = j_lo; j0 < j_hi; j0 += groups * kUnr) {
    float4 a[kUnr][QPT];
#pragma unroll
    for (int u = 0; u < kUnr; ++u) {
      const int j = j0 + u * groups + g;
      const float* row = U + static_cast<int64_t>(j) * row_words;
#pragma unroll
      for (int k = 0; k < QPT; ++k) {
        const int q = sub + k * tpc;
        if (j < j_hi && q < q4) {
          if constexpr (PACKED)
            a[u][k] = unpack_u24(*reinterpret_cast<const u32x3u*>(row + 3 * q));
          else
            a[u][k] = reinterpret_cast<const float4*>(row)[q];
        } else {
          a[u][k] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kUnr; ++u) {
      const int j = j0 + u * groups + g;
      float acc = 0.0f;
      if (j < j_hi) {
        const float4* wp = reinterpret_cast<const float4*>(wts + (j / span_chunks - s_lo) * R_pad);
#pragma unroll
        for (int k = 0; k < QPT; ++k) {
          const int q = sub + k * tpc;
          if (q < q4) {
            const float4 wv = wp[q];
            acc = fmaf(a[u][k].x, wv.x, acc);
            acc = fmaf(a[u][k].y, wv.y, acc);
            acc = fmaf(a[u][k].z, wv.z, acc);
            acc = fmaf(a[u][k].w, wv.w, acc);
          }
        }
      }
      for (int o = tpc >> 1; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
      if (sub == 0 && j < j_hi) S[j] = acc;
    }
  }
}

}  // namespace ckv
