// Log-sum-exp combine of the score kernels' span partials into chunk scores
// (ChunkKV page, section 4.1, Algorithm 1 step 3; each attention row is
// normalised over all T keys as in Kara eq. (1)).
//
// For row r of a KV head with per-span statistics (m_s, l_s):
//   M_r = max_s m_s,  L_r = sum_s 2^((m_s - M_r) * scale) * l_s,
// and a chunk j of span s scores
//   S_j = sum_r U[j][r] * 2^((m_s,r - M_r) * scale) / L_r.
// Two launches: row_lse_kernel forms (M_r, L_r) once per (layer, sequence,
// KV head) from the span statistics; combine_kernel's work item is (layer,
// sequence, KV head, block of spans), enough items to fill the GPU, each
// reading the head's row statistics and streaming its chunks' U rows with
// eight 16-byte loads in flight per thread.  When every head's span
// statistics are small (at most 32 KB: one round of loads at 128 rows), each
// combine block forms its head's row statistics itself and the row_lse
// launch is skipped.  The row sums follow the fixed
// order of combine_chunks: results are deterministic.
#include "lse_combine.h"

namespace ckv {
namespace {

#ifndef CKV_COMBINE_SPANS
#define CKV_COMBINE_SPANS 4
#endif
constexpr int kMaxRows = 4096;
constexpr int kWeightFloats = 16384;  // weights of one item's spans (64 KB at most)

template <int QPT, bool PACKED>
__global__ __launch_bounds__(kThreads) void combine_kernel(const CombineParams P) {
  // dynamic LDS: weights [spans_per_blk][R_pad], then (fuse_lse) the row
  // statistics [R_pad] as float2
  extern __shared__ float wts[];
  const int tid = threadIdx.x;

  const int li = blockIdx.x / P.items_per_layer;
  int item = blockIdx.x - li * P.items_per_layer;
  int b = 0;
  while (b + 1 < P.n_seqs && item >= P.item0[b + 1]) ++b;
  item -= P.item0[b];
  const int nblk = P.n_blk[b];
  const int blk = item % nblk;
  const int h = item / nblk;
  const int C = P.C[b], nspan = P.n_span[b];

  const float2* st = P.stats + li * P.st_layer_stride + P.st_off[b] +
                     static_cast<int64_t>(h) * nspan * P.R_pad;
  const float2* lse_g = P.lse + li * P.lse_layer_stride + P.lse_off[b] + static_cast<int64_t>(h) * P.R_pad;
  const int s_lo = blk * P.spans_per_blk;
  const int ns = min(P.spans_per_blk, nspan - s_lo);
  if (P.fuse_lse) {
    // short heads: the row statistics are formed here (the same function and
    // thread count as row_lse_kernel, so the same bits) into LDS after the weights
    float2* lse_l = reinterpret_cast<float2*>(wts + P.spans_per_blk * P.R_pad);
    rows_lse<kThreads>(st, nspan, P.R, P.R_pad, P.scale, lse_l);
    __syncthreads();
    for (int e = tid; e < ns * P.R_pad; e += kThreads) {
      const int s = e / P.R_pad, r = e - s * P.R_pad;
      wts[e] = r < P.R ? span_weight(st[static_cast<int64_t>(s_lo + s) * P.R_pad + r].x, lse_l[r], P.scale)
                       : 0.0f;
    }
  } else {
    // the row statistics and the spans' maxima are read together (one memory
    // round trip before the weights)
    for (int e = tid; e < ns * P.R_pad; e += kThreads) {
      const int s = e / P.R_pad, r = e - s * P.R_pad;
      wts[e] = r < P.R ? span_weight(st[static_cast<int64_t>(s_lo + s) * P.R_pad + r].x, lse_g[r], P.scale)
                       : 0.0f;
    }
  }
  __syncthreads();

  const float* U = P.U + li * P.u_layer_stride + P.u_off[b] + static_cast<int64_t>(h) * C * u_row_words(P.R_pad, PACKED);
  float* S = P.scores + li * P.score_layer_stride + P.score_off[b] + static_cast<int64_t>(h) * C;
  const int j_lo = s_lo * P.span_chunks;
  const int j_hi = min(C, (s_lo + ns) * P.span_chunks);
  combine_chunks<kThreads, QPT, PACKED>(U, wts, j_lo, j_hi, s_lo, P.span_chunks, P.R_pad, S);
}

// Row statistics of one (layer, sequence, KV head): (M_r, L_r) over all spans,
// once per head for every combine block of the head.
__global__ __launch_bounds__(kThreads) void row_lse_kernel(const CombineParams P) {
  const int per_layer = P.head0[P.n_seqs];
  const int li = blockIdx.x / per_layer;
  const int item = blockIdx.x - li * per_layer;
  int b = 0;
  while (b + 1 < P.n_seqs && item >= P.head0[b + 1]) ++b;
  const int h = item - P.head0[b];
  const int nspan = P.n_span[b];
  const float2* st = P.stats + li * P.st_layer_stride + P.st_off[b] +
                     static_cast<int64_t>(h) * nspan * P.R_pad;
  float2* lse_g = P.lse + li * P.lse_layer_stride + P.lse_off[b] + static_cast<int64_t>(h) * P.R_pad;
  rows_lse<kThreads>(st, nspan, P.R, P.R_pad, P.scale, lse_g);
}

}  // namespace

hipError_t launch_row_lse(const CombineParams& p, int n_blocks, hipStream_t s) {
  return launch1(row_lse_kernel, dim3(n_blocks), dim3(kThreads), 0, s, p);
}

int combine_spans_per_blk(int R_pad) {
  const int spb = 4096 / R_pad;
  return spb < 1 ? 1 : (spb > CKV_COMBINE_SPANS ? CKV_COMBINE_SPANS : spb);
}

hipError_t launch_combine(const CombineParams& p, int n_blocks, hipStream_t s) {
  if (p.R_pad > kMaxRows || p.spans_per_blk * p.R_pad > kWeightFloats) return hipErrorInvalidValue;
  const size_t lds = static_cast<size_t>(p.spans_per_blk) * p.R_pad * sizeof(float) +
                    (p.fuse_lse ? static_cast<size_t>(p.R_pad) * sizeof(float2) : 0);
#define CKV_COMBINE(Q)                                                                                   \
  case Q:                                                                                                \
    return p.u_packed ? launch1(combine_kernel<Q, true>, dim3(n_blocks), dim3(kThreads), lds, s, p)    \
                      : launch1(combine_kernel<Q, false>, dim3(n_blocks), dim3(kThreads), lds, s, p);
  switch (combine_qpt(p.R_pad)) {
    CKV_COMBINE(1)
    CKV_COMBINE(2)
    CKV_COMBINE(4)
    CKV_COMBINE(8)
    CKV_COMBINE(16)
    default: return hipErrorInvalidValue;
  }
#undef CKV_COMBINE
}

}  // namespace ckv
