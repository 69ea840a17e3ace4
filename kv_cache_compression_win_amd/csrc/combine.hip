// Log-sum-exp combine of the score kernels' span partials into chunk scores
// (ChunkKV page, section 4.1, Algorithm 1 step 3; each attention row is
// normalised over all T keys as in Kara eq. (1)).
//
// For row r of a KV head with per-span statistics (m_s, l_s):
//   M_r = max_s m_s,  L_r = sum_s 2^((m_s - M_r) * scale) * l_s,
// and a chunk j of span s scores
//   S_j = sum_r U[j][r] * 2^((m_s,r - M_r) * scale) / L_r.
// Work item = (layer, sequence, KV head, span); rows are summed in a fixed
// order (lane-strided, then a fixed butterfly), so results are deterministic.
#include "chunkkv_internal.h"

namespace ckv {
namespace {

constexpr int kMaxRows = 4096;

__global__ __launch_bounds__(kThreads) void combine_kernel(const CombineParams P) {
  __shared__ float wts[kMaxRows];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  const int li = blockIdx.x / P.items_per_layer;
  int item = blockIdx.x - li * P.items_per_layer;
  int b = 0;
  while (b + 1 < P.n_seqs && item >= P.item0[b + 1]) ++b;
  item -= P.item0[b];
  const int nspan = P.n_span[b];
  const int span = item % nspan;
  const int h = item / nspan;
  const int C = P.C[b];

  const float2* st = P.stats + li * P.st_layer_stride + P.st_off[b] +
                     static_cast<int64_t>(h) * nspan * P.R_pad;
  for (int r = tid; r < P.R; r += kThreads) {
    float M = -INFINITY;
    for (int s = 0; s < nspan; ++s) M = fmaxf(M, st[static_cast<int64_t>(s) * P.R_pad + r].x);
    float L = 0.0f;
    for (int s = 0; s < nspan; ++s) {
      const float2 ml = st[static_cast<int64_t>(s) * P.R_pad + r];
      L += __builtin_amdgcn_exp2f((ml.x - M) * P.scale) * ml.y;
    }
    const float m_this = st[static_cast<int64_t>(span) * P.R_pad + r].x;
    wts[r] = __builtin_amdgcn_exp2f((m_this - M) * P.scale) / L;
  }
  __syncthreads();

  const int j0 = span * P.span_chunks;
  const int nch = min(P.span_chunks, C - j0);
  const float* U = P.U + li * P.u_layer_stride + P.u_off[b] +
                   (static_cast<int64_t>(h) * C + j0) * P.R_pad;
  float* S = P.scores + li * P.score_layer_stride + P.score_off[b] + static_cast<int64_t>(h) * C + j0;
  for (int j = wave; j < nch; j += 4) {
    const float* u = U + static_cast<int64_t>(j) * P.R_pad;
    float acc = 0.0f;
    for (int r = lane; r < P.R; r += 64) acc = fmaf(u[r], wts[r], acc);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
    if (lane == 0) S[j] = acc;
  }
}

}  // namespace

hipError_t launch_combine(const CombineParams& p, int n_blocks, hipStream_t s) {
  if (p.R > kMaxRows) return hipErrorInvalidValue;
  hipLaunchKernelGGL(combine_kernel, dim3(n_blocks), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace ckv
