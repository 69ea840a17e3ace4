// Top-k chunk selection, recent-window merge and index build (ChunkKV page,
// section 4.1, Algorithm 1 steps 4-6; the TopK -> index form is Kara eqs.
// (2)-(3)).
//
// Work item = (scoring layer, sequence, KV head), one workgroup.
//  1. Radix select on the fp32 score bit patterns (scores are >= 0, so the
//     unsigned order of the bits is the value order): four 8-bit passes over
//     the C scores find the exact k-th largest pattern tau and how many
//     scores equal to tau are still needed.
//  2. One ordered pass over the chunks: a chunk is selected if its score is
//     above tau, or equal to tau and among the first `need` equal ones in id
//     order (lower chunk id first).  Each chunk then contributes either all
//     its tokens (selected) or its overlap with the recent window [T-w, T);
//     an exclusive scan over the chunks gives every kept token its place, so
//     the index list comes out ascending and without duplicates.
#include "chunkkv_internal.h"

namespace ckv {
namespace {

// Exclusive prefix sum over the workgroup in thread order; `total` gets the sum.
__device__ __forceinline__ int block_exclusive_scan(int v, int* wave_tot, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) wave_tot[wave] = x;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kThreads / 64; ++i) {
    const int t = wave_tot[i];
    base += i < wave ? t : 0;
    tot += t;
  }
  __syncthreads();
  total = tot;
  return base + x - v;
}

__global__ __launch_bounds__(kThreads) void select_kernel(const SelectParams P) {
  __shared__ unsigned hist[256];
  __shared__ int wave_tot[kThreads / 64];
  __shared__ unsigned sh_prefix, sh_mask;
  __shared__ int sh_rem;
  const int tid = threadIdx.x;

  const int per_layer = P.n_seqs * P.H_kv;
  const int li = blockIdx.x / per_layer;
  const int rest = blockIdx.x - li * per_layer;
  const int b = rest / P.H_kv, h = rest - b * P.H_kv;
  const int T = P.T[b], C = P.C[b], c = P.c, w = P.w;
  const int kk = min(P.kk[b], C);
  const unsigned* S = reinterpret_cast<const unsigned*>(P.scores + li * P.score_layer_stride +
                                                        P.score_off[b] + static_cast<int64_t>(h) * C);
  int32_t* idx = P.indices + li * P.index_layer_stride + P.index_off[b] +
                 static_cast<int64_t>(h) * P.L_cap[b];
  const bool all = kk >= C, none = kk == 0;

  unsigned tau = 0;
  int need = 0;
  if (!all && !none) {
    unsigned prefix = 0, mask = 0;
    int rem = kk;
    for (int shift = 24; shift >= 0; shift -= 8) {
      hist[tid] = 0;
      __syncthreads();
      for (int j = tid; j < C; j += kThreads) {
        const unsigned key = S[j];
        if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (tid == 0) {
        int cum = 0, dsel = 0;
        for (int dg = 255; dg >= 0; --dg) {
          const int hc = static_cast<int>(hist[dg]);
          if (cum + hc >= rem) {
            dsel = dg;
            break;
          }
          cum += hc;
        }
        sh_rem = rem - cum;
        sh_prefix = prefix | (static_cast<unsigned>(dsel) << shift);
        sh_mask = mask | (255u << shift);
      }
      __syncthreads();
      prefix = sh_prefix;
      mask = sh_mask;
      rem = sh_rem;
    }
    tau = prefix;
    need = rem;
  }

  const int64_t t_win = static_cast<int64_t>(T) - w;
  int carry_eq = 0, carry_off = 0;
  for (int base = 0; base < C; base += kThreads) {
    const int j = base + tid;
    const bool in = j < C;
    const unsigned key = in ? S[j] : 0u;
    const int is_eq = (in && !all && !none && key == tau) ? 1 : 0;
    int tot_eq;
    const int eq_rank = block_exclusive_scan(is_eq, wave_tot, tot_eq) + carry_eq;
    const bool sel = in && (all || (!none && (key > tau || (is_eq && eq_rank < need))));
    const int64_t t0 = static_cast<int64_t>(j) * c;
    const int64_t t1 = min(t0 + c, static_cast<int64_t>(T));
    const int64_t s0 = sel ? t0 : max(t0, t_win);
    const int cnt = in ? static_cast<int>(max(static_cast<int64_t>(0), t1 - s0)) : 0;
    int tot_cnt;
    const int off = block_exclusive_scan(cnt, wave_tot, tot_cnt) + carry_off;
    for (int i = 0; i < cnt; ++i) idx[off + i] = static_cast<int32_t>(s0 + i);
    carry_eq += tot_eq;
    carry_off += tot_cnt;
  }
  if (tid == 0) P.lengths[li * P.len_layer_stride + P.len_off[b] + h] = carry_off;
}

}  // namespace

hipError_t launch_select(const SelectParams& p, int n_blocks, hipStream_t s) {
  hipLaunchKernelGGL(select_kernel, dim3(n_blocks), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace ckv
