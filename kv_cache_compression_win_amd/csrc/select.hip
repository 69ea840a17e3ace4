// Top-k chunk selection, recent-window merge and index build (ChunkKV page,
// section 4.1, Algorithm 1 steps 4-6; the TopK -> index form is Kara eqs.
// (2)-(3)).
//
// Work item = (scoring layer, sequence, KV head), one workgroup of 1024
// threads (16 waves).
//  1. Threshold: the scores are >= 0, so the unsigned order of their fp32 bit
//     patterns is the value order.  tau = the largest 32-bit pattern v with
//     #{S_j >= v} >= k is built greedily from the top bit, two bits per
//     workgroup-wide count; it is exactly the k-th largest score.
//     Scores stay in registers (16 per thread) when C <= 16384.
//  2. One ordered pass over the chunks: a chunk is selected if its score is
//     above tau, or equal to tau and among the first k - #{S > tau} equal ones
//     in id order (lower chunk id first).  Each chunk contributes all its
//     tokens (selected) or its overlap with the recent window [T-w, T); an
//     exclusive scan over the chunks places every kept token, so the index
//     list is ascending and duplicate-free.
#include "chunkkv_internal.h"

namespace ckv {
namespace {

constexpr int kWaves = kSelectThreads / 64;
constexpr int kKPT = kSelectKeysPerThread;

// Workgroup-wide sum; every thread receives the total.
__device__ __forceinline__ int block_sum(int v, int* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  if (lane == 0) red[wave] = v;
  __syncthreads();
  int t = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) t += red[i];
  __syncthreads();
  return t;
}

// Workgroup-wide sums of three counters at once.
__device__ __forceinline__ int3 block_sum3(int3 v, int3* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    v.x += __shfl_xor(v.x, o, 64);
    v.y += __shfl_xor(v.y, o, 64);
    v.z += __shfl_xor(v.z, o, 64);
  }
  if (lane == 0) red[wave] = v;
  __syncthreads();
  int3 t = make_int3(0, 0, 0);
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    t.x += red[i].x;
    t.y += red[i].y;
    t.z += red[i].z;
  }
  __syncthreads();
  return t;
}

// Exclusive prefix sum over the workgroup in thread order; `total` gets the sum.
__device__ __forceinline__ int block_exclusive_scan(int v, int* red, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) red[wave] = x;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    const int t = red[i];
    base += i < wave ? t : 0;
    tot += t;
  }
  __syncthreads();
  total = tot;
  return base + x - v;
}

__global__ __launch_bounds__(kSelectThreads) void select_kernel(const SelectParams P) {
  __shared__ int red[kWaves];
  __shared__ int3 red3[kWaves];
  const int tid = threadIdx.x;

  const int per_layer = P.n_seqs * P.H_kv;
  const int li = blockIdx.x / per_layer;
  const int rest = blockIdx.x - li * per_layer;
  const int b = rest / P.H_kv, h = rest - b * P.H_kv;
  const int T = P.T[b], C = P.C[b], c = P.c, w = P.w;
  const int kk = min(P.kk[b], C);
  const float* S = P.scores + li * P.score_layer_stride + P.score_off[b] + static_cast<int64_t>(h) * C;
  int32_t* idx = P.indices + li * P.index_layer_stride + P.index_off[b] +
                 static_cast<int64_t>(h) * P.L_cap[b];

  const unsigned* Sb = reinterpret_cast<const unsigned*>(S);
  const bool all = kk >= C, none = kk == 0;
  const bool in_regs = C <= kSelectThreads * kKPT;
  unsigned key[kKPT];
#pragma unroll
  for (int i = 0; i < kKPT; ++i) {
    const int j = i * kSelectThreads + tid;
    key[i] = (in_regs && j < C) ? Sb[j] : 0u;
  }

  unsigned tau = 0;
  int need = 0;
  if (!all && !none) {
    // greedy over the 31 value bits (bit 31 is 0 for scores >= 0): bit 30
    // alone, then two bits per step with the three candidates counted at once
    auto count_ge = [&](unsigned cand) {
      int cnt = 0;
      if (in_regs) {
#pragma unroll
        for (int i = 0; i < kKPT; ++i) cnt += key[i] >= cand ? 1 : 0;
      } else {
        for (int j = tid; j < C; j += kSelectThreads) cnt += Sb[j] >= cand ? 1 : 0;
      }
      return cnt;
    };
    unsigned prefix = 0;
    if (block_sum(count_ge(1u << 30), red) >= kk) prefix = 1u << 30;
    for (int bit = 28; bit >= 0; bit -= 2) {
      const unsigned c1 = prefix | (1u << bit), c2 = prefix | (2u << bit), c3 = prefix | (3u << bit);
      int3 cnt = make_int3(0, 0, 0);
      if (in_regs) {
#pragma unroll
        for (int i = 0; i < kKPT; ++i) {
          cnt.x += key[i] >= c1 ? 1 : 0;
          cnt.y += key[i] >= c2 ? 1 : 0;
          cnt.z += key[i] >= c3 ? 1 : 0;
        }
      } else {
        for (int j = tid; j < C; j += kSelectThreads) {
          const unsigned kj = Sb[j];
          cnt.x += kj >= c1 ? 1 : 0;
          cnt.y += kj >= c2 ? 1 : 0;
          cnt.z += kj >= c3 ? 1 : 0;
        }
      }
      const int3 tot = block_sum3(cnt, red3);
      prefix = tot.z >= kk ? c3 : tot.y >= kk ? c2 : tot.x >= kk ? c1 : prefix;
    }
    tau = prefix;
    int gt = 0;
    if (in_regs) {
#pragma unroll
      for (int i = 0; i < kKPT; ++i) gt += key[i] > tau ? 1 : 0;
    } else {
      for (int j = tid; j < C; j += kSelectThreads) gt += Sb[j] > tau ? 1 : 0;
    }
    need = kk - block_sum(gt, red);
  }

  const int64_t t_win = static_cast<int64_t>(T) - w;
  int carry_eq = 0, carry_off = 0;
  auto tile = [&](int j, unsigned k_j) {
    const bool in = j < C;
    const int is_eq = (in && !all && !none && k_j == tau) ? 1 : 0;
    int tot_eq;
    const int eq_rank = block_exclusive_scan(is_eq, red, tot_eq) + carry_eq;
    const bool sel = in && (all || (!none && (k_j > tau || (is_eq && eq_rank < need))));
    const int64_t t0 = static_cast<int64_t>(j) * c;
    const int64_t t1 = min(t0 + c, static_cast<int64_t>(T));
    const int64_t s0 = sel ? t0 : max(t0, t_win);
    const int cnt = in ? static_cast<int>(max(static_cast<int64_t>(0), t1 - s0)) : 0;
    int tot_cnt;
    const int off = block_exclusive_scan(cnt, red, tot_cnt) + carry_off;
    for (int i = 0; i < cnt; ++i) idx[off + i] = static_cast<int32_t>(s0 + i);
    carry_eq += tot_eq;
    carry_off += tot_cnt;
  };
  if (in_regs) {
#pragma unroll
    for (int i = 0; i < kKPT; ++i)
      if (i * kSelectThreads < C) tile(i * kSelectThreads + tid, key[i]);
  } else {
    for (int base = 0; base < C; base += kSelectThreads) {
      const int j = base + tid;
      tile(j, j < C ? Sb[j] : 0u);
    }
  }
  if (tid == 0) P.lengths[li * P.len_layer_stride + P.len_off[b] + h] = carry_off;
}

}  // namespace

hipError_t launch_select(const SelectParams& p, int n_blocks, hipStream_t s) {
  hipLaunchKernelGGL(select_kernel, dim3(n_blocks), dim3(kSelectThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace ckv
