// Top-k chunk selection, recent-window merge and index build (ChunkKV page,
// section 4.1, Algorithm 1 steps 4-6; the TopK -> index form is Kara eqs.
// (2)-(3)).
//
// Threshold: the scores are >= 0, so the unsigned order of their fp32 bit
// patterns is the value order.  tau = the largest 32-bit pattern v with
// #{S_j >= v} >= k is built greedily from the top bit (bit 30 alone, then two
// bits per workgroup-wide count of three candidates); it is exactly the k-th
// largest score.  The search stops as soon as exactly k chunks reach the
// prefix built so far: they are the selection whatever the lower bits.  A
// chunk is selected if its score is above tau, or equal to tau and among the
// first k - #{S > tau} equal ones in id order (lower chunk id first).
//
// Index list: with j_w = floor((T - w) / c), the first chunk that reaches the
// recent window [T - w, T), the kept tokens in ascending order are the c
// tokens of every selected chunk j < j_w, followed by the contiguous tail
// [j_w * c, T) if chunk j_w is selected, else [T - w, T) (a selected chunk
// after j_w lies inside the window).  So n = m * c + |tail| with m the number
// of selected chunks before j_w.
//
// Two kernels, one workgroup per (scoring layer, sequence, KV head):
//   select_fast_kernel  512 threads for C <= 16384, 1024 threads for
//     C <= 32768 (token-level chunks of long sequences): scores in registers
//     (chunk j in slot j / NTH of thread j % NTH), counts by wave ballots,
//     one barrier per greedy step, the selected ids compacted into LDS and
//     the index list written position-parallel (coalesced).
//   select_kernel       1024 threads, any C: scores re-read from memory
//     above 32768 chunks; one exclusive scan per tile of 1024 chunks places
//     every kept token.
#include <algorithm>

#include "chunkkv_internal.h"

namespace ckv {
namespace {

constexpr int kWaves = kSelectThreads / 64;

// The key of a score: its fp32 bit pattern, whose unsigned order is the value
// order for scores >= 0.  A pattern with the sign bit set (a negative score,
// -0 or a negative NaN, none of which the score kernels produce) counts as 0,
// so every pattern is below 2^31, the threshold search is exact and exactly
// min(k, C) chunks are selected: the index list never exceeds L_cap.
__device__ __forceinline__ unsigned score_key(unsigned pattern) { return (pattern >> 31) ? 0u : pattern; }
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
    key[i] = (in_regs && j < C) ? score_key(Sb[j]) : 0u;
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
        for (int j = tid; j < C; j += kSelectThreads) cnt += score_key(Sb[j]) >= cand ? 1 : 0;
      }
      return cnt;
    };
    unsigned prefix = 0;
    int n_pre = C;   // #{S_j >= prefix}
    {
      const int t = block_sum(count_ge(1u << 30), red);
      if (t >= kk) {
        prefix = 1u << 30;
        n_pre = t;
      }
    }
    // once exactly k chunks reach the prefix they are the selection: the
    // remaining bits cannot change it (the k-th largest is >= prefix, the
    // (k+1)-th below it), so the search stops there
    for (int bit = 28; bit >= 0 && n_pre != kk; bit -= 2) {
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
          const unsigned kj = score_key(Sb[j]);
          cnt.x += kj >= c1 ? 1 : 0;
          cnt.y += kj >= c2 ? 1 : 0;
          cnt.z += kj >= c3 ? 1 : 0;
        }
      }
      const int3 tot = block_sum3(cnt, red3);
      if (tot.z >= kk) {
        prefix = c3;
        n_pre = tot.z;
      } else if (tot.y >= kk) {
        prefix = c2;
        n_pre = tot.y;
      } else if (tot.x >= kk) {
        prefix = c1;
        n_pre = tot.x;
      }
    }
    tau = prefix;
    int gt = 0;
    if (in_regs) {
#pragma unroll
      for (int i = 0; i < kKPT; ++i) gt += key[i] > tau ? 1 : 0;
    } else {
      for (int j = tid; j < C; j += kSelectThreads) gt += score_key(Sb[j]) > tau ? 1 : 0;
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
      tile(j, j < C ? score_key(Sb[j]) : 0u);
    }
  }
  if (tid == 0) P.lengths[li * P.len_layer_stride + P.len_off[b] + h] = carry_off;
}


// ------------------------------------------------------------ fast path --
#ifndef CKV_SELECT_THREADS
#define CKV_SELECT_THREADS 512
#endif
constexpr int kFastThreads = CKV_SELECT_THREADS;
constexpr int kFastWaves = kFastThreads / 64;
constexpr int kFastMaxKPT = 256 / kFastWaves;   // (slot, wave) tables of at most 256 entries
constexpr int kFastMaxChunks = kFastThreads * kFastMaxKPT;
// 1024 threads with 32 scores each: C <= 32768 (token-level chunks of long sequences)
constexpr int kWideThreads = 1024;
constexpr int kWideMaxChunks = kWideThreads * 32;

__device__ __forceinline__ int wave_count(bool pred) { return __popcll(__ballot(pred)); }

// Lanes below this one with their bit set in `mask`.
__device__ __forceinline__ int lanes_below(unsigned long long mask) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<unsigned>(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<unsigned>(mask), 0));
}

// Exclusive prefix sum, in place, of tab[0 .. E) (E <= 64 * EPL) by wave 0,
// EPL consecutive entries per lane; tab[E] receives the total.  Callers
// barrier before and after.
template <int EPL>
__device__ __forceinline__ void wave0_scan_table(int* tab, int E) {
  if (threadIdx.x >= 64) return;
  const int lane = threadIdx.x;
  const int e0 = EPL * lane;
  int a[EPL];
  int own = 0;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    a[i] = e0 + i < E ? tab[e0 + i] : 0;
    own += a[i];
  }
  int x = own;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  int base = x - own;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    if (e0 + i < E) tab[e0 + i] = base;
    base += a[i];
  }
  if (lane == 63) tab[E] = x;
}

template <int KPT, int NTH>
__global__ __launch_bounds__(NTH) void select_fast_kernel(const SelectParams P) {
  constexpr int kFastThreads = NTH, kFastWaves = NTH / 64;
  constexpr int kEPL = (KPT * kFastWaves + 63) / 64;   // table entries per lane of the wave-0 scans
  static_assert(kEPL <= 8, "(slot, wave) tables of at most 512 entries");
  extern __shared__ int sel_ids[];                  // selected chunk ids < j_w, ascending
  __shared__ int4 red[2][kFastWaves];
  __shared__ int eq_tab[KPT * kFastWaves + 1];
  __shared__ int sel_tab[KPT * kFastWaves + 1];
  __shared__ int jw_selected;
  const int tid = threadIdx.x, wave = tid >> 6;
  constexpr int E = KPT * kFastWaves;               // (slot, wave) table entries

  const int per_layer = P.n_seqs * P.H_kv;
  const int li = blockIdx.x / per_layer;
  const int rest = blockIdx.x - li * per_layer;
  const int b = rest / P.H_kv, h = rest - b * P.H_kv;
  const int T = P.T[b], C = P.C[b], c = P.c, w = P.w;
  const int kk = min(P.kk[b], C);
  const unsigned* Sb = reinterpret_cast<const unsigned*>(P.scores + li * P.score_layer_stride +
                                                         P.score_off[b] + static_cast<int64_t>(h) * C);
  int32_t* idx = P.indices + li * P.index_layer_stride + P.index_off[b] + static_cast<int64_t>(h) * P.L_cap[b];

  unsigned key[KPT];
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const int j = i * kFastThreads + tid;
    key[i] = j < C ? score_key(Sb[j]) : 0u;   // padding 0 is below every candidate (>= 1)
  }

  // greedy threshold; n_ge tracks #{j < C : S_j >= tau}
  unsigned tau = 0;
  int n_ge = C;
  int buf = 0;
  auto wg_sum = [&](int4 v) {
    if ((tid & 63) == 0) red[buf][wave] = v;   // v is uniform across the wave
    __syncthreads();
    int4 t = red[buf][0];
#pragma unroll
    for (int q = 1; q < kFastWaves; ++q) {
      const int4 u = red[buf][q];
      t.x += u.x;
      t.y += u.y;
      t.z += u.z;
    }
    buf ^= 1;   // the next sum writes the other buffer: no second barrier
    return t;
  };
  if (kk > 0 && kk < C) {
    {
      const unsigned c1 = 1u << 30;
      int n1 = 0;
#pragma unroll
      for (int i = 0; i < KPT; ++i) n1 += wave_count(key[i] >= c1);
      const int4 t = wg_sum(make_int4(n1, 0, 0, 0));
      if (t.x >= kk) {
        tau = c1;
        n_ge = t.x;
      }
    }
    // stops once exactly k chunks reach tau (see select_kernel)
    for (int bit = 28; bit >= 0 && n_ge != kk; bit -= 2) {
      const unsigned c1 = tau | (1u << bit), c2 = tau | (2u << bit), c3 = tau | (3u << bit);
      int n1 = 0, n2 = 0, n3 = 0;
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        n1 += wave_count(key[i] >= c1);
        n2 += wave_count(key[i] >= c2);
        n3 += wave_count(key[i] >= c3);
      }
      const int4 t = wg_sum(make_int4(n1, n2, n3, 0));
      if (t.z >= kk) {
        tau = c3;
        n_ge = t.z;
      } else if (t.y >= kk) {
        tau = c2;
        n_ge = t.y;
      } else if (t.x >= kk) {
        tau = c1;
        n_ge = t.x;
      }
    }
  }

  // ties: only when more than k chunks reach tau are the equal ones ranked
  const bool all = kk >= C, none = kk == 0;
  const bool ranked = !all && !none && n_ge > kk;
  int need = 0;
  if (ranked) {
    int gt = 0;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int j = i * kFastThreads + tid;
      const unsigned long long m = __ballot(j < C && key[i] == tau);
      gt += wave_count(key[i] > tau);
      eq_tab[i * kFastWaves + wave] = __popcll(m);
    }
    const int4 t = wg_sum(make_int4(gt, 0, 0, 0));   // its barrier also publishes eq_tab
    need = kk - t.x;
    wave0_scan_table<kEPL>(eq_tab, E);
    __syncthreads();
  }

  const int j_w = (T - w) / c;
  unsigned long long pre[KPT];   // per slot: wave mask of selected chunks before j_w
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const int j = i * kFastThreads + tid;
    bool sel;
    if (j >= C || none) {
      sel = false;
    } else if (all) {
      sel = true;
    } else if (!ranked) {
      sel = key[i] >= tau;
    } else {
      const bool eq = key[i] == tau;
      const unsigned long long m = __ballot(eq);
      sel = key[i] > tau || (eq && eq_tab[i * kFastWaves + wave] + lanes_below(m) < need);
    }
    if (j == j_w) jw_selected = sel ? 1 : 0;
    pre[i] = __ballot(sel && j < j_w);
    sel_tab[i * kFastWaves + wave] = __popcll(pre[i]);
  }
  __syncthreads();
  wave0_scan_table<kEPL>(sel_tab, E);
  __syncthreads();
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    if ((pre[i] >> (tid & 63)) & 1ull)
      sel_ids[sel_tab[i * kFastWaves + wave] + lanes_below(pre[i])] = i * kFastThreads + tid;
  }
  __syncthreads();

  const int m = sel_tab[E];
  const int tail0 = jw_selected ? j_w * c : T - w;
  const int head = m * c;
  const int n = head + (T - tail0);
  for (int p = tid; p < n; p += kFastThreads) {
    int tok;
    if (p < head) {
      const int q = p / c;
      tok = sel_ids[q] * c + (p - q * c);
    } else {
      tok = tail0 + (p - head);
    }
    idx[p] = tok;
  }
  if (tid == 0) P.lengths[li * P.len_layer_stride + P.len_off[b] + h] = n;
}

template <int KPT, int NTH = kFastThreads>
hipError_t launch_fast(const SelectParams& p, int n_blocks, hipStream_t s) {
  // LDS for the selected chunk ids: exactly min(k, C) chunks are selected
  int sel_max = 1;
  for (int b = 0; b < p.n_seqs; ++b) sel_max = std::max(sel_max, std::min(p.kk[b], p.C[b]));
  const size_t lds = static_cast<size_t>(sel_max) * sizeof(int);
  return launch1(select_fast_kernel<KPT, NTH>, dim3(n_blocks), dim3(NTH), lds, s, p);
}

}  // namespace

hipError_t launch_select(const SelectParams& p, int n_blocks, hipStream_t s) {
  int c_max = 1;
  for (int b = 0; b < p.n_seqs; ++b) c_max = p.C[b] > c_max ? p.C[b] : c_max;
  if (c_max <= kFastMaxChunks) {
    if (c_max <= 1 * kFastThreads) return launch_fast<1>(p, n_blocks, s);
    if (c_max <= 2 * kFastThreads) return launch_fast<2>(p, n_blocks, s);
    if (c_max <= 4 * kFastThreads) return launch_fast<4>(p, n_blocks, s);
    if constexpr (kFastMaxKPT >= 8)
      if (c_max <= 8 * kFastThreads) return launch_fast<8>(p, n_blocks, s);
    if constexpr (kFastMaxKPT >= 16)
      if (c_max <= 16 * kFastThreads) return launch_fast<16>(p, n_blocks, s);
    if constexpr (kFastMaxKPT >= 32) return launch_fast<32>(p, n_blocks, s);
  }
  if (c_max <= kWideMaxChunks) return launch_fast<32, kWideThreads>(p, n_blocks, s);
  return launch1(select_kernel, dim3(n_blocks), dim3(kSelectThreads), 0, s, p);
}

}  // namespace ckv
