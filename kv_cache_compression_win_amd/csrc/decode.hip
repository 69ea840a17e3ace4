// Decode attention over the compacted cache: the consumer of the compressed
// K'/V' (the ChunkKV page's latency / throughput section decodes over it).
// For every sequence b and query head hq, one new query attends over the n
// kept rows of KV head hq / G with weights softmax(q . k / sqrt(d)) (Kara
// eq. (1)); the output is the weighted sum of the kept value rows.
//
// Split over the rows (flash-decoding style): work item = (sequence, KV head,
// block of kDecRows rows).  An item computes, for up to kDecQ query heads of
// the group at a time, every row's logit (one row per thread, the queries in
// LDS), the block's maximum and sum of exponentials, and the unnormalised
// value sum (consecutive threads read consecutive 16-byte pieces of a value
// row; per-thread partial sums are added over the row subsets through LDS in
// a fixed order).  A second kernel merges the blocks of each query head by
// their (max, sum) and normalises.  Everything is accumulated in fp32 in a
// fixed order: results are deterministic.
#include "decode_internal.h"

namespace ckv {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// 16 bytes of a row as fp32 values: 8 bf16 or 4 fp32 elements.
template <int EB>
__device__ __forceinline__ void widen16(const u32x4 raw, float (&f)[16 / EB]) {
  if constexpr (EB == 4) {
#pragma unroll
    for (int e = 0; e < 4; ++e) f[e] = __uint_as_float(raw[e]);
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[2 * e] = __uint_as_float(raw[e] << 16);
      f[2 * e + 1] = __uint_as_float(raw[e] & 0xffff0000u);
    }
  }
}

template <int EB>
__global__ __launch_bounds__(kThreads) void decode_partial_kernel(const DecodeParams P) {
  constexpr int EPP = 16 / EB;                   // elements per 16-byte piece
  extern __shared__ float smem[];
  const int tid = threadIdx.x;
  const int d = P.d, pieces = P.row_bytes >> 4;
  float* q_l = smem;                             // [kDecQ][d]
  float* p_l = q_l + kDecQ * d;                  // [kDecRows][kDecQ] weights
  float* acc_l = p_l + kDecRows * kDecQ;         // [subsets][kDecQ][d] partial value sums
  __shared__ float red[kThreads / 64][kDecQ];
  __shared__ float mx_l[kDecQ], sum_l[kDecQ];

  int item = blockIdx.x;
  int b = 0;
  while (b + 1 < P.n_seqs && item >= P.item0[b + 1]) ++b;
  item -= P.item0[b];
  const int nblk = P.blocks_per_head[b];
  const int h = item / nblk, blk = item - h * nblk;
  const int n = min(max(P.lengths[P.len_off[b] + h], 0), P.L_cap[b]);
  const int r0 = blk * kDecRows;
  if (r0 >= n) return;                           // the merge reads only blocks below n
  const int rows = min(kDecRows, n - r0);
  const int64_t row0 = P.index_off[b] + static_cast<int64_t>(h) * P.L_cap[b] + r0;
  const char* kb = static_cast<const char*>(P.k) + row0 * P.row_bytes;
  const char* vb = static_cast<const char*>(P.v) + row0 * P.row_bytes;
  const int subsets = kThreads / pieces;         // value-phase row subsets
  const int lane = tid & 63, wave = tid >> 6;

  for (int g0 = 0; g0 < P.G; g0 += kDecQ) {
    const int nq = min(kDecQ, P.G - g0);
    // the queries of this pass, widened to fp32
    for (int e = tid; e < nq * d; e += kThreads) {
      const int g = e / d, j = e - g * d;
      const char* qp = static_cast<const char*>(P.q) +
                       ((static_cast<int64_t>(P.qseq[b]) * P.H_q + h * P.G + g0 + g) * d + j) * EB;
      q_l[g * d + j] = EB == 4 ? *reinterpret_cast<const float*>(qp)
                               : __uint_as_float(static_cast<unsigned>(*reinterpret_cast<const uint16_t*>(qp)) << 16);
    }
    __syncthreads();
    // logits: one row per thread, pieces in order
    float x[kDecQ];
#pragma unroll
    for (int g = 0; g < kDecQ; ++g) x[g] = 0.0f;
    const bool live = tid < rows;
    if (live) {
      const u32x4* kr = reinterpret_cast<const u32x4*>(kb + static_cast<int64_t>(tid) * P.row_bytes);
      for (int pc = 0; pc < pieces; ++pc) {
        float f[EPP];
        widen16<EB>(kr[pc], f);
#pragma unroll
        for (int g = 0; g < kDecQ; ++g) {
          if (g < nq) {
            const float* qg = q_l + g * d + pc * EPP;
#pragma unroll
            for (int e = 0; e < EPP; ++e) x[g] = fmaf(f[e], qg[e], x[g]);
          }
        }
      }
    }
    // block maximum, exponentials and their sum per query head
#pragma unroll
    for (int g = 0; g < kDecQ; ++g) {
      float m = (live && g < nq) ? x[g] * P.inv_sqrt_d : -INFINITY;
      x[g] = m;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
      if (lane == 0) red[wave][g] = m;
    }
    __syncthreads();
    if (tid < kDecQ) {
      float m = red[0][tid];
      for (int w2 = 1; w2 < kThreads / 64; ++w2) m = fmaxf(m, red[w2][tid]);
      mx_l[tid] = m;
    }
    __syncthreads();
#pragma unroll
    for (int g = 0; g < kDecQ; ++g) {
      const float p = (live && g < nq) ? expf(x[g] - mx_l[g]) : 0.0f;
      if (tid < kDecRows) p_l[tid * kDecQ + g] = p;
      float s = p;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
      if (lane == 0) red[wave][g] = s;
    }
    __syncthreads();
    if (tid < kDecQ) {
      float s = red[0][tid];
      for (int w2 = 1; w2 < kThreads / 64; ++w2) s += red[w2][tid];
      sum_l[tid] = s;
    }
    // unnormalised value sums: thread (subset, piece) adds rows subset,
    // subset + subsets, ... of its piece
    const int pc = tid % pieces, sub = tid / pieces;
    float a[kDecQ][EPP];
#pragma unroll
    for (int g = 0; g < kDecQ; ++g)
#pragma unroll
      for (int e = 0; e < EPP; ++e) a[g][e] = 0.0f;
    if (sub < subsets) {
      for (int i = sub; i < rows; i += subsets) {
        float f[EPP];
        widen16<EB>(reinterpret_cast<const u32x4*>(vb + static_cast<int64_t>(i) * P.row_bytes)[pc], f);
#pragma unroll
        for (int g = 0; g < kDecQ; ++g) {
          const float p = p_l[i * kDecQ + g];
#pragma unroll
          for (int e = 0; e < EPP; ++e) a[g][e] = fmaf(p, f[e], a[g][e]);
        }
      }
#pragma unroll
      for (int g = 0; g < kDecQ; ++g)
        if (g < nq)
#pragma unroll
          for (int e = 0; e < EPP; ++e) acc_l[(sub * kDecQ + g) * d + pc * EPP + e] = a[g][e];
    }
    __syncthreads();
    // the block's partial for each query head of the pass: (max, sum, value sums)
    float* part = P.part + ((P.part_off[b] + static_cast<int64_t>(h) * nblk + blk) * P.G + g0) * (d + 2);
    for (int e = tid; e < nq * d; e += kThreads) {
      const int g = e / d, j = e - g * d;
      float s = 0.0f;
      for (int u = 0; u < subsets; ++u) s += acc_l[(u * kDecQ + g) * d + j];
      part[g * (d + 2) + 2 + j] = s;
    }
    if (tid < nq) {
      part[tid * (d + 2)] = mx_l[tid];
      part[tid * (d + 2) + 1] = sum_l[tid];
    }
    __syncthreads();   // before the next pass rewrites q_l, p_l and acc_l
  }
}

// out[b][hq][:] = sum_blocks e^(m_blk - M) o_blk / sum_blocks e^(m_blk - M) l_blk,
// blocks merged in order; zeros when the head keeps no rows.
__global__ __launch_bounds__(kThreads) void decode_merge_kernel(const DecodeParams P) {
  int item = blockIdx.x;   // (sequence, query head)
  const int b = item / P.H_q, hq = item - b * P.H_q;
  const int h = hq / P.G, g = hq - h * P.G;
  const int d = P.d;
  const int n = min(max(P.lengths[P.len_off[b] + h], 0), P.L_cap[b]);
  const int nb = (n + kDecRows - 1) / kDecRows;
  const float* part = P.part + (P.part_off[b] + static_cast<int64_t>(h) * P.blocks_per_head[b]) * P.G * (d + 2) +
                      static_cast<int64_t>(g) * (d + 2);
  const int64_t stride = static_cast<int64_t>(P.G) * (d + 2);
  float M = -INFINITY;
  for (int k = 0; k < nb; ++k) M = fmaxf(M, part[k * stride]);
  float L = 0.0f;
  for (int k = 0; k < nb; ++k) L += expf(part[k * stride] - M) * part[k * stride + 1];
  float* o = P.out + (static_cast<int64_t>(P.qseq[b]) * P.H_q + hq) * d;
  for (int j = threadIdx.x; j < d; j += kThreads) {
    float s = 0.0f;
    for (int k = 0; k < nb; ++k) s += expf(part[k * stride] - M) * part[k * stride + 2 + j];
    o[j] = nb > 0 ? s / L : 0.0f;
  }
}

}  // namespace

size_t decode_lds_bytes(const DecodeParams& p) {
  const int subsets = kThreads / (p.row_bytes >> 4);
  return (static_cast<size_t>(kDecQ) * p.d + static_cast<size_t>(kDecRows) * kDecQ +
          static_cast<size_t>(subsets) * kDecQ * p.d) * sizeof(float);
}

hipError_t launch_decode(const DecodeParams& p, int n_items, int n_heads_out, hipStream_t s) {
  const size_t lds = decode_lds_bytes(p);
  hipError_t e = p.elem_bytes == 4
                     ? launch1(decode_partial_kernel<4>, dim3(n_items), dim3(kThreads), lds, s, p)
                     : launch1(decode_partial_kernel<2>, dim3(n_items), dim3(kThreads), lds, s, p);
  if (e != hipSuccess) return e;
  return launch1(decode_merge_kernel, dim3(n_heads_out), dim3(kThreads), 0, s, p);
}

}  // namespace ckv
