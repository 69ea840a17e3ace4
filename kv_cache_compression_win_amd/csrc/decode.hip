// Decode attention over the compacted cache: the consumer of the compressed
// K'/V' (the ChunkKV page's latency / throughput section decodes over it).
// For every sequence b and query head hq, one new query attends over the n
// kept rows of KV head hq / G with weights softmax(q . k / sqrt(d)) (Kara
// eq. (1)); the output is the weighted sum of the kept value rows.
//
// Split over the rows (flash-decoding style): work item = (sequence, KV head,
// block of rows), walked a step of rows at a time with a running maximum and
// sum of exponentials (the value sums rescaled when the maximum grows).  Per
// step, for up to 8 query heads of the group at a time (4 when the group has
// at most 4, with half the accumulators): every row's logit (a team of lanes
// per key row, partial dot products added by a butterfly inside the team;
// the queries in LDS), the step's weights, and the value sums (consecutive
// lanes read consecutive 16-byte pieces of a value row; the row subsets'
// partial sums are added in a fixed order at the end).  Two partial kernels:
// rows of 16 pieces take one wavefront per item (32-row steps, no workgroup
// barriers), other widths one workgroup per item (64-row steps).  A merge
// kernel combines the blocks of each query head by their (max, sum) and
// normalises.  Everything is accumulated in fp32 in a fixed order: results
// are deterministic.
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

// QN: query heads per pass (4 or 8), a multiple of the waves per workgroup
template <int EB, int QN>
__global__ __launch_bounds__(kThreads, 2) void decode_partial_kernel(const DecodeParams P) {
  constexpr int EPP = 16 / EB;                   // elements per 16-byte piece
  extern __shared__ float smem[];
  const int tid = threadIdx.x;
  const int d = P.d, pieces = P.row_bytes >> 4;
  float* q_l = smem;                             // [QN][d]
  float* p_l = q_l + QN * d;                  // [kDecRows][QN] logits, then weights
  float* acc_l = p_l + kDecRows * QN;         // [subsets][QN][d] partial value sums
  __shared__ float red[kThreads / 64][QN];
  __shared__ float res[QN];

  int item = blockIdx.x;
  int b = 0;
  while (b + 1 < P.n_seqs && item >= P.item0[b + 1]) ++b;
  item -= P.item0[b];
  const int nblk = P.blocks_per_head[b];
  const int h = item / nblk, blk = item - h * nblk;
  const int n = min(max(P.lengths[P.len_off[b] + h], 0), P.L_cap[b]);
  const int rpb = P.rows_per_block[b];
  const int r_begin = blk * rpb;
  if (r_begin >= n) return;                      // the merge reads only blocks below n
  const int r_end = min(n, r_begin + rpb);
  const int64_t head0 = P.index_off[b] + static_cast<int64_t>(h) * P.L_cap[b];
  const int subsets = kThreads / pieces;         // value-phase row subsets
  const int pc_v = tid % pieces, sub = tid / pieces;

  // logits: a team of TS threads per key row (TS = 4, 2 or 1 dividing the
  // piece count), each thread a run of ppt consecutive 16-byte pieces,
  // partial dot products added by a butterfly inside the team; at most one
  // row per thread and step, since kThreads / TS >= kDecRows
  const int TS = (pieces % 4 == 0) ? 4 : ((pieces % 2 == 0) ? 2 : 1);
  const int ppt = pieces / TS, tp = tid % TS, kr_row = tid / TS;
  // register copies of a step's key pieces (the first kKMax of this thread's
  // run) and value pieces (the first kVMax rows of this thread's subset);
  // wider rows read the rest from memory where they are used
  constexpr int kKMax = 4, kVMax = 4;
  auto load_step = [&](int c0, u32x4 (&kr)[kKMax], u32x4 (&vr)[kVMax]) {
    const int rows = min(kDecRows, r_end - c0);
    const char* kb = static_cast<const char*>(P.k) + (head0 + c0) * P.row_bytes;
    const char* vb = static_cast<const char*>(P.v) + (head0 + c0) * P.row_bytes;
    if (kr_row < rows) {
      const u32x4* row = reinterpret_cast<const u32x4*>(kb + static_cast<int64_t>(kr_row) * P.row_bytes);
#pragma unroll
      for (int k = 0; k < kKMax; ++k)
        if (k < ppt) kr[k] = row[tp * ppt + k];
    }
    if (sub < subsets) {
#pragma unroll
      for (int t = 0; t < kVMax; ++t) {
        const int i = sub + t * subsets;
        if (i < rows) vr[t] = reinterpret_cast<const u32x4*>(vb + static_cast<int64_t>(i) * P.row_bytes)[pc_v];
      }
    }
  };

  for (int g0 = 0; g0 < P.G; g0 += QN) {
    const int nq = min(QN, P.G - g0);
    // the first step's rows are requested before the queries, so the two
    // round trips overlap
    u32x4 kc[kKMax], vc[kVMax], kn[kKMax], vn[kVMax];
    load_step(r_begin, kc, vc);
    // the queries of this pass, widened to fp32
    for (int e = tid; e < nq * d; e += kThreads) {
      const int g = e / d, j = e - g * d;
      const char* qp = static_cast<const char*>(P.q) +
                       ((static_cast<int64_t>(P.qseq[b]) * P.H_q + h * P.G + g0 + g) * d + j) * EB;
      q_l[g * d + j] = EB == 4 ? *reinterpret_cast<const float*>(qp)
                               : __uint_as_float(static_cast<unsigned>(*reinterpret_cast<const uint16_t*>(qp)) << 16);
    }
    __syncthreads();
    // running maximum and sum of exponentials of the block's rows so far, and
    // this thread's unnormalised value sums (rescaled when the maximum grows)
    float m_run[QN], l_run[QN], a[QN][EPP];
#pragma unroll
    for (int g = 0; g < QN; ++g) {
      m_run[g] = -INFINITY;
      l_run[g] = 0.0f;
#pragma unroll
      for (int e = 0; e < EPP; ++e) a[g][e] = 0.0f;
    }
    for (int c0 = r_begin; c0 < r_end; c0 += kDecRows) {
      const int rows = min(kDecRows, r_end - c0);
      const bool more = c0 + kDecRows < r_end;
      if (more) load_step(c0 + kDecRows, kn, vn);   // next step's rows in flight during this one
      const char* kb = static_cast<const char*>(P.k) + (head0 + c0) * P.row_bytes;
      const char* vb = static_cast<const char*>(P.v) + (head0 + c0) * P.row_bytes;
      {
        float x[QN];
#pragma unroll
        for (int g = 0; g < QN; ++g) x[g] = 0.0f;
        if (kr_row < rows) {
          const u32x4* kr = reinterpret_cast<const u32x4*>(kb + static_cast<int64_t>(kr_row) * P.row_bytes);
          auto dot = [&](const u32x4 raw, int pc) {
            float f[EPP];
            widen16<EB>(raw, f);
#pragma unroll
            for (int g = 0; g < QN; ++g) {
              if (g < nq) {
                const float* qg = q_l + g * d + pc * EPP;
#pragma unroll
                for (int e = 0; e < EPP; ++e) x[g] = fmaf(f[e], qg[e], x[g]);
              }
            }
          };
#pragma unroll
          for (int k = 0; k < kKMax; ++k)
            if (k < ppt) dot(kc[k], tp * ppt + k);
          for (int k = kKMax; k < ppt; ++k) dot(kr[tp * ppt + k], tp * ppt + k);
        }
        for (int o = TS >> 1; o > 0; o >>= 1)
#pragma unroll
          for (int g = 0; g < QN; ++g) x[g] += __shfl_xor(x[g], o, 64);
        if (tp == 0 && kr_row < rows)
#pragma unroll
          for (int g = 0; g < QN; ++g) p_l[kr_row * QN + g] = x[g] * P.inv_sqrt_d;
      }
      __syncthreads();
      // each wave takes query heads wave, wave + 4 (one lane per row of the
      // step): the step's maximum, the new running maximum, the weights and
      // their sum, published through LDS
      {
        const int lane = tid & 63, wave = tid >> 6;
        const bool live = lane < rows;
#pragma unroll
        for (int gg = 0; gg < QN / (kThreads / 64); ++gg) {
          const int g = wave + gg * (kThreads / 64);
          const float x = (live && g < nq) ? p_l[lane * QN + g] : -INFINITY;
          float m = x;
#pragma unroll
          for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
          float mr = m_run[0];   // m_run[g] without indexing the register array by a lane-varying value
#pragma unroll
          for (int gi = 1; gi < QN; ++gi) mr = gi == g ? m_run[gi] : mr;
          const float mn = fmaxf(mr, m);
          const float pw = (live && g < nq) ? expf(x - mn) : 0.0f;
          p_l[lane * QN + g] = pw;
          float sc = pw;
#pragma unroll
          for (int o = 32; o > 0; o >>= 1) sc += __shfl_xor(sc, o, 64);
          if (lane == 0) {
            res[g] = mn;
            red[0][g] = sc;
          }
        }
      }
      __syncthreads();
      float f[QN];
#pragma unroll
      for (int g = 0; g < QN; ++g) {
        const float mn = res[g];
        f[g] = m_run[g] == -INFINITY ? 0.0f : expf(m_run[g] - mn);
        l_run[g] = l_run[g] * f[g] + red[0][g];
        m_run[g] = mn;
      }
      // value sums: thread (subset, piece) adds rows subset, subset + subsets, ...
      if (sub < subsets) {
#pragma unroll
        for (int g = 0; g < QN; ++g)
#pragma unroll
          for (int e = 0; e < EPP; ++e) a[g][e] *= f[g];
#pragma unroll
        for (int t = 0; t < kVMax; ++t) {
          const int i = sub + t * subsets;
          if (i < rows) {
            float fv[EPP];
            widen16<EB>(vc[t], fv);
#pragma unroll
            for (int g = 0; g < QN; ++g) {
              const float p = p_l[i * QN + g];
#pragma unroll
              for (int e = 0; e < EPP; ++e) a[g][e] = fmaf(p, fv[e], a[g][e]);
            }
          }
        }
        for (int i = sub + kVMax * subsets; i < rows; i += subsets) {   // wide rows: fewer subsets
          float fv[EPP];
          widen16<EB>(reinterpret_cast<const u32x4*>(vb + static_cast<int64_t>(i) * P.row_bytes)[pc_v], fv);
#pragma unroll
          for (int g = 0; g < QN; ++g) {
            const float p = p_l[i * QN + g];
#pragma unroll
            for (int e = 0; e < EPP; ++e) a[g][e] = fmaf(p, fv[e], a[g][e]);
          }
        }
      }
      __syncthreads();   // p_l, res and red are rewritten by the next step
      if (more) {
#pragma unroll
        for (int k = 0; k < kKMax; ++k) kc[k] = kn[k];
#pragma unroll
        for (int t = 0; t < kVMax; ++t) vc[t] = vn[t];
      }
    }
    if (sub < subsets)
#pragma unroll
      for (int g = 0; g < QN; ++g)
        if (g < nq)
#pragma unroll
          for (int e = 0; e < EPP; ++e) acc_l[(sub * QN + g) * d + pc_v * EPP + e] = a[g][e];
    __syncthreads();
    // the block's partial for each query head of the pass: (max, sum, value sums)
    float* part = P.part + ((P.part_off[b] + static_cast<int64_t>(h) * nblk + blk) * P.G + g0) * (d + kPartHead);
    for (int e = tid; e < nq * d; e += kThreads) {
      const int g = e / d, j = e - g * d;
      float s = 0.0f;
      for (int u = 0; u < subsets; ++u) s += acc_l[(u * QN + g) * d + j];
      part[g * (d + kPartHead) + kPartHead + j] = s;
    }
    if (tid < nq) {
      part[tid * (d + kPartHead)] = m_run[tid];
      part[tid * (d + kPartHead) + 1] = l_run[tid];
    }
    __syncthreads();   // before the next pass rewrites q_l, p_l and acc_l
  }
}

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// One wavefront per work item, for rows of 16 pieces (EPP elements each).
// Step of kWaveRows = 32 rows, each step's keys and values requested during
// the previous step:
//   logits  lane = (row team_row of each 16-row half, piece run tp): 4 lanes
//           per row, 4 pieces each, dot products added by a butterfly (xor 1,
//           2), so every lane of a team holds its row's logit;
//   weights max and sum over the step by butterflies across the teams (xor
//           4 .. 32), running max and sum updated in every lane alike;
//   values  lane = (row subset vs of 4, piece pc of 16): rows vs, vs + 4, ...
//           with their weights read from the wave's LDS.
// The four subsets are added by butterflies (xor 16, 32) at the end.
template <int EB, int QN>
__global__ __launch_bounds__(kThreads) void decode_wave_kernel(const DecodeParams P) {
  constexpr int EPP = 16 / EB, D = kWavePieces * EPP, kW = kThreads / 64;
  constexpr int kHalf = kWaveRows / 2;                 // rows per logit half-step (64 lanes / 4)
  constexpr int kVRows = kWaveRows / 4;                // value rows per lane and step
  __shared__ float q_s[kW][QN * D];
  __shared__ float p_s[kW][kWaveRows * QN];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int item = blockIdx.x * kW + wave;
  if (item >= P.item0[P.n_seqs]) return;               // the wave's item is past the last
  int b = 0;
  while (b + 1 < P.n_seqs && item >= P.item0[b + 1]) ++b;
  item -= P.item0[b];
  const int nblk = P.blocks_per_head[b];
  const int h = item / nblk, blk = item - h * nblk;
  const int n = min(max(P.lengths[P.len_off[b] + h], 0), P.L_cap[b]);
  const int rpb = P.rows_per_block[b];
  const int r_begin = blk * rpb;
  if (r_begin >= n) return;                            // the merge reads only blocks below n
  const int r_end = min(n, r_begin + rpb);
  const int64_t head0 = P.index_off[b] + static_cast<int64_t>(h) * P.L_cap[b];
  const int team_row = lane >> 2, tp = lane & 3;
  const int vs = lane >> 4, pc = lane & 15;
  float* qw = q_s[wave];
  float* pw = p_s[wave];
  const u32x4* kbase = reinterpret_cast<const u32x4*>(static_cast<const char*>(P.k) + head0 * (16 * kWavePieces));
  const u32x4* vbase = reinterpret_cast<const u32x4*>(static_cast<const char*>(P.v) + head0 * (16 * kWavePieces));

  auto load_k = [&](int c0, u32x4 (&kr)[2][4]) {
    const int rows = min(kWaveRows, r_end - c0);
#pragma unroll
    for (int hs = 0; hs < 2; ++hs) {
      const int r = team_row + hs * kHalf;
      if (r < rows) {
#pragma unroll
        for (int k = 0; k < 4; ++k) kr[hs][k] = kbase[static_cast<int64_t>(c0 + r) * kWavePieces + tp * 4 + k];
      }
    }
  };
  auto load_v = [&](int c0, u32x4 (&vr)[kVRows]) {
    const int rows = min(kWaveRows, r_end - c0);
#pragma unroll
    for (int t = 0; t < kVRows; ++t) {
      const int i = vs + 4 * t;
      if (i < rows) vr[t] = vbase[static_cast<int64_t>(c0 + i) * kWavePieces + pc];
    }
  };

  for (int g0 = 0; g0 < P.G; g0 += QN) {
    const int nq = min(QN, P.G - g0);
    // one register copy of a step's keys and values: the next step's keys
    // are requested as soon as this step's logits are formed, its values as
    // soon as this step's value sums are, so each load has a phase to land in
    u32x4 kc[2][4], vc[kVRows];
    load_k(r_begin, kc);
    load_v(r_begin, vc);
    // the pass's queries: nq rows of 16 pieces, all requested at once, then
    // widened into the wave's LDS
    {
      const u32x4* qb = reinterpret_cast<const u32x4*>(
          static_cast<const char*>(P.q) + (static_cast<int64_t>(P.qseq[b]) * P.H_q + h * P.G + g0) * (D * EB));
      constexpr int kQPer = QN * kWavePieces / 64;
      u32x4 qr[kQPer];
#pragma unroll
      for (int t = 0; t < kQPer; ++t)
        if (lane + 64 * t < nq * kWavePieces) qr[t] = qb[lane + 64 * t];
#pragma unroll
      for (int t = 0; t < kQPer; ++t) {
        const int u = lane + 64 * t;
        if (u < nq * kWavePieces) {
          float f[EPP];
          widen16<EB>(qr[t], f);
#pragma unroll
          for (int e = 0; e < EPP; ++e) qw[u * EPP + e] = f[e];
        }
      }
    }
    wave_sync();
    float m_run[QN], l_run[QN], a[QN][EPP];
#pragma unroll
    for (int g = 0; g < QN; ++g) {
      m_run[g] = -INFINITY;
      l_run[g] = 0.0f;
#pragma unroll
      for (int e = 0; e < EPP; ++e) a[g][e] = 0.0f;
    }
    for (int c0 = r_begin; c0 < r_end; c0 += kWaveRows) {
      const int rows = min(kWaveRows, r_end - c0);
      const bool more = c0 + kWaveRows < r_end;
      float x[2][QN];
#pragma unroll
      for (int hs = 0; hs < 2; ++hs) {
#pragma unroll
        for (int g = 0; g < QN; ++g) x[hs][g] = 0.0f;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          float f[EPP];
          widen16<EB>(kc[hs][k], f);
          const int off = (tp * 4 + k) * EPP;
#pragma unroll
          for (int g = 0; g < QN; ++g) {
            if (g < nq) {
#pragma unroll
              for (int e = 0; e < EPP; ++e) x[hs][g] = fmaf(f[e], qw[g * D + off + e], x[hs][g]);
            }
          }
        }
      }
      if (more) load_k(c0 + kWaveRows, kc);
      float fs[QN];
#pragma unroll
      for (int g = 0; g < QN; ++g) {
#pragma unroll
        for (int hs = 0; hs < 2; ++hs) {
          x[hs][g] += __shfl_xor(x[hs][g], 1, 64);
          x[hs][g] += __shfl_xor(x[hs][g], 2, 64);
          x[hs][g] = (team_row + hs * kHalf < rows) ? x[hs][g] * P.inv_sqrt_d : -INFINITY;
        }
        float m = fmaxf(x[0][g], x[1][g]);
#pragma unroll
        for (int o = 4; o < 64; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
        const float mn = fmaxf(m_run[g], m);
        const float p0 = expf(x[0][g] - mn), p1 = expf(x[1][g] - mn);
        float sc = p0 + p1;
#pragma unroll
        for (int o = 4; o < 64; o <<= 1) sc += __shfl_xor(sc, o, 64);
        fs[g] = m_run[g] == -INFINITY ? 0.0f : expf(m_run[g] - mn);
        l_run[g] = l_run[g] * fs[g] + sc;
        m_run[g] = mn;
        if (tp == 0) {
          pw[team_row * QN + g] = p0;
          pw[(team_row + kHalf) * QN + g] = p1;
        }
      }
      wave_sync();
#pragma unroll
      for (int g = 0; g < QN; ++g)
#pragma unroll
        for (int e = 0; e < EPP; ++e) a[g][e] *= fs[g];
#pragma unroll
      for (int t = 0; t < kVRows; ++t) {
        const int i = vs + 4 * t;
        if (i < rows) {
          float fv[EPP];
          widen16<EB>(vc[t], fv);
#pragma unroll
          for (int g = 0; g < QN; ++g) {
            const float p = pw[i * QN + g];
#pragma unroll
            for (int e = 0; e < EPP; ++e) a[g][e] = fmaf(p, fv[e], a[g][e]);
          }
        }
      }
      if (more) load_v(c0 + kWaveRows, vc);
      wave_sync();   // pw is rewritten by the next step
    }
    // the four row subsets of each piece, added in a fixed order
    float* part = P.part + ((P.part_off[b] + static_cast<int64_t>(h) * nblk + blk) * P.G + g0) * (D + kPartHead);
#pragma unroll
    for (int g = 0; g < QN; ++g) {
#pragma unroll
      for (int e = 0; e < EPP; ++e) {
        a[g][e] += __shfl_xor(a[g][e], 16, 64);
        a[g][e] += __shfl_xor(a[g][e], 32, 64);
      }
      if (g < nq && lane < 16) {
#pragma unroll
        for (int e = 0; e < EPP; ++e) part[g * (D + kPartHead) + kPartHead + pc * EPP + e] = a[g][e];
      }
      if (g < nq && lane == 16) {
        part[g * (D + kPartHead)] = m_run[g];
        part[g * (D + kPartHead) + 1] = l_run[g];
      }
    }
    wave_sync();   // before the next pass rewrites qw
  }
}

// out[b][hq][:] = sum_blocks e^(m_blk - M) o_blk / sum_blocks e^(m_blk - M) l_blk
// over the blocks that hold rows; zeros when the head keeps no rows.  One
// workgroup per query head: the blocks' weights are formed in parallel (into
// LDS), then thread (block lane, 16-byte group of the output) adds every
// KB-th block's value sums of that group and the KB lanes are added in order.
__global__ __launch_bounds__(kThreads) void decode_merge_kernel(const DecodeParams P) {
  extern __shared__ float w_l[];   // [blocks_per_head] weights (padded to 4), then [KB][d] block-lane sums
  __shared__ float red[kThreads / 64];
  __shared__ float bc;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int item = blockIdx.x;     // (sequence, query head)
  const int b = item / P.H_q, hq = item - b * P.H_q;
  const int h = hq / P.G, g = hq - h * P.G;
  const int d = P.d;
  const int n = min(max(P.lengths[P.len_off[b] + h], 0), P.L_cap[b]);
  const int nb = (n + P.rows_per_block[b] - 1) / P.rows_per_block[b];
  float* o = P.out + (static_cast<int64_t>(P.qseq[b]) * P.H_q + hq) * d;
  if (nb == 0) {
    for (int j = tid; j < d; j += kThreads) o[j] = 0.0f;
    return;
  }
  const float* part = P.part + (P.part_off[b] + static_cast<int64_t>(h) * P.blocks_per_head[b]) * P.G * (d + kPartHead) +
                      static_cast<int64_t>(g) * (d + kPartHead);
  const int64_t stride = static_cast<int64_t>(P.G) * (d + kPartHead);
  // M: the largest block maximum
  float m = -INFINITY;
  for (int k = tid; k < nb; k += kThreads) m = fmaxf(m, part[k * stride]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  if (lane == 0) red[wave] = m;
  __syncthreads();
  if (tid == 0) {
    float x = red[0];
    for (int w2 = 1; w2 < kThreads / 64; ++w2) x = fmaxf(x, red[w2]);
    bc = x;
  }
  __syncthreads();
  const float M = bc;
  // block weights e^(m_blk - M) and L = sum_blocks weight * l_blk
  float l = 0.0f;
  for (int k = tid; k < nb; k += kThreads) {
    const float wk = expf(part[k * stride] - M);
    w_l[k] = wk;
    l += wk * part[k * stride + 1];
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) l += __shfl_xor(l, off, 64);
  __syncthreads();
  if (lane == 0) red[wave] = l;
  __syncthreads();
  if (tid == 0) {
    float x = red[0];
    for (int w2 = 1; w2 < kThreads / 64; ++w2) x += red[w2];
    bc = x;
  }
  __syncthreads();
  const float L = bc;
  // value sums: thread (block lane kb, 16-byte group j4) adds blocks kb,
  // kb + KB, ... of elements 4*j4 .. 4*j4 + 3 (records are 16-byte aligned),
  // then the KB block lanes are added in order
  const int d4 = d >> 2;
  const int KB = max(1, kThreads / d4);
  float4* sub_l = reinterpret_cast<float4*>(w_l + ((P.blocks_per_head[b] + 3) & ~3));
  if (tid < KB * d4) {
    const int kb = tid / d4, j4 = tid - kb * d4;
    const float4* pv = reinterpret_cast<const float4*>(part + kPartHead) + j4;
    const int64_t stride4 = stride >> 2;
    float4 s = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    int k = kb;
    constexpr int kInFlight = 8;             // independent loads in flight per thread
    for (; k + (kInFlight - 1) * KB < nb; k += kInFlight * KB) {
      float4 x[kInFlight];
#pragma unroll
      for (int u = 0; u < kInFlight; ++u) x[u] = pv[(k + u * KB) * stride4];
#pragma unroll
      for (int u = 0; u < kInFlight; ++u) {
        const float wk = w_l[k + u * KB];
        s.x = fmaf(wk, x[u].x, s.x);
        s.y = fmaf(wk, x[u].y, s.y);
        s.z = fmaf(wk, x[u].z, s.z);
        s.w = fmaf(wk, x[u].w, s.w);
      }
    }
    for (; k < nb; k += KB) {
      const float4 x = pv[k * stride4];
      const float wk = w_l[k];
      s.x = fmaf(wk, x.x, s.x);
      s.y = fmaf(wk, x.y, s.y);
      s.z = fmaf(wk, x.z, s.z);
      s.w = fmaf(wk, x.w, s.w);
    }
    sub_l[kb * d4 + j4] = s;
  }
  __syncthreads();
  const float* sub_f = reinterpret_cast<const float*>(sub_l);
  for (int j = tid; j < d; j += kThreads) {
    float s = 0.0f;
    for (int kb = 0; kb < KB; ++kb) s += sub_f[kb * d + j];
    o[j] = s / L;
  }
}

}  // namespace

hipError_t launch_merge(const DecodeParams& p, int n_heads_out, hipStream_t s);

size_t decode_lds_bytes(const DecodeParams& p) {
  if (decode_wave_path(p.row_bytes)) return 0;     // static LDS only
  const int subsets = kThreads / (p.row_bytes >> 4);
  const size_t qn = p.G <= 4 ? 4 : kDecQ;   // query heads per pass of the launched variant
  return (qn * p.d + static_cast<size_t>(kDecRows) * qn + static_cast<size_t>(subsets) * qn * p.d) * sizeof(float);
}

hipError_t launch_decode(const DecodeParams& p, int n_items, int n_heads_out, hipStream_t s) {
  const bool q4 = p.G <= 4;
  if (decode_wave_path(p.row_bytes)) {
    const int n_wg = (n_items + kThreads / 64 - 1) / (kThreads / 64);
    void (*wk)(DecodeParams) = p.elem_bytes == 4 ? (q4 ? decode_wave_kernel<4, 4> : decode_wave_kernel<4, kDecQ>)
                                                : (q4 ? decode_wave_kernel<2, 4> : decode_wave_kernel<2, kDecQ>);
    hipError_t e = launch1(wk, dim3(n_wg), dim3(kThreads), 0, s, p);
    if (e != hipSuccess) return e;
    return launch_merge(p, n_heads_out, s);
  }
  const size_t lds = decode_lds_bytes(p);
  // a group of at most 4 query heads takes the variant with half the value
  // accumulators (fewer registers, more workgroups per CU)
  void (*kern)(DecodeParams) = p.elem_bytes == 4 ? (q4 ? decode_partial_kernel<4, 4> : decode_partial_kernel<4, kDecQ>)
                                                  : (q4 ? decode_partial_kernel<2, 4> : decode_partial_kernel<2, kDecQ>);
  hipError_t e = launch1(kern, dim3(n_items), dim3(kThreads), lds, s, p);
  if (e != hipSuccess) return e;
  return launch_merge(p, n_heads_out, s);
}

hipError_t launch_merge(const DecodeParams& p, int n_heads_out, hipStream_t s) {
  int nbh = 1;
  for (int i = 0; i < p.n_seqs; ++i) nbh = nbh > p.blocks_per_head[i] ? nbh : p.blocks_per_head[i];
  const int KB = kThreads / (p.d / 4) > 1 ? kThreads / (p.d / 4) : 1;
  const size_t merge_lds = (static_cast<size_t>((nbh + 3) & ~3) + static_cast<size_t>(KB) * p.d) * sizeof(float);
  return launch1(decode_merge_kernel, dim3(n_heads_out), dim3(kThreads), merge_lds, s, p);
}

}  // namespace ckv
