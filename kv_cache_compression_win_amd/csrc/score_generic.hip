// Generic observe-window score kernel (ChunkKV page, section 4.1, Algorithm 1
// steps 1-3; softmax(QK^T / sqrt(d)) from Kara eq. (1)) for the shapes the
// MFMA path does not cover: fp32 caches, head_dim != 128, chunk sizes without
// a static MFMA layout.  fp32 VALU dot products.
//
// Work item = (layer, sequence, KV head, span of whole chunks); all R = G*w
// window rows are handled by the item.  Each wave takes one row at a time and
// 64 keys per step (one per lane); chunk partials are summed in token order
// by one lane per chunk, so results are deterministic.  Output layout is the
// MFMA kernel's: U[j][r] chunk partials and per-row (m_ref, l) statistics.
#include "chunkkv_internal.h"

namespace ckv {
namespace {

constexpr int kLdsBudget = 64 * 1024;
constexpr int kMaxD = 256;

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Orders this wave's LDS writes before its later LDS reads by other lanes
// (rows are per wave, so a workgroup barrier is not needed or possible here).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

template <typename E>
__device__ __forceinline__ float to_f32(E x);
template <>
__device__ __forceinline__ float to_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ float to_f32<__bf16>(__bf16 x) { return static_cast<float>(x); }

template <typename E>
__global__ __launch_bounds__(kThreads) void score_generic_kernel(const ScoreParams P) {
  extern __shared__ float smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int span_chunks = P.span_chunks;
  const int d = P.d;
  float* u_lds = smem;                                  // [span_chunks][R_pad]
  float* q_lds = u_lds + span_chunks * P.R_pad;         // [4][d]
  float* p_lds = q_lds + 4 * d;                         // [4][64]

  const int li = blockIdx.x / P.items_per_layer;
  int item = blockIdx.x - li * P.items_per_layer;
  int b = 0;
  while (b + 1 < P.n_seqs && item >= P.item0[b + 1]) ++b;
  item -= P.item0[b];
  const int nspan = P.n_span[b];
  const int span = item % nspan;
  const int h = item / nspan;
  const int T = P.T[b], C = P.C[b], c = P.c;
  const int chunk0 = span * span_chunks;
  const int tok_begin = chunk0 * c;
  const int tok_end = min(T, tok_begin + span_chunks * c);
  const int nch = min(span_chunks, C - chunk0);

  for (int e = tid; e < span_chunks * P.R_pad; e += kThreads) u_lds[e] = 0.0f;
  __syncthreads();

  const E* kb = static_cast<const E*>(P.k[li]) + P.tok0[b] * P.kv_st + static_cast<int64_t>(h) * P.kv_sh;
  const E* qb = static_cast<const E*>(P.q[li]) + P.qseq[b] * P.q_ss;
  float* qrow = q_lds + wave * d;
  float* prow = p_lds + wave * 64;

  for (int r = wave; r < P.R; r += 4) {
    const int g = r / P.w, rr = r - g * P.w, hq = h * P.G + g;
    for (int i = lane; i < d; i += 64) qrow[i] = to_f32<E>(qb[rr * P.q_sr + hq * P.q_sh + i]);
    wave_sync();
    float m_ref = -INFINITY;
    for (int t0 = tok_begin; t0 < tok_end; t0 += 64) {
      const int t = t0 + lane;
      const bool ok = t < tok_end;
      float x = 0.0f;
      if (ok) {
        const E* kr = kb + t * P.kv_st;
        for (int i = 0; i < d; ++i) x = fmaf(qrow[i], to_f32<E>(kr[i]), x);
      }
      const float mx = wave_max(ok ? x : -INFINITY);
      if (mx > m_ref + P.rebase_raw) {
        const float f = (m_ref == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f((m_ref - mx) * P.scale);
        for (int j = lane; j < nch; j += 64) u_lds[j * P.R_pad + r] *= f;
        m_ref = mx;
      }
      prow[lane] = ok ? __builtin_amdgcn_exp2f(fmaf(x, P.scale, -m_ref * P.scale)) : 0.0f;
      wave_sync();
      // one lane per chunk touching [t0, t0 + 64), summing in token order
      const int j_first = t0 / c, j_last = (min(t0 + 64, tok_end) - 1) / c;
      const int j = j_first + lane;
      if (j <= j_last) {
        const int a = max(j * c, t0), z = min(j * c + c, min(t0 + 64, tok_end));
        float u = 0.0f;
        for (int t2 = a; t2 < z; ++t2) u += prow[t2 - t0];
        u_lds[(j - chunk0) * P.R_pad + r] += u;
      }
      wave_sync();
    }
    float l = 0.0f;
    for (int j = lane; j < nch; j += 64) l += u_lds[j * P.R_pad + r];
    l = wave_sum(l);
    if (lane == 0)
      P.stats[li * P.st_layer_stride + P.st_off[b] + (static_cast<int64_t>(h) * nspan + span) * P.R_pad + r] =
          make_float2(m_ref, l);
    wave_sync();
  }
  __syncthreads();
  const int64_t row_words = u_row_words(P.R_pad, P.u_packed != 0);
  float* ug = P.U + li * P.u_layer_stride + P.u_off[b] + (static_cast<int64_t>(h) * C + chunk0) * row_words;
  if (P.u_packed) {
    // 24-bit partials: 4 rows in 3 words
    const int q4 = P.R_pad / 4;
    for (int e = tid; e < nch * q4; e += kThreads) {
      const int j = e / q4, q = e - j * q4;
      const float4 v = *reinterpret_cast<const float4*>(u_lds + j * P.R_pad + 4 * q);
      *reinterpret_cast<u32x3u*>(ug + j * row_words + 3 * q) = pack_u24(v.x, v.y, v.z, v.w);
    }
  } else {
    for (int e = tid; e < nch * P.R_pad; e += kThreads) ug[e] = u_lds[e];
  }
}

}  // namespace

int score_generic_span_chunks(int R_pad, int chunk) {
  (void)chunk;
  const int fixed = (4 * kMaxD + 4 * 64) * 4;
  int sc = (kLdsBudget - fixed) / (R_pad * 4);
  return sc < 1 ? 1 : sc;
}

size_t score_generic_lds_bytes(int R_pad, int span_chunks, int d) {
  return (static_cast<size_t>(span_chunks) * R_pad + 4 * d + 4 * 64) * sizeof(float);
}

hipError_t launch_score_generic(const ScoreParams& p, int dtype, int n_blocks, hipStream_t s) {
  const size_t lds = score_generic_lds_bytes(p.R_pad, p.span_chunks, p.d);
  if (dtype == 0) return launch1(score_generic_kernel<float>, dim3(n_blocks), dim3(kThreads), lds, s, p);
  return launch1(score_generic_kernel<__bf16>, dim3(n_blocks), dim3(kThreads), lds, s, p);
}

}  // namespace ckv
