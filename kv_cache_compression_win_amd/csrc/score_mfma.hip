// Fused observe-window score kernel for bf16 caches with head_dim 128 on
// gfx950 (CDNA4): ChunkKV page, section 4.1, Algorithm 1 steps 1-3, with the
// softmax(QK^T / sqrt(d)) of Kara eq. (1).
//
// Work item = (layer, sequence, KV head, 128-row block of the G*w window
// rows, span of whole chunks).  Persistent workgroups walk contiguous ranges
// of items; keys are streamed HBM -> VGPR -> LDS once, one group ahead.
// Logits come from v_mfma_f32_32x32x16_bf16 with the KEYS as the A operand (32 token slots x 16 dims) and the window queries as B (16 dims x
// 32 query rows), so in the 32x32 fp32 result each lane owns one query row
// and 16 token slots.  Token slots are permuted so that each lane half holds
// CPH whole chunks: the chunk sums are then straight-line adds fixed at
// compile time for each chunk size.  The logits never leave registers: the
// kernel writes, per query row, the chunk partials
//   U[j][r] = sum_{t in chunk j} 2^((x_rt - m_r) * log2(e)/sqrt(d))
// and (m_r, l_r = sum over the span) for the log-sum-exp combine.
#include "chunkkv_internal.h"

namespace ckv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kD = 128;              // head_dim of this path
constexpr int kKSteps = kD / 16;     // MFMA k-steps per logit tile
constexpr int kPieces = kD / 8;      // 16-byte pieces per bf16 key row

// Number of 32-slot MFMA tiles per group for chunk size c: the least padding
// (slots per lane half = 16 * nt, holding floor(16 * nt / c) whole chunks),
// ties to the smaller tile count, at most kMaxTiles tiles.
constexpr int pick_tiles(int c) {
  int best = 0, best_waste_num = 1, best_waste_den = 0;  // waste = num/den
  for (int nt = 1; nt <= kMaxTiles; ++nt) {
    const int cph = 16 * nt / c;
    if (cph == 0) continue;
    const int num = 16 * nt - cph * c, den = 16 * nt;
    if (best == 0 || num * best_waste_den < best_waste_num * den) {
      best = nt;
      best_waste_num = num;
      best_waste_den = den;
    }
  }
  return best;
}

template <int CC>
struct Geo {
  static constexpr int NT = pick_tiles(CC);
  static_assert(NT >= 1, "chunk size has no static MFMA layout");
  static constexpr int CPH = 16 * NT / CC;         // chunks per lane half per group
  static constexpr int HALF_TOK = CPH * CC;        // tokens per lane half per group
  static constexpr int GROUP_CHUNKS = 2 * CPH;
  static constexpr int GROUP_TOK = 2 * HALF_TOK;
  static constexpr int GPS = (kSpanTarget / GROUP_CHUNKS) > 0 ? (kSpanTarget / GROUP_CHUNKS) : 1;
  static constexpr int SPAN_CHUNKS = GROUP_CHUNKS * GPS;
  static constexpr int LOADS = NT * 32 * kPieces / kThreads;  // uint4 per thread per group
};

__device__ __forceinline__ float shfl_xor32(float v) { return __shfl_xor(v, 32, 64); }

// Softmax pieces of one group for this lane's row: rebase the reference if the
// group's maximum exceeds it by more than 2^kRebaseLog2, then write the chunk
// partials of this lane half to LDS.  Slots past the end of the sequence are
// masked to -inf (exp2 gives 0) before anything else.
template <int CC>
__device__ __forceinline__ void group_softmax(f32x16 (&acc)[Geo<CC>::NT], bool full, int nvalid,
                                              float scale, float rebase_raw, float& m_ref,
                                              float& l_acc, float* u_row, int gi) {
  using G = Geo<CC>;
  if (!full) {
#pragma unroll
    for (int tau = 0; tau < G::NT; ++tau)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int lam = 16 * tau + v;
        if (lam < G::HALF_TOK) acc[tau][v] = lam < nvalid ? acc[tau][v] : -INFINITY;
      }
  }
  float mx = -INFINITY;
#pragma unroll
  for (int tau = 0; tau < G::NT; ++tau)
#pragma unroll
    for (int v = 0; v < 16; ++v)
      if (16 * tau + v < G::HALF_TOK) mx = fmaxf(mx, acc[tau][v]);
  mx = fmaxf(mx, shfl_xor32(mx));
  if (mx > m_ref + rebase_raw) {
    const float f = (m_ref == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f((m_ref - mx) * scale);
    for (int gg = 0; gg < gi; ++gg)
#pragma unroll
      for (int q = 0; q < G::CPH; ++q) u_row[(gg * G::GROUP_CHUNKS + q) * kMfmaRows] *= f;
    l_acc *= f;
    m_ref = mx;
  }
  const float mrs = m_ref * scale;
  float* dst = u_row + gi * G::GROUP_CHUNKS * kMfmaRows;
#pragma unroll
  for (int q = 0; q < G::CPH; ++q) {
    float u = 0.0f;
#pragma unroll
    for (int e = 0; e < CC; ++e) {
      const int lam = q * CC + e;
      u += __builtin_amdgcn_exp2f(fmaf(acc[lam >> 4][lam & 15], scale, -mrs));
    }
    dst[q * kMfmaRows] = u;
    l_acc += u;
  }
}

// One work item: (layer, sequence, KV head, row block, span of whole chunks).
struct Item {
  int li, b, h, rb, span, nspan, C, tok_begin, tok_end, ngroups;
};

template <int CC>
__device__ __forceinline__ Item decode_item(const ScoreParams& P, int flat) {
  using G = Geo<CC>;
  Item it;
  it.li = flat / P.items_per_layer;
  int item = flat - it.li * P.items_per_layer;
  int b = 0;
  while (b + 1 < P.n_seqs && item >= P.item0[b + 1]) ++b;
  item -= P.item0[b];
  it.b = b;
  it.nspan = P.n_span[b];
  it.span = item % it.nspan;
  const int hr = item / it.nspan;
  it.rb = hr % P.n_rb;
  it.h = hr / P.n_rb;
  it.C = P.C[b];
  it.tok_begin = it.span * G::SPAN_CHUNKS * CC;
  it.tok_end = min(P.T[b], it.tok_begin + G::SPAN_CHUNKS * CC);
  it.ngroups = (it.tok_end - it.tok_begin + G::GROUP_TOK - 1) / G::GROUP_TOK;
  return it;
}

// Persistent workgroups: workgroup w takes the contiguous range of work items
// [w*N/W, (w+1)*N/W) (consecutive spans of the same head, so the window-query
// fragments change rarely) and keeps one group of keys in flight across item
// boundaries: while group g is multiplied and reduced, group g+1 -- of the
// same item or of the next one -- is already being loaded.
template <int CC>
__global__ __launch_bounds__(kThreads, 2) void score_mfma_kernel(const ScoreParams P) {
  using G = Geo<CC>;
  __shared__ uint4 k_lds[G::NT * 32 * kPieces];
  __shared__ float u_lds[G::SPAN_CHUNKS * kMfmaRows];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, ho = lane >> 5;
  const int total = P.n_layers * P.items_per_layer;
  const int lo = static_cast<int>(static_cast<int64_t>(blockIdx.x) * total / P.n_workers);
  const int hi = static_cast<int>(static_cast<int64_t>(blockIdx.x + 1) * total / P.n_workers);
  if (lo >= hi) return;

  // window-query fragments (B operand) of this wave's 32 rows; rows >= R are zero
  bf16x8 bq[kKSteps];
  auto load_q = [&](const Item& it) {
    const int r = it.rb * kMfmaRows + wave * 32 + n;
    if (r < P.R) {
      const int g = r / P.w;
      const int rr = r - g * P.w;
      const int hq = it.h * P.G + g;
      const __bf16* qp = static_cast<const __bf16*>(P.q[it.li]) + P.qseq[it.b] * P.q_ss + rr * P.q_sr +
                         hq * P.q_sh + ho * (kD / 2);
#pragma unroll
      for (int s = 0; s < kKSteps; ++s) bq[s] = *reinterpret_cast<const bf16x8*>(qp + 8 * s);
    } else {
#pragma unroll
      for (int s = 0; s < kKSteps; ++s) bq[s] = bf16x8{};
    }
  };

  // key streaming: slot (tile tau, row i) <-> token of lane half (i/4)%2.
  // Rows past the end of the span are loaded clamped (their logits are masked).
  uint4 regs[G::LOADS];
  const int64_t st_bytes = P.kv_st * 2;
  auto load_group = [&](const Item& it, int gi) {
    const char* kbase = static_cast<const char*>(P.k[it.li]) +
                        (P.tok0[it.b] * P.kv_st + static_cast<int64_t>(it.h) * P.kv_sh) * 2;
    const int gtok0 = it.tok_begin + gi * G::GROUP_TOK;
#pragma unroll
    for (int x = 0; x < G::LOADS; ++x) {
      const int gp = x * kThreads + tid;
      const int sr = gp / kPieces, p = gp % kPieces;
      const int tau = sr >> 5, i = sr & 31;
      const int lam = 16 * tau + 4 * (i >> 3) + (i & 3);
      const int tok = min(gtok0 + ((i >> 2) & 1) * G::HALF_TOK + lam, it.tok_end - 1);
      if (lam < G::HALF_TOK)
        regs[x] = *reinterpret_cast<const uint4*>(kbase + tok * st_bytes + p * 16);
      else
        regs[x] = make_uint4(0u, 0u, 0u, 0u);
    }
  };
  auto store_group = [&]() {
#pragma unroll
    for (int x = 0; x < G::LOADS; ++x) {
      const int gp = x * kThreads + tid;
      const int sr = gp / kPieces, p = gp % kPieces;
      k_lds[sr * kPieces + (p ^ (sr & 15))] = regs[x];
    }
  };
  // per-row span statistics and chunk partials of a finished item
  auto flush = [&](const Item& it, float m_ref, float l_acc) {
    const int r = it.rb * kMfmaRows + wave * 32 + n;
    const float l_row = l_acc + shfl_xor32(l_acc);
    if (ho == 0 && r < P.R)
      P.stats[it.li * P.st_layer_stride + P.st_off[it.b] +
              (static_cast<int64_t>(it.h) * it.nspan + it.span) * P.R_pad + r] = make_float2(m_ref, l_row);
    __syncthreads();
    const int nch = min(G::SPAN_CHUNKS, it.C - it.span * G::SPAN_CHUNKS);
    float* ug = P.U + it.li * P.u_layer_stride + P.u_off[it.b] +
                (static_cast<int64_t>(it.h) * it.C + it.span * G::SPAN_CHUNKS) * P.R_pad + it.rb * kMfmaRows;
    for (int e = tid; e < nch * (kMfmaRows / 4); e += kThreads) {
      const int j = e / (kMfmaRows / 4), c4 = e % (kMfmaRows / 4);
      const float4 val = *reinterpret_cast<const float4*>(&u_lds[j * kMfmaRows + c4 * 4]);
      *reinterpret_cast<float4*>(ug + static_cast<int64_t>(j) * P.R_pad + c4 * 4) = val;
    }
  };

  float* u_row = u_lds + ho * G::CPH * kMfmaRows + wave * 32 + n;
  int flat = lo, g = 0;
  Item cur = decode_item<CC>(P, flat);
  load_q(cur);
  load_group(cur, 0);
  float m_ref = -INFINITY, l_acc = 0.0f;
  for (;;) {
    __syncthreads();  // previous group's LDS reads (and any flush) are done
    store_group();
    __syncthreads();

    int nflat = flat, ng = g + 1;
    if (ng == cur.ngroups) {
      ++nflat;
      ng = 0;
    }
    const bool has_next = nflat < hi;
    Item nxt = cur;
    if (has_next && nflat != flat) nxt = decode_item<CC>(P, nflat);
    if (has_next) load_group(nxt, ng);

    f32x16 acc[G::NT];
#pragma unroll
    for (int tau = 0; tau < G::NT; ++tau) {
      acc[tau] = f32x16{};
#pragma unroll
      for (int s = 0; s < kKSteps; ++s) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(
            &k_lds[(tau * 32 + n) * kPieces + ((8 * ho + s) ^ (n & 15))]);
        acc[tau] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bq[s], acc[tau], 0, 0, 0);
      }
    }
    const int gtok0 = cur.tok_begin + g * G::GROUP_TOK;
    const int nvalid = cur.tok_end - (gtok0 + ho * G::HALF_TOK);
    group_softmax<CC>(acc, gtok0 + G::GROUP_TOK <= cur.tok_end, nvalid, P.scale, P.rebase_raw, m_ref,
                      l_acc, u_row, g);
    if (g + 1 == cur.ngroups) {
      flush(cur, m_ref, l_acc);
      m_ref = -INFINITY;
      l_acc = 0.0f;
    }
    if (!has_next) break;
    if (nflat != flat) {
      if (nxt.li != cur.li || nxt.b != cur.b || nxt.h != cur.h || nxt.rb != cur.rb) load_q(nxt);
      cur = nxt;
      flat = nflat;
    }
    g = ng;
  }
}

#define CKV_CHUNKS(X) X(1) X(2) X(3) X(4) X(5) X(6) X(8) X(10) X(12) X(15) X(16) X(20) X(25) X(30) X(32) X(40) X(64)

}  // namespace

bool score_mfma_supported(int chunk) {
  switch (chunk) {
#define CKV_CASE(c) \
  case c:           \
    return pick_tiles(c) >= 1;
    CKV_CHUNKS(CKV_CASE)
#undef CKV_CASE
    default:
      return false;
  }
}

template <int CC>
int span_chunks_of() {
  if constexpr (pick_tiles(CC) >= 1)
    return Geo<CC>::SPAN_CHUNKS;
  else
    return 0;
}

int score_mfma_span_chunks(int chunk) {
  switch (chunk) {
#define CKV_CASE(c) \
  case c:           \
    return span_chunks_of<c>();
    CKV_CHUNKS(CKV_CASE)
#undef CKV_CASE
    default:
      return 0;
  }
}

template <int CC>
hipError_t launch_persistent(ScoreParams p, int n_items, hipStream_t s) {
  static thread_local int cached_dev = -1, cached_workers = 0;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev != cached_dev) {
    int cus = 0, per_cu = 0;
    if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
    if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, score_mfma_kernel<CC>, kThreads, 0)) !=
        hipSuccess)
      return e;
    cached_dev = dev;
    cached_workers = cus * (per_cu > 0 ? per_cu : 1);
  }
  p.n_workers = n_items < cached_workers ? n_items : cached_workers;
  hipLaunchKernelGGL(score_mfma_kernel<CC>, dim3(p.n_workers), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

template <int CC>
hipError_t launch_if_laid_out(const ScoreParams& p, int n_items, hipStream_t s) {
  if constexpr (pick_tiles(CC) >= 1)
    return launch_persistent<CC>(p, n_items, s);
  else
    return hipErrorInvalidValue;
}

hipError_t launch_score_mfma(ScoreParams p, int n_items, hipStream_t s) {
  switch (p.c) {
#define CKV_CASE(c) \
  case c:           \
    return launch_if_laid_out<c>(p, n_items, s);
    CKV_CHUNKS(CKV_CASE)
#undef CKV_CASE
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace ckv
