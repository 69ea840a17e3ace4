// Fused observe-window score kernel for bf16 caches with head_dim 128 on
// gfx950 (CDNA4): ChunkKV page, section 4.1, Algorithm 1 steps 1-3, with the
// softmax(QK^T / sqrt(d)) of Kara eq. (1).
//
// Work item = (layer, sequence, KV head, 128-row block of the G*w window
// rows, span of whole chunks).  Workgroups (about one per resident slot; more,
// with shorter ranges, when a head has several row blocks) walk contiguous
// ranges of items; keys are streamed HBM -> VGPR -> LDS once, a register ring
// of groups ahead.  Logits come from v_mfma_f32_32x32x16_bf16 with the KEYS as
// the A operand (32 token slots x 16 dims) and the window queries as B (16
// dims x 32 query rows), so in the 32x32 fp32 result each lane owns one query row
// and 16 token slots.  Token slots are permuted so that each lane half holds
// CPH whole chunks: the chunk sums are then straight-line adds fixed at
// compile time for each chunk size.  The logits never leave registers: the
// kernel writes, per query row, the chunk partials
//   U[j][r] = sum_{t in chunk j} 2^((x_rt - m_r) * log2(e)/sqrt(d))
// and (m_r, l_r = sum over the span) for the log-sum-exp combine.
//
// Short chunks (c <= 3) with one 128-row block per head take two passes over
// the keys instead, since their partials U (one float per row and chunk)
// would outweigh the keys: the first pass writes only the span statistics;
// after the row statistics (M_r, L_r) are formed, the second computes each
// logit's final probability 2^((x - M_r)*scale - log2 L_r), sums it per chunk
// in registers and over the block's 128 rows through LDS, and writes the
// chunk scores themselves.
#include <type_traits>

#include "chunkkv_internal.h"

namespace ckv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
// Explicitly global-address-space element types, so that loads through
// addresses kept in LDS compile to global (not flat) instructions.
typedef __attribute__((address_space(1))) const bf16x8 gbf16x8;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const u32x4 gu32x4;

constexpr int kD = 128;              // head_dim of this path
// Buffer resource word 3 for raw dword loads on gfx9-family (CDNA) parts.
constexpr int kBufferWord3 = 0x00020000;
// Cache policies of the key loads (buffer instruction aux bits).  With one
// row block per head every key is read once: non-temporal, so the keys do not
// displace the chunk partials and window queries in L2.  With several row
// blocks (G*w > 128) the blocks of a head read the same keys on one XCD at
// about the same time: ordinary caching lets that XCD's L2 serve the repeats.
constexpr int kKeysOnce = 2;
constexpr int kKeysShared = 0;
constexpr int kSharedKeySpans = 8;
// Chunk sizes scored in two passes over the keys (statistics, then final
// scores) when a head has one row block: there the chunk partials U
// (4*R_pad/c bytes per key token and head, written and read back) would
// outweigh a second read of the keys (2*d bytes).
constexpr int kTwoPassMaxChunk = 3;
constexpr int kKSteps = kD / 16;     // MFMA k-steps per logit tile
constexpr int kLdsAhead = 4;         // key fragment reads issued ahead of their MFMA
constexpr int kPieces = kD / 8;      // 16-byte pieces per bf16 key row

// Number of 32-slot MFMA tiles per group for chunk size c (slots per lane
// half = 16 * nt, holding floor(16 * nt / c) whole chunks): the smallest
// count whose padding is at most 1/16 of the slots, else the one with the
// least padding (ties to fewer tiles), at most kMaxTiles.
constexpr int pick_tiles(int c) {
  int best = 0, best_num = 1, best_den = 0;  // padding = num/den
  for (int nt = 1; nt <= kMaxTiles; ++nt) {
    const int cph = 16 * nt / c;
    if (cph == 0) continue;
    const int num = 16 * nt - cph * c, den = 16 * nt;
    if (num * 16 <= den) return nt;
    if (best == 0 || num * best_den < best_num * den) {
      best = nt;
      best_num = num;
      best_den = den;
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
  // register stages (groups of keys in flight), at least 2
  static constexpr int STAGES = (kStageTiles / NT) >= 2 ? (kStageTiles / NT > 4 ? 4 : kStageTiles / NT) : 2;
};

__device__ __forceinline__ float shfl_xor32(float v) { return __shfl_xor(v, 32, 64); }

// Sum of the exponentials of one chunk's logits (terms q*CC .. q*CC+CC-1 of
// the lane half), as a balanced tree: short dependency chains.
template <int CC>
__device__ __forceinline__ float chunk_exp_sum(const f32x16 (&acc)[Geo<CC>::NT], int q, float scale, float nmrs) {
  float t[CC];
#pragma unroll
  for (int e = 0; e < CC; ++e) {
    const int lam = q * CC + e;
    t[e] = __builtin_amdgcn_exp2f(fmaf(acc[lam >> 4][lam & 15], scale, nmrs));
  }
#pragma unroll
  for (int w = 1; w < CC; w *= 2)
#pragma unroll
    for (int e = 0; e + w < CC; e += 2 * w) t[e] += t[e + w];
  return t[0];
}

// Softmax pieces of one group for this lane's row: write the chunk partials
// of this lane half to LDS, relative to the row's reference m_ref.  The
// reference is moved (and the earlier partials and l rescaled) only when the
// group's maximum exceeds it by more than 2^kRebaseLog2.  That test needs the
// group maximum, so it is made only when some lane's chunk sum reaches 2^63
// or is not finite (always the case on a span's first group, where m_ref is
// -inf): without it, every term is below 2^64 and the test would fail anyway.
// Slots past the end of the sequence are masked to -inf (exp2 gives 0).
template <int CC, bool STORE>
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
  float u[G::CPH];
  bool ok = true;
#pragma unroll
  for (int q = 0; q < G::CPH; ++q) {
    u[q] = chunk_exp_sum<CC>(acc, q, scale, -m_ref * scale);
    ok = ok && (u[q] < 0x1p63f);   // false for +inf and NaN too
  }
  if (__ballot(!ok) != 0) {
    float mx = -INFINITY;
#pragma unroll
    for (int tau = 0; tau < G::NT; ++tau)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        if (16 * tau + v < G::HALF_TOK) mx = fmaxf(mx, acc[tau][v]);
    mx = fmaxf(mx, shfl_xor32(mx));
    if (mx > m_ref + rebase_raw) {
      const float f = (m_ref == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f((m_ref - mx) * scale);
      if constexpr (STORE)
        for (int gg = 0; gg < gi; ++gg)
#pragma unroll
          for (int q = 0; q < G::CPH; ++q) u_row[(gg * G::GROUP_CHUNKS + q) * kMfmaRows] *= f;
      l_acc *= f;
      m_ref = mx;
#pragma unroll
      for (int q = 0; q < G::CPH; ++q) u[q] = chunk_exp_sum<CC>(acc, q, scale, -m_ref * scale);
    }
  }
  float* dst = u_row + gi * G::GROUP_CHUNKS * kMfmaRows;
#pragma unroll
  for (int q = 0; q < G::CPH; ++q) {
    if constexpr (STORE) dst[q * kMfmaRows] = u[q];
    l_acc += u[q];
  }
}

// Orders this wave's LDS writes before its later LDS reads by other lanes.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Row stride (floats) of the per-wave transpose buffer of the final pass:
// 16-byte aligned rows whose 16-byte reads by 16 consecutive lanes fall in
// distinct banks.
constexpr int kRedStride = 36;

// Final pass, one group: this lane's row probabilities summed per chunk
// (exp2((x - M_r)*scale - log2 L_r), nfin = -(M_r*scale + log2 L_r), -inf for
// padding rows), then summed over the wave's 32 rows through LDS: chunk q of
// lane half ho goes to row (ho*CPH + q) of `red`, column n; lanes then add
// their chunk's 16-row half in row order and the two halves meet by one
// cross-half exchange.  Lane l < GROUP_CHUNKS writes chunk l's sum to s_row[l].
template <int CC>
__device__ __forceinline__ void group_final(f32x16 (&acc)[Geo<CC>::NT], bool full, int nvalid, float scale,
                                            float nfin, float* red, float* s_row, int lane, int n, int ho) {
  using G = Geo<CC>;
  static_assert(G::GROUP_CHUNKS <= 32, "final pass: one lane per chunk of a group");
  if (!full) {
#pragma unroll
    for (int tau = 0; tau < G::NT; ++tau)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int lam = 16 * tau + v;
        if (lam < G::HALF_TOK) acc[tau][v] = lam < nvalid ? acc[tau][v] : -INFINITY;
      }
  }
#pragma unroll
  for (int q = 0; q < G::CPH; ++q) red[(ho * G::CPH + q) * kRedStride + n] = chunk_exp_sum<CC>(acc, q, scale, nfin);
  wave_sync();
  const int cl = lane & 31, rh = lane >> 5;
  float sum = 0.0f;
  if (cl < G::GROUP_CHUNKS) {
    const float4* p = reinterpret_cast<const float4*>(red + cl * kRedStride + 16 * rh);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 v = p[i];
      sum += (v.x + v.y) + (v.z + v.w);
    }
  }
  sum += shfl_xor32(sum);
  if (lane < G::GROUP_CHUNKS) s_row[lane] = sum;
  wave_sync();
}

// One work item: (layer, sequence, KV head, row block, span of whole chunks).
struct Item {
  int li, b, h, rb, span, nspan, C, tok_begin, tok_end, ngroups;
  uint64_t kbase;   // byte address of token 0 of this sequence, head h
};

// Values read from the LDS tables are the same in every lane; moving them to
// scalar registers keeps the address and cursor arithmetic on the scalar unit.
__device__ __forceinline__ int sgpr(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ uint64_t sgpr64(uint64_t v) {
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(v)));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(v >> 32)));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// The launch's per-layer and per-sequence tables, copied to LDS once so that
// decoding an item with a runtime index never issues a vector memory load
// (those would share the counter the key stream is waited on with).
struct Tables {
  uint64_t q[kMaxLayers];        // device addresses (global address space)
  uint64_t k[kMaxLayers];
  int64_t tok0[kMaxSeqs];
  int64_t u_off[kMaxSeqs];
  int64_t st_off[kMaxSeqs];
  int64_t s_off[kMaxSeqs];
  int64_t lse_off[kMaxSeqs];
  int32_t item0[kMaxSeqs + 1];
  int32_t n_span[kMaxSeqs];
  int32_t T[kMaxSeqs];
  int32_t C[kMaxSeqs];
  int32_t qseq[kMaxSeqs];
  int32_t wpu[kMaxSeqs];
  int32_t worker0[kMaxSeqs + 1];
};

__device__ __forceinline__ void load_tables(const ScoreParams& P, Tables& t) {
  const int i = threadIdx.x;
  if (i < kMaxLayers) {
    t.q[i] = reinterpret_cast<uint64_t>(P.q[i]);
    t.k[i] = reinterpret_cast<uint64_t>(P.k[i]);
  }
  if (i < kMaxSeqs) {
    t.tok0[i] = P.tok0[i];
    t.u_off[i] = P.u_off[i];
    t.st_off[i] = P.st_off[i];
    t.s_off[i] = P.s_off[i];
    t.lse_off[i] = P.lse_off[i];
    t.n_span[i] = P.n_span[i];
    t.T[i] = P.T[i];
    t.C[i] = P.C[i];
    t.qseq[i] = P.qseq[i];
    t.wpu[i] = P.wpu[i];
  }
  if (i <= kMaxSeqs) {
    t.item0[i] = P.item0[i];
    t.worker0[i] = P.worker0[i];
  }
}

template <int CC>
__device__ __forceinline__ Item decode_item(const ScoreParams& P, const Tables& t, int flat) {
  using G = Geo<CC>;
  Item it;
  it.li = flat / P.items_per_layer;
  int item = flat - it.li * P.items_per_layer;
  int b = 0;
  while (b + 1 < P.n_seqs && item >= sgpr(t.item0[b + 1])) ++b;
  item -= sgpr(t.item0[b]);
  it.b = b;
  it.nspan = sgpr(t.n_span[b]);
  it.span = item % it.nspan;
  const int hr = item / it.nspan;
  it.rb = hr % P.n_rb;
  it.h = hr / P.n_rb;
  it.C = sgpr(t.C[b]);
  it.tok_begin = it.span * G::SPAN_CHUNKS * CC;
  it.tok_end = min(sgpr(t.T[b]), it.tok_begin + G::SPAN_CHUNKS * CC);
  it.ngroups = (it.tok_end - it.tok_begin + G::GROUP_TOK - 1) / G::GROUP_TOK;
  it.kbase = sgpr64(t.k[it.li]) +
             2 * static_cast<uint64_t>(static_cast<int64_t>(sgpr64(t.tok0[b])) * P.kv_st +
                                       static_cast<int64_t>(it.h) * P.kv_sh);
  return it;
}

// Position in a workgroup's stream of key groups.
struct Cursor {
  int flat, g;
  Item it;
};

template <int CC>
__device__ __forceinline__ bool cursor_next(const ScoreParams& P, const Tables& t, Cursor& c, int hi) {
  if (++c.g == c.it.ngroups) {
    c.g = 0;
    if (++c.flat >= hi) return false;
    c.it = decode_item<CC>(P, t, c.flat);
  }
  return true;
}

// Each workgroup takes a balanced range of consecutive spans of ONE unit
// (layer, sequence, KV head, row block), so its window-query fragments are
// loaded once.  Its key groups form one stream, loaded through a ring of
// STAGES register stages: while group k is multiplied and reduced,
// groups k+1 .. k+STAGES-1 -- of this item or the next ones -- are in flight.
// The ring is indexed statically (the loop is unrolled by STAGES), so each
// LDS store waits only for the loads of its own stage.
template <int CC, int KAUX, int MODE>
__global__ __launch_bounds__(kThreads, CKV_MIN_WAVES) void score_mfma_kernel(const ScoreParams P) {
  using G = Geo<CC>;
  constexpr int kLoadEvery = G::NT * kKSteps / G::LOADS;   // MFMAs per key load of the next group
  static_assert(kLoadEvery * G::LOADS == G::NT * kKSteps, "key loads must spread evenly over the MFMAs");
  __shared__ u32x4 k_lds[G::NT * 32 * kPieces];
  __shared__ float u_lds[G::SPAN_CHUNKS * kMfmaRows];
  __shared__ Tables tab;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, ho = lane >> 5;
  load_tables(P, tab);
  __syncthreads();
  int lo, hi;
  {
    const int li = blockIdx.x / P.workers_per_layer;
    const int wr = blockIdx.x - li * P.workers_per_layer;
    int b = 0;
    while (b + 1 < P.n_seqs && wr >= tab.worker0[b + 1]) ++b;
    const int wpu = tab.wpu[b], ns = tab.n_span[b];
    const int m = wr - tab.worker0[b];
    int unit = m / wpu, piece = m % wpu;
    if (P.rb_interleave) {
      // m = (g, rb, x) with x < 8: (head, piece) number g * 8 + x, row block rb
      const int g = m / (8 * P.n_rb), x = m % 8, rb = (m / 8) % P.n_rb;
      const int hp = g * 8 + x;
      unit = (hp / wpu) * P.n_rb + rb;
      piece = hp % wpu;
    }
    const int base = li * P.items_per_layer + tab.item0[b] + unit * ns;
    lo = base + piece * ns / wpu;
    hi = base + (piece + 1) * ns / wpu;
  }
  if (lo >= hi) return;

  // window-query fragments (B operand) of this wave's 32 rows; rows >= R are zero
  bf16x8 bq[kKSteps];
  auto load_q = [&](const Item& it) {
    const int r = it.rb * kMfmaRows + wave * 32 + n;
    if (r < P.R) {
      const int g = r / P.w;
      const int rr = r - g * P.w;
      const int hq = it.h * P.G + g;
      const uint64_t qa = tab.q[it.li] + 2 * static_cast<uint64_t>(tab.qseq[it.b] * P.q_ss + rr * P.q_sr +
                                                                   hq * P.q_sh + ho * (kD / 2));
#pragma unroll
      for (int s = 0; s < kKSteps; ++s) bq[s] = *((gbf16x8*)(qa + 16 * s));
    } else {
#pragma unroll
      for (int s = 0; s < kKSteps; ++s) bq[s] = bf16x8{};
    }
  };

  // key streaming: slot (tile tau, row i) <-> token of lane half (i/4)%2.
  // Keys are read through a buffer resource whose base is the group's first
  // token and whose size ends at the span's end, so each lane's offsets are
  // fixed for the whole kernel and tokens past the end of the sequence read
  // as zeros (their logits are masked).  Padding slots (lam >= HALF_TOK)
  // repeat the half's last slot; their logits are never used.
  u32x4 regs[G::STAGES][G::LOADS];
  const int st_bytes = static_cast<int>(P.kv_st * 2);   // < 2^31 / 128, checked on the host
  int voff[G::LOADS];
#pragma unroll
  for (int x = 0; x < G::LOADS; ++x) {
    const int gp = x * kThreads + tid;
    const int sr = gp / kPieces, p = gp % kPieces;
    const int tau = sr >> 5, i = sr & 31;
    const int lam = min(16 * tau + 4 * (i >> 3) + (i & 3), G::HALF_TOK - 1);
    voff[x] = (((i >> 2) & 1) * G::HALF_TOK + lam) * st_bytes + p * 16;
  }
  auto group_rsrc = [&](const Item& it, int gi) {
    const int gtok0 = it.tok_begin + gi * G::GROUP_TOK;
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(it.kbase + static_cast<uint64_t>(gtok0) * st_bytes),
                                             0, min(it.tok_end - gtok0, G::GROUP_TOK) * st_bytes, kBufferWord3);
  };
  auto store_group = [&](const u32x4 (&src)[G::LOADS]) {
#pragma unroll
    for (int x = 0; x < G::LOADS; ++x) {
      const int gp = x * kThreads + tid;
      const int sr = gp / kPieces, p = gp % kPieces;
      k_lds[sr * kPieces + (p ^ (sr & 15))] = src[x];
    }
  };
  // Per-row span statistics and chunk partials of a finished item.  The
  // stores go through buffer resources sized to the data (pieces past the
  // span's last chunk are dropped), so their number is fixed: the compiler's
  // memory-counter waits in the main loop then stay exact.
  // final pass: per-wave transpose buffers, then the span's per-wave chunk sums
  float* const red = u_lds + wave * (G::GROUP_CHUNKS * kRedStride);
  float* const s_lds = u_lds + 4 * G::GROUP_CHUNKS * kRedStride;   // [4 waves][SPAN_CHUNKS]
  static_assert(MODE != kScoreFinal ||
                    4 * G::GROUP_CHUNKS * kRedStride + 4 * G::SPAN_CHUNKS <= G::SPAN_CHUNKS * kMfmaRows,
                "final-pass buffers fit in the partials' LDS");
  auto flush = [&](const Item& it, float m_ref, float l_acc) {
    if constexpr (MODE == kScoreFinal) {
      // the span's chunk scores: the 4 waves' row sums added in wave order;
      // every thread issues one store, those past the span's chunks are dropped
      __syncthreads();
      const int nch = sgpr(min(G::SPAN_CHUNKS, it.C - it.span * G::SPAN_CHUNKS));
      const uint64_t sb = reinterpret_cast<uint64_t>(P.S + it.li * P.s_layer_stride) +
                          4 * static_cast<uint64_t>(sgpr64(tab.s_off[it.b]) + static_cast<int64_t>(it.h) * it.C +
                                                    it.span * G::SPAN_CHUNKS);
      const __amdgpu_buffer_rsrc_t rsS = __builtin_amdgcn_make_buffer_rsrc(
          reinterpret_cast<void*>(sgpr64(sb)), 0, nch * 4, kBufferWord3);
      const int j = min(tid, G::SPAN_CHUNKS - 1);
      const float v = (s_lds[j] + s_lds[G::SPAN_CHUNKS + j]) +
                      (s_lds[2 * G::SPAN_CHUNKS + j] + s_lds[3 * G::SPAN_CHUNKS + j]);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), rsS, tid * 4, 0, 0);
      return;
    }
    const float l_row = l_acc + shfl_xor32(l_acc);
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    const uint64_t sbase = reinterpret_cast<uint64_t>(P.stats + it.li * P.st_layer_stride) +
                           8 * static_cast<uint64_t>(sgpr64(tab.st_off[it.b]) +
                                                     (static_cast<int64_t>(it.h) * it.nspan + it.span) * P.R_pad +
                                                     it.rb * kMfmaRows);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        reinterpret_cast<void*>(sgpr64(sbase)), 0, kMfmaRows * 8, kBufferWord3);
    // both lane halves hold the row's statistics; half 1 aims past the end
    __builtin_amdgcn_raw_buffer_store_b64(u32x2{__float_as_uint(m_ref), __float_as_uint(l_row)}, rs,
                                          (wave * 32 + n) * 8 + ho * kMfmaRows * 8, 0, 0);
    if constexpr (MODE == kScoreStats) return;
    __syncthreads();
    const int nch = sgpr(min(G::SPAN_CHUNKS, it.C - it.span * G::SPAN_CHUNKS));
    const uint64_t ubase = reinterpret_cast<uint64_t>(P.U + it.li * P.u_layer_stride) +
                           4 * static_cast<uint64_t>(sgpr64(tab.u_off[it.b]) +
                                                     (static_cast<int64_t>(it.h) * it.C + it.span * G::SPAN_CHUNKS) *
                                                         P.R_pad +
                                                     it.rb * kMfmaRows);
    const int chunk_bytes = P.R_pad * 4;
    const __amdgpu_buffer_rsrc_t ru = __builtin_amdgcn_make_buffer_rsrc(
        reinterpret_cast<void*>(sgpr64(ubase)), 0, nch * chunk_bytes, kBufferWord3);
    constexpr int kPieces4 = G::SPAN_CHUNKS * (kMfmaRows / 4);
#pragma unroll
    for (int x = 0; x < (kPieces4 + kThreads - 1) / kThreads; ++x) {
      const int e = x * kThreads + tid;
      const int j = e / (kMfmaRows / 4), c4 = e % (kMfmaRows / 4);
      const u32x4 val = reinterpret_cast<const u32x4*>(u_lds)[min(e, kPieces4 - 1)];
      __builtin_amdgcn_raw_buffer_store_b128(val, ru, j * chunk_bytes + c4 * 16, 0, 0);
    }
  };

  float* u_row = u_lds + ho * G::CPH * kMfmaRows + wave * 32 + n;
  Cursor cc{lo, 0, decode_item<CC>(P, tab, lo)};   // group being computed
  Cursor lc = cc;                             // next group to load
  // Every step issues exactly one group of loads: past the end of the range
  // the last group is loaded again (its data is never used), so the number of
  // loads younger than any stage is fixed and each stage store waits only
  // for its own loads.
  auto next_rsrc = [&]() {
    const __amdgpu_buffer_rsrc_t rsrc = group_rsrc(lc.it, lc.g);
    Cursor t = lc;
    if (cursor_next<CC>(P, tab, t, hi)) lc = t;
    return rsrc;
  };
  auto load_next = [&](u32x4 (&dst)[G::LOADS]) {
    const __amdgpu_buffer_rsrc_t rsrc = next_rsrc();
#pragma unroll
    for (int x = 0; x < G::LOADS; ++x) dst[x] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, voff[x], 0, KAUX);
  };
  load_q(cc.it);
  // final pass: -(M_r*scale + log2 L_r) of this lane's row (a workgroup's
  // range lies in one unit), -inf for padding rows
  float nfin = -INFINITY;
  if constexpr (MODE == kScoreFinal) {
    const Item& u0 = cc.it;
    const int r = u0.rb * kMfmaRows + wave * 32 + n;
    if (r < P.R) {
      const float2 ml = P.lse[u0.li * P.lse_layer_stride + sgpr64(tab.lse_off[u0.b]) +
                              static_cast<int64_t>(u0.h) * P.R_pad + r];
      nfin = -fmaf(ml.x, P.scale, log2f(ml.y));
    }
  }
  // issue the stages strictly in ring order (stage 0 oldest)
#pragma unroll
  for (int s = 0; s < G::STAGES; ++s) {
    load_next(regs[s]);
    __builtin_amdgcn_sched_barrier(0);
  }
  float m_ref = -INFINITY, l_acc = 0.0f;

  // total key groups of this workgroup's range: the main loop is counted, so
  // its only branches are uniform ones around the compute and write-back
  int total = 0;
  for (int f = lo; f < hi; ++f) total += decode_item<CC>(P, tab, f).ngroups;

  // one group of the stream, held in ring stage S; steps past the end of the
  // range (live == false) still issue their loads (repeats of the last group)
  auto step = [&](auto stage_tag, bool live) {
    constexpr int S = decltype(stage_tag)::value;
    __syncthreads();  // previous group's LDS reads (and any flush) are done
    store_group(regs[S]);
    __syncthreads();
    // the next group's loads go out one per kLoadEvery MFMAs of this group
    // (issued together right after the barrier, the 4 waves' loads queue up
    // at the vector-memory unit); past the end of the range, all at once
    const __amdgpu_buffer_rsrc_t rsrc = next_rsrc();
    if (live) {
      f32x16 acc[G::NT];
#pragma unroll
      for (int tau = 0; tau < G::NT; ++tau) {
        acc[tau] = f32x16{};
#pragma unroll
        for (int s = 0; s < kKSteps; ++s) {
          const int mi = tau * kKSteps + s;
          if (mi % kLoadEvery == 0)
            regs[S][mi / kLoadEvery] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, voff[mi / kLoadEvery], 0, KAUX);
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(
              &k_lds[(tau * 32 + n) * kPieces + ((8 * ho + s) ^ (n & 15))]);
          acc[tau] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bq[s], acc[tau], 0, 0, 0);
        }
      }
      // schedule: the first kLdsAhead fragment reads, then per MFMA: its
      // key load (every kLoadEvery-th), the MFMA, the fragment read kLdsAhead
      // ahead (group masks: 0x008 MFMA, 0x020 vector-memory read, 0x100 LDS read)
      __builtin_amdgcn_sched_group_barrier(0x100, kLdsAhead, 0);
#pragma unroll
      for (int mi = 0; mi < G::NT * kKSteps; ++mi) {
        if (mi % kLoadEvery == 0) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (mi + kLdsAhead < G::NT * kKSteps) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      const Item& it = cc.it;
      const int gtok0 = it.tok_begin + cc.g * G::GROUP_TOK;
      const int nvalid = it.tok_end - (gtok0 + ho * G::HALF_TOK);
      if constexpr (MODE == kScoreFinal)
        group_final<CC>(acc, gtok0 + G::GROUP_TOK <= it.tok_end, nvalid, P.scale, nfin, red,
                        s_lds + wave * G::SPAN_CHUNKS + cc.g * G::GROUP_CHUNKS, lane, n, ho);
      else
        group_softmax<CC, MODE == kScorePartials>(acc, gtok0 + G::GROUP_TOK <= it.tok_end, nvalid, P.scale,
                                                  P.rebase_raw, m_ref, l_acc, u_row, cc.g);
      if (cc.g + 1 == it.ngroups) {
        flush(it, m_ref, l_acc);
        m_ref = -INFINITY;
        l_acc = 0.0f;
      }
      cursor_next<CC>(P, tab, cc, hi);
    } else {
#pragma unroll
      for (int x = 0; x < G::LOADS; ++x) regs[S][x] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, voff[x], 0, KAUX);
    }
  };
  const int rounds = (total + G::STAGES - 1) / G::STAGES;
  for (int rd = 0; rd < rounds; ++rd) {
    const int k0 = rd * G::STAGES;
    step(std::integral_constant<int, 0>{}, k0 < total);
    if constexpr (G::STAGES > 1) step(std::integral_constant<int, 1 % G::STAGES>{}, k0 + 1 < total);
    if constexpr (G::STAGES > 2) step(std::integral_constant<int, 2 % G::STAGES>{}, k0 + 2 < total);
    if constexpr (G::STAGES > 3) step(std::integral_constant<int, 3 % G::STAGES>{}, k0 + 3 < total);
    if constexpr (G::STAGES > 4) step(std::integral_constant<int, 4 % G::STAGES>{}, k0 + 4 < total);
    if constexpr (G::STAGES > 5) step(std::integral_constant<int, 5 % G::STAGES>{}, k0 + 5 < total);
    if constexpr (G::STAGES > 6) step(std::integral_constant<int, 6 % G::STAGES>{}, k0 + 6 < total);
    if constexpr (G::STAGES > 7) step(std::integral_constant<int, 7 % G::STAGES>{}, k0 + 7 < total);
  }
}

#define CKV_CHUNKS(X) X(1) X(2) X(3) X(4) X(5) X(6) X(8) X(10) X(12) X(15) X(16) X(20) X(25) X(30) X(32) X(40) X(64)

}  // namespace

bool score_two_pass_supported(int chunk) { return chunk >= 1 && chunk <= kTwoPassMaxChunk; }

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

// Work split: balanced ranges of consecutive spans of one unit, about one
// workgroup per resident slot (shorter ranges for heads of several row blocks).
template <int CC, int KAUX, int MODE>
hipError_t launch_split(ScoreParams p, int n_items, hipStream_t s, hipEvent_t ev_start, hipEvent_t ev_stop) {
  static thread_local int cached_dev = -1, cached_slots = 0;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev != cached_dev) {
    int cus = 0, per_cu = 0;
    if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
    if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, score_mfma_kernel<CC, KAUX, MODE>, kThreads, 0)) !=
        hipSuccess)
      return e;
    cached_dev = dev;
    cached_slots = cus * (per_cu > 0 ? per_cu : 1);
  }
  // spans per workgroup: about one workgroup per resident slot; with several
  // row blocks per head at most kSharedKeySpans, so that the blocks of a span
  // range (dispatched together onto one XCD) stay close enough in time for
  // that XCD's L2 to serve their repeated key reads
  int per_worker = (n_items + cached_slots - 1) / cached_slots;
  if (p.n_rb > 1 && per_worker > kSharedKeySpans) per_worker = kSharedKeySpans;
  int w = 0;
  for (int b = 0; b < p.n_seqs; ++b) {
    p.wpu[b] = (p.n_span[b] + per_worker - 1) / per_worker;
    p.worker0[b] = w;
    w += p.H_kv * p.n_rb * p.wpu[b];
  }
  p.worker0[p.n_seqs] = w;
  p.workers_per_layer = w;
  // workgroups are dealt to the 8 XCDs in id order; the interleave needs every
  // sequence's worker count to be a multiple of 8 * n_rb
  p.rb_interleave = p.n_rb > 1 ? 1 : 0;
  for (int b = 0; b < p.n_seqs; ++b)
    if ((p.H_kv * p.wpu[b]) % 8 != 0) p.rb_interleave = 0;
  return launch1(score_mfma_kernel<CC, KAUX, MODE>, dim3(w * p.n_layers), dim3(kThreads), 0, s, p, ev_start,
                 ev_stop);
}

template <int CC>
hipError_t launch_if_laid_out(const ScoreParams& p, int n_items, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  if constexpr (pick_tiles(CC) >= 1) {
    if (p.mode != kScorePartials) {
      // two passes: short chunks, one row block (keys read once per pass)
      if constexpr (CC <= kTwoPassMaxChunk) {
        if (p.n_rb != 1) return hipErrorInvalidValue;
        return p.mode == kScoreStats ? launch_split<CC, kKeysOnce, kScoreStats>(p, n_items, s, e0, e1)
                                     : launch_split<CC, kKeysOnce, kScoreFinal>(p, n_items, s, e0, e1);
      } else {
        return hipErrorInvalidValue;
      }
    }
    return p.n_rb > 1 ? launch_split<CC, kKeysShared, kScorePartials>(p, n_items, s, e0, e1)
                      : launch_split<CC, kKeysOnce, kScorePartials>(p, n_items, s, e0, e1);
  } else {
    return hipErrorInvalidValue;
  }
}

hipError_t launch_score_mfma(ScoreParams p, int n_items, hipStream_t s, hipEvent_t ev_start, hipEvent_t ev_stop) {
  switch (p.c) {
#define CKV_CASE(c) \
  case c:           \
    return launch_if_laid_out<c>(p, n_items, s, ev_start, ev_stop);
    CKV_CHUNKS(CKV_CASE)
#undef CKV_CASE
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace ckv
