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
#include <algorithm>
#include <type_traits>

#include "chunkkv_internal.h"
#include "lse_combine.h"

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
#ifndef CKV_KEYS_AUX
#define CKV_KEYS_AUX 2
#endif
#ifndef CKV_U_STORE_AUX
#define CKV_U_STORE_AUX 0
#endif
constexpr int kKeysOnce = CKV_KEYS_AUX;
constexpr int kKeysShared = 0;
constexpr int kSharedKeySpans = 8;
// Chunk sizes scored in two passes over the keys (statistics, then final
// scores) when a head has one row block: there the chunk partials U
// (4*R_pad/c bytes per key token and head, written and read back) would
// outweigh a second read of the keys (2*d bytes).
#ifndef CKV_TWO_PASS_MAX_CHUNK
#define CKV_TWO_PASS_MAX_CHUNK 3
#endif
constexpr int kTwoPassMaxChunk = CKV_TWO_PASS_MAX_CHUNK;
constexpr int kKSteps = kD / 16;     // MFMA k-steps per logit tile
// LDS of an exchange-mode workgroup at most (three per 160 KB CU) and the
// share of it kept for the launch tables.
constexpr int kExchangeLdsBytes = 53 * 1024;
constexpr int kTablesReserve = 1536;
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
  // Exchange mode: a ring of XSLOTS group slots of chunk partials in LDS,
  // one more than the longest span (XGPS groups), so that the next span's
  // first group has a free slot while the previous span still waits for its
  // head's row statistics.  As many slots as keep three workgroups per CU.
  static constexpr int KLDS_BYTES = NT * 32 * kPieces * 16;
  static constexpr int SLOT_FLOATS = GROUP_CHUNKS * kMfmaRows;
  static constexpr int XFIT = (kExchangeLdsBytes - KLDS_BYTES - kTablesReserve) / (SLOT_FLOATS * 4);
  static constexpr int XSLOTS = XFIT < GPS + 1 ? XFIT : GPS + 1;
  static constexpr int XGPS = XSLOTS >= 2 ? XSLOTS - 1 : 0;
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
                                              float& l_acc, float* u_row, int gi, int base = 0,
                                              int nslot = 1 << 20) {
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
  // a span's first group (m_ref still -inf) needs the group maximum anyway:
  // its exponentials are only formed once, against that maximum
  bool ok = __builtin_amdgcn_readfirstlane(gi) != 0;
  if (ok) {
#pragma unroll
    for (int q = 0; q < G::CPH; ++q) {
      u[q] = chunk_exp_sum<CC>(acc, q, scale, -m_ref * scale);
      ok = ok && (u[q] < 0x1p63f);   // false for +inf and NaN too
    }
  } else {
#pragma unroll
    for (int q = 0; q < G::CPH; ++q) u[q] = 0.0f;
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
        for (int gg = 0; gg < gi; ++gg) {
          const int sl = base + gg >= nslot ? base + gg - nslot : base + gg;
#pragma unroll
          for (int q = 0; q < G::CPH; ++q) u_row[(sl * G::GROUP_CHUNKS + q) * kMfmaRows] *= f;
        }
      l_acc *= f;
      m_ref = mx;
#pragma unroll
      for (int q = 0; q < G::CPH; ++q) u[q] = chunk_exp_sum<CC>(acc, q, scale, -m_ref * scale);
    }
  }
  float* dst = u_row + (base + gi >= nslot ? base + gi - nslot : base + gi) * G::GROUP_CHUNKS * kMfmaRows;
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
  int32_t round_start[kMaxRounds + 1];
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
  if (i <= kMaxRounds) t.round_start[i] = P.round_start[i];
}

template <int CC>
__device__ __forceinline__ Item decode_item(const ScoreParams& P, const Tables& t, int flat,
                                            int span_chunks = Geo<CC>::SPAN_CHUNKS) {
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
  it.tok_begin = it.span * span_chunks * CC;
  it.tok_end = min(sgpr(t.T[b]), it.tok_begin + span_chunks * CC);
  it.ngroups = (it.tok_end - it.tok_begin + G::GROUP_TOK - 1) / G::GROUP_TOK;
  it.kbase = sgpr64(t.k[it.li]) +
             2 * static_cast<uint64_t>(static_cast<int64_t>(sgpr64(t.tok0[b])) * P.kv_st +
                                       static_cast<int64_t>(it.h) * P.kv_sh);
  return it;
}

// Position in a workgroup's stream of key groups: item `flat` (in round r
// in exchange mode), group g of it.
struct Cursor {
  int flat, g, r;
  Item it;
};

// Next round from r on (exclusive) in which the workgroup at position pos
// has an item; n_rounds when there is none.
__device__ __forceinline__ int next_round(const ScoreParams& P, const Tables& t, int r, int pos) {
  ++r;
  while (r < P.n_rounds && sgpr(t.round_start[r]) + pos >= sgpr(t.round_start[r + 1])) ++r;
  return r;
}

template <int CC, int MODE>
__device__ __forceinline__ bool cursor_next(const ScoreParams& P, const Tables& t, Cursor& c, int hi, int pos,
                                            int span_chunks) {
  if (++c.g == c.it.ngroups) {
    c.g = 0;
    if constexpr (MODE == kScoreExchange) {
      const int r = next_round(P, t, c.r, pos);
      if (r >= P.n_rounds) return false;
      c.r = r;
      c.flat = sgpr(t.round_start[r]) + pos;
    } else {
      if (++c.flat >= hi) return false;
    }
    c.it = decode_item<CC>(P, t, c.flat, span_chunks);
  }
  return true;
}

// Exchange mode: the chunk scores of one span from its chunk partials (LDS
// ring slots from `base`, or consecutive packed U rows in global memory) and
// the per-row weights wts[r] = 2^((m_span,r - M_r) * scale) / L_r.  Eight
// teams of 32 lanes take one chunk each per pass; lane l multiplies rows
// 4l .. 4l+3 and the team adds by a fixed butterfly.  Partials read from LDS
// are rounded to the 24 bits U stores, so both sources give the same bits.
template <int CC, bool FROM_LDS>
__device__ __forceinline__ void span_scores(const float* src, int base, const float* wts, int nch, float* S) {
  using G = Geo<CC>;
  const int tid = threadIdx.x, team = tid >> 5, l = tid & 31;
  const float4 w4 = reinterpret_cast<const float4*>(wts)[l];
  for (int q0 = 0; q0 < nch; q0 += kThreads / 32) {
    const int q = q0 + team;
    float acc = 0.0f;
    if (q < nch) {
      float4 u4;
      if constexpr (FROM_LDS) {
        int sl = base + q / G::GROUP_CHUNKS;
        if (sl >= G::XSLOTS) sl -= G::XSLOTS;
        u4 = reinterpret_cast<const float4*>(src + (sl * G::GROUP_CHUNKS + q % G::GROUP_CHUNKS) * kMfmaRows)[l];
        u4 = make_float4(round_u24(u4.x), round_u24(u4.y), round_u24(u4.z), round_u24(u4.w));
      } else {
        u4 = unpack_u24(*reinterpret_cast<const u32x3u*>(src + static_cast<int64_t>(q) * (kMfmaRows / 4 * 3) + 3 * l));
      }
      acc = fmaf(u4.x, w4.x, acc);
      acc = fmaf(u4.y, w4.y, acc);
      acc = fmaf(u4.z, w4.z, acc);
      acc = fmaf(u4.w, w4.w, acc);
    }
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
    if (l == 0 && q < nch) S[q] = acc;
  }
}

// Device-coherent accesses of the exchange (agent-scope relaxed atomics: on
// gfx950 the stores write through the XCD's L2 and the loads read past it),
// and the wait that orders this wave's earlier stores before its later
// memory operations: compiler fences on both sides of an s_waitcnt on every
// counter, so neither the compiler nor the hardware moves a store past it.
// The common path of the exchange needs no L2-wide writeback or invalidate.
__device__ __forceinline__ uint32_t load_coherent(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float2 load_coherent(const float2* p) {
  const uint64_t v =
      __hip_atomic_load(reinterpret_cast<uint64_t*>(const_cast<float2*>(p)), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return make_float2(__uint_as_float(static_cast<uint32_t>(v)), __uint_as_float(static_cast<uint32_t>(v >> 32)));
}
__device__ __forceinline__ void store_coherent(float2* p, float2 x) {
  const uint64_t v = static_cast<uint64_t>(__float_as_uint(x.x)) | (static_cast<uint64_t>(__float_as_uint(x.y)) << 32);
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wait_stores() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// rows_lse (same merge order and thread split) over the exchange's
// device-coherent accesses: (M_r, L_r) of rows r < R from the head's n_span
// published span statistics.
__device__ __forceinline__ void rows_lse_coherent(const float2* st, int nspan, int R, int64_t R_pad, float scale,
                                                  float2* lse) {
  constexpr int kUnr = 16;
  const int tpr = lse_tpr(R, kThreads);
  const int sub = threadIdx.x % tpr;
  for (int r = threadIdx.x / tpr; r < R; r += kThreads / tpr) {
    float m = -INFINITY, l = 0.0f;
    for (int s0 = sub; s0 < nspan; s0 += tpr * kUnr) {
      float2 ml[kUnr];
#pragma unroll
      for (int u = 0; u < kUnr; ++u) {
        const int s = s0 + u * tpr;
        ml[u] = s < nspan ? load_coherent(st + s * R_pad + r) : make_float2(-INFINITY, 0.0f);
      }
#pragma unroll
      for (int u = 0; u < kUnr; ++u) lse_merge(m, l, ml[u].x, ml[u].y, scale);
    }
    for (int o = 1; o < tpr; o <<= 1) {
      const float m2 = __shfl_xor(m, o, 64), l2 = __shfl_xor(l, o, 64);
      lse_merge(m, l, m2, l2, scale);
    }
    if (sub == 0) store_coherent(lse + r, make_float2(m, l));
  }
}

// Each workgroup takes a balanced range of consecutive spans of ONE unit
// (layer, sequence, KV head, row block), so its window-query fragments are
// loaded once.  Its key groups form one stream, loaded through a ring of
// STAGES register stages: while group k is multiplied and reduced,
// groups k+1 .. k+STAGES-1 -- of this item or the next ones -- are in flight.
// The ring is indexed statically (the loop is unrolled by STAGES), so each
// LDS store waits only for the loads of its own stage.
//
// Exchange mode (kScoreExchange): the launch is persistent, one workgroup per
// resident slot.  Round r holds whole heads; the workgroup at position p
// (positions count the workgroups of XCD 0 first, then XCD 1, ..., so the
// spans of a head share one XCD's L2) takes item round_start[r] + p, its
// window-query fragments loaded per item during the previous item's last
// group.  Chunk partials go to a ring of LDS slots instead of U.  At the end
// of a span the workgroup publishes (m_ref, l) of its 128 rows and counts
// itself in the head's arrivals; the last arrival forms the head's row
// statistics (M_r, L_r) and raises the head's ready flag.  The span stays
// pending (its slots untouched) while the next span starts; just before that
// span would overwrite the pending slots (or at its own end), the workgroup
// waits for the flag (a bounded number of polls), weights each row's partials
// by 2^((m_ref - M_r) * scale) / L_r and writes the span's chunk scores.  If
// the wait runs out (only when a head's spans are not all resident at once),
// the partials go to U and the span is marked in spill; the last span of the
// head to finish scores the marked spans from U.  Every flag and counter is
// zero on entry (a separate launch clears them).
template <int CC, int KAUX, int MODE>
__global__ __launch_bounds__(kThreads, MODE == kScoreExchange ? CKV_XCH_WAVES : CKV_MIN_WAVES) void score_mfma_kernel(
    const ScoreParams P) {
  using G = Geo<CC>;
  constexpr bool XCH = MODE == kScoreExchange;
  constexpr int kLoadEvery = G::NT * kKSteps / G::LOADS;   // MFMAs per key load of the next group
  static_assert(kLoadEvery * G::LOADS == G::NT * kKSteps, "key loads must spread evenly over the MFMAs");
  static_assert(!XCH || G::XGPS >= 1, "exchange mode needs at least two LDS group slots");
  constexpr int kUFloats = XCH ? G::XSLOTS * G::SLOT_FLOATS : G::SPAN_CHUNKS * kMfmaRows;
  __shared__ u32x4 k_lds[G::NT * 32 * kPieces];
  __shared__ float u_lds[kUFloats];
  __shared__ Tables tab;
  __shared__ int x_word;   // exchange: a flag or counter value broadcast to the workgroup
  static_assert(!XCH || sizeof(k_lds) + sizeof(u_lds) + sizeof(Tables) + 16 <= kExchangeLdsBytes,
                "exchange-mode LDS must leave room for three workgroups per CU");

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, ho = lane >> 5;
  load_tables(P, tab);
  __syncthreads();
  // chunks per span: the host's choice (whole groups, at most SPAN_CHUNKS);
  // the two-pass final mode keeps SPAN_CHUNKS (its LDS row sums are laid out for it)
  const int span_chunks = MODE == kScoreFinal ? G::SPAN_CHUNKS : P.span_chunks;
  int lo = 0, hi = 0, pos = 0, r0 = 0;
  if constexpr (XCH) {
    const int per_xcd = static_cast<int>(gridDim.x) / 8;
    pos = (gridDim.x % 8 == 0) ? static_cast<int>(blockIdx.x % 8) * per_xcd + static_cast<int>(blockIdx.x / 8)
                               : static_cast<int>(blockIdx.x);
    r0 = next_round(P, tab, -1, pos);
    if (r0 >= P.n_rounds) return;
    lo = sgpr(tab.round_start[r0]) + pos;
  } else {
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
    if (lo >= hi) return;
  }

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

  // ---- exchange-mode addressing and steps ----
  auto unit_sync = [&](const Item& it) {
    return P.sync + (static_cast<int64_t>(it.li) * P.n_seqs * P.H_kv + it.b * P.H_kv + it.h) * kSyncWords;
  };
  auto unit_stats = [&](const Item& it) {   // span 0 of the head
    return P.stats + it.li * P.st_layer_stride + sgpr64(tab.st_off[it.b]) +
           static_cast<int64_t>(it.h) * it.nspan * P.R_pad;
  };
  auto unit_lse = [&](const Item& it) {
    return P.lse_w + it.li * P.lse_layer_stride + sgpr64(tab.lse_off[it.b]) + static_cast<int64_t>(it.h) * P.R_pad;
  };
  auto unit_scores = [&](const Item& it) {  // chunk 0 of the head
    return P.S + it.li * P.s_layer_stride + sgpr64(tab.s_off[it.b]) + static_cast<int64_t>(it.h) * it.C;
  };
  auto unit_u = [&](const Item& it) {       // chunk 0 of the head (32-bit words, packed partials)
    return P.U + it.li * P.u_layer_stride + sgpr64(tab.u_off[it.b]) +
           static_cast<int64_t>(it.h) * it.C * u_row_words(kMfmaRows, true);
  };
  int xbase = 0;               // ring slot of the current item's group 0
  bool pend = false;           // a finished span waits for its head's row statistics
  Item p_it{};
  int p_flat = 0, p_base = 0;
  float p_m = 0.0f;            // the pending span's reference m_ref of this lane's row
  float* const wts = reinterpret_cast<float*>(k_lds);   // per-row weights (k_lds is free there)

  // The pending span's chunk scores (or its partials to U), then its count in
  // the head's finished spans; the last to finish scores the spilled spans.
  auto finalize_pending = [&]() __attribute__((always_inline)) {
    uint32_t* sy = unit_sync(p_it);
    __syncthreads();   // every thread has read the last broadcast word
    if (tid == 0) {
      uint32_t v = load_coherent(sy + 2);
      for (int spins = 0; v == 0 && spins < P.spin_limit; ++spins) {
        __builtin_amdgcn_s_sleep(2);
        v = load_coherent(sy + 2);
      }
      x_word = v != 0;
    }
    __syncthreads();
    const bool ready = x_word != 0;
    const int nch = min(span_chunks, p_it.C - p_it.span * span_chunks);
    if (ready) {
      if (ho == 0) {
        const int r = wave * 32 + n;
        float w = 0.0f;
        if (r < P.R) {
          w = span_weight(p_m, load_coherent(unit_lse(p_it) + r), P.scale);
        }
        wts[r] = w;
      }
      __syncthreads();
      span_scores<CC, true>(u_lds, p_base, wts, nch, unit_scores(p_it) + p_it.span * span_chunks);
    } else {
      constexpr int kRowWords = kMfmaRows / 4 * 3;
      float* U = unit_u(p_it) + static_cast<int64_t>(p_it.span) * span_chunks * kRowWords;
      for (int e = tid; e < nch * (kMfmaRows / 4); e += kThreads) {
        const int q = e / (kMfmaRows / 4), c4 = e % (kMfmaRows / 4);
        int sl = p_base + q / G::GROUP_CHUNKS;
        if (sl >= G::XSLOTS) sl -= G::XSLOTS;
        const float4 v =
            reinterpret_cast<const float4*>(u_lds + (sl * G::GROUP_CHUNKS + q % G::GROUP_CHUNKS) * kMfmaRows)[c4];
        *reinterpret_cast<u32x3u*>(U + static_cast<int64_t>(q) * kRowWords + 3 * c4) = pack_u24(v.x, v.y, v.z, v.w);
      }
      if (tid == 0) P.spill[p_flat] = 1u;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    }
    __syncthreads();
    if (tid == 0) {
      // finished spans count in the low 16 bits, spilled ones in the high bits
      if (!ready) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      const uint32_t inc = ready ? 1u : 0x10001u;
      x_word = static_cast<int>(__hip_atomic_fetch_add(sy + 1, inc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + inc);
    }
    __syncthreads();
    if ((x_word & 0xffff) == p_it.nspan && (x_word >> 16) != 0) {
      // every span of the head is scored or spilled and some spilled: score
      // the spilled ones (their partials were released to U before their count)
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      const uint32_t* sp = P.spill + (p_flat - p_it.span);
      const float2* st = unit_stats(p_it);
      const float2* lse = unit_lse(p_it);
      for (int sidx = 0; sidx < p_it.nspan; ++sidx) {
        if (load_coherent(sp + sidx) == 0) continue;
        if (tid < kMfmaRows) {
          float w = 0.0f;
          if (tid < P.R) w = span_weight(load_coherent(st + sidx * P.R_pad + tid).x, load_coherent(lse + tid), P.scale);
          wts[tid] = w;
        }
        __syncthreads();
        span_scores<CC, false>(unit_u(p_it) + static_cast<int64_t>(sidx) * span_chunks * (kMfmaRows / 4 * 3), 0, wts,
                               min(span_chunks, p_it.C - sidx * span_chunks),
                               unit_scores(p_it) + sidx * span_chunks);
        __syncthreads();
      }
    }
    pend = false;
  };

  // End of an exchange-mode item: publish its row statistics, count it in
  // its head's arrivals (the last arrival forms the row statistics and raises
  // the ready flag), score the previous pending span if any, and leave this
  // one pending.
  auto publish = [&](const Item& it, float m_ref, float l_acc, int flat) __attribute__((always_inline)) {
    const float l_row = l_acc + shfl_xor32(l_acc);
    __syncthreads();   // every wave is past this group's fragment reads
    float2* stage = reinterpret_cast<float2*>(k_lds);
    if (ho == 0) stage[wave * 32 + n] = make_float2(m_ref, l_row);
    __syncthreads();
    uint32_t* sy = unit_sync(it);
    if (wave == 0) {
      float2* st = unit_stats(it) + it.span * P.R_pad;
      store_coherent(st + lane, stage[lane]);
      store_coherent(st + lane + 64, stage[lane + 64]);
      wait_stores();
      if (lane == 0) x_word = static_cast<int>(__hip_atomic_fetch_add(sy, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    }
    __syncthreads();
    if (x_word + 1 == it.nspan) {
      // the last arrival: every span of the head has published
      rows_lse_coherent(unit_stats(it), it.nspan, P.R, P.R_pad, P.scale, unit_lse(it));
      wait_stores();
      __syncthreads();
      if (tid == 0) __hip_atomic_store(sy + 2, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (pend) finalize_pending();
    pend = true;
    p_it = it;
    p_flat = flat;
    p_base = xbase;
    p_m = m_ref;
    xbase += it.ngroups;
    if (xbase >= G::XSLOTS) xbase -= G::XSLOTS;
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
    // packed 24-bit partials (bf16 problems): 12 bytes per 4 rows
    const int nch = sgpr(min(span_chunks, it.C - it.span * span_chunks));
    const int64_t row_words = u_row_words(P.R_pad, true);
    const uint64_t ubase = reinterpret_cast<uint64_t>(P.U + it.li * P.u_layer_stride) +
                           4 * static_cast<uint64_t>(sgpr64(tab.u_off[it.b]) +
                                                     (static_cast<int64_t>(it.h) * it.C + it.span * span_chunks) *
                                                         row_words +
                                                     u_row_words(it.rb * kMfmaRows, true));
    const int chunk_bytes = static_cast<int>(row_words * 4);
    const __amdgpu_buffer_rsrc_t ru = __builtin_amdgcn_make_buffer_rsrc(
        reinterpret_cast<void*>(sgpr64(ubase)), 0, nch * chunk_bytes, kBufferWord3);
    constexpr int kPieces4 = G::SPAN_CHUNKS * (kMfmaRows / 4);
#pragma unroll
    for (int x = 0; x < (kPieces4 + kThreads - 1) / kThreads; ++x) {
      const int e = x * kThreads + tid;
      const int j = e / (kMfmaRows / 4), c4 = e % (kMfmaRows / 4);
      const float4 val = reinterpret_cast<const float4*>(u_lds)[min(e, kPieces4 - 1)];
      __builtin_amdgcn_raw_buffer_store_b96(pack_u24(val.x, val.y, val.z, val.w), ru, j * chunk_bytes + c4 * 12, 0,
                                            CKV_U_STORE_AUX);
    }
  };

  float* u_row = u_lds + ho * G::CPH * kMfmaRows + wave * 32 + n;
  Cursor cc{lo, 0, r0, decode_item<CC>(P, tab, lo, span_chunks)};   // group being computed
  Cursor lc = cc;                             // next group to load
  // Every step issues exactly one group of loads: past the end of the range
  // the last group is loaded again (its data is never used), so the number of
  // loads younger than any stage is fixed and each stage store waits only
  // for its own loads.
  auto next_rsrc = [&]() {
    const __amdgpu_buffer_rsrc_t rsrc = group_rsrc(lc.it, lc.g);
    Cursor t = lc;
    if (cursor_next<CC, MODE>(P, tab, t, hi, pos, span_chunks)) lc = t;
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

  // total key groups of this workgroup's items: the main loop is counted, so
  // its only branches are uniform ones around the compute and write-back
  int total = 0;
  if constexpr (XCH) {
    for (int r = r0; r < P.n_rounds; r = next_round(P, tab, r, pos))
      total += decode_item<CC>(P, tab, sgpr(tab.round_start[r]) + pos, span_chunks).ngroups;
  } else {
    for (int f = lo; f < hi; ++f) total += decode_item<CC>(P, tab, f, span_chunks).ngroups;
  }

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
      const bool last_group = cc.g + 1 == it.ngroups;
      const int gtok0 = it.tok_begin + cc.g * G::GROUP_TOK;
      const int nvalid = it.tok_end - (gtok0 + ho * G::HALF_TOK);
      if constexpr (MODE == kScoreFinal) {
        group_final<CC>(acc, gtok0 + G::GROUP_TOK <= it.tok_end, nvalid, P.scale, nfin, red,
                        s_lds + wave * G::SPAN_CHUNKS + cc.g * G::GROUP_CHUNKS, lane, n, ho);
      } else if constexpr (XCH) {
        group_softmax<CC, true>(acc, gtok0 + G::GROUP_TOK <= it.tok_end, nvalid, P.scale, P.rebase_raw, m_ref,
                                l_acc, u_row, cc.g, xbase, G::XSLOTS);
      } else {
        group_softmax<CC, MODE == kScorePartials>(acc, gtok0 + G::GROUP_TOK <= it.tok_end, nvalid, P.scale,
                                                  P.rebase_raw, m_ref, l_acc, u_row, cc.g);
      }
      if (last_group) {
        if constexpr (XCH) {
          // the next item's window queries load while this one is published
          Cursor t = cc;
          if (cursor_next<CC, MODE>(P, tab, t, hi, pos, span_chunks)) load_q(t.it);
          publish(it, m_ref, l_acc, cc.flat);
        } else {
          flush(it, m_ref, l_acc);
        }
        m_ref = -INFINITY;
        l_acc = 0.0f;
      }
      cursor_next<CC, MODE>(P, tab, cc, hi, pos, span_chunks);
      if constexpr (XCH) {
        // the next group would overwrite the pending span's first slot:
        // score that span now (k_lds is free until the next store_group)
        if (pend) {
          const int sl = xbase + cc.g >= G::XSLOTS ? xbase + cc.g - G::XSLOTS : xbase + cc.g;
          if (sl == p_base) finalize_pending();
        }
      }
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
  if constexpr (XCH) {
    if (pend) finalize_pending();
  }
}

struct ZeroArgs {
  uint32_t* p;
  int64_t n;
};

__global__ __launch_bounds__(kThreads) void zero_words_kernel(const ZeroArgs a) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; i < a.n;
       i += static_cast<int64_t>(gridDim.x) * kThreads)
    a.p[i] = 0u;
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

// Chunk sizes with an exchange-mode kernel: a static layout, not scored in
// two passes, and at least two LDS group slots.
// (Chunk sizes whose exchange kernel needs more than 168 VGPRs at three
// waves per SIMD -- 12, 20, 30, 32, 40, 64 -- keep the chunk-partial path.)
constexpr bool exchange_fits_registers(int c) {
  return c == 4 || c == 5 || c == 6 || c == 8 || c == 10 || c == 15 || c == 16 || c == 25;
}

template <int CC>
constexpr bool has_exchange() {
  if constexpr (pick_tiles(CC) >= 1)
    return CC > kTwoPassMaxChunk && Geo<CC>::XGPS >= 1 && exchange_fits_registers(CC);
  else
    return false;
}

template <int CC>
int exchange_span_of() {
  if constexpr (has_exchange<CC>())
    return Geo<CC>::XGPS * Geo<CC>::GROUP_CHUNKS;
  else
    return 0;
}

template <int CC>
int group_chunks_of() {
  if constexpr (pick_tiles(CC) >= 1)
    return Geo<CC>::GROUP_CHUNKS;
  else
    return 0;
}

template <int CC>
hipError_t exchange_slots_of(int* slots) {
  if constexpr (has_exchange<CC>()) {
    static thread_local int cached_dev = -1, cached = 0;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev != cached_dev) {
      int cus = 0, per_cu = 0;
      if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
      if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, score_mfma_kernel<CC, kKeysOnce, kScoreExchange>,
                                                            kThreads, 0)) != hipSuccess)
        return e;
      cached_dev = dev;
      cached = cus * per_cu / 8 * 8;
    }
    *slots = cached;
    return hipSuccess;
  } else {
    *slots = 0;
    return hipSuccess;
  }
}

template <int CC>
hipError_t launch_if_laid_out(const ScoreParams& p, int n_items, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  if constexpr (pick_tiles(CC) >= 1) {
    if (p.mode == kScoreExchange) {
      // n_items is the persistent grid here (the largest round, a multiple of 8)
      if constexpr (has_exchange<CC>())
        return launch1(score_mfma_kernel<CC, kKeysOnce, kScoreExchange>, dim3(n_items), dim3(kThreads), 0, s, p, e0,
                       e1);
      else
        return hipErrorInvalidValue;
    }
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

int score_exchange_max_span_chunks(int chunk) {
  switch (chunk) {
#define CKV_CASE(c) \
  case c:           \
    return exchange_span_of<c>();
    CKV_CHUNKS(CKV_CASE)
#undef CKV_CASE
    default:
      return 0;
  }
}

int score_group_chunks(int chunk) {
  switch (chunk) {
#define CKV_CASE(c) \
  case c:           \
    return group_chunks_of<c>();
    CKV_CHUNKS(CKV_CASE)
#undef CKV_CASE
    default:
      return 0;
  }
}

hipError_t score_exchange_slots(int chunk, int* slots) {
  switch (chunk) {
#define CKV_CASE(c) \
  case c:           \
    return exchange_slots_of<c>(slots);
    CKV_CHUNKS(CKV_CASE)
#undef CKV_CASE
    default:
      *slots = 0;
      return hipSuccess;
  }
}

hipError_t launch_zero_words(uint32_t* p, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((n + kThreads - 1) / kThreads, 1024);
  return launch1(zero_words_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, s, ZeroArgs{p, n});
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
