// Host side of libchunkkv.so: validation, planning and launch sequencing
// behind the C-ABI declared in include/chunkkv.h.
//
// Phases (ChunkKV page, section 4.1 Algorithm 1 and section 4.2 Algorithm 2):
//   score    window attention -> per-row chunk partials   (score_mfma / score_generic)
//   combine  log-sum-exp normalisation -> chunk scores      (combine)
//   select   top-k chunks + recent window -> indices        (select)
//   gather   index_select of K and V                        (gather)
// Everything is validated here before the first launch; launches are
// asynchronous on the caller's stream and nothing synchronises with the host.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "chunkkv.h"
#include "chunkkv_internal.h"
#include "decode_internal.h"
#include "paged_internal.h"

namespace {

using namespace ckv;

thread_local std::string g_err;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return status;
}

int ok() {
  g_err.clear();
  return CHUNKKV_OK;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(CHUNKKV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Seq {
  int64_t tok0;
  int32_t T, C, kk, L_cap, n_span;
  int32_t n_span_final;   // two passes: spans of the final pass (n_span counts the statistics pass's)
  int64_t score_off, index_off, u_off, st_off, lse_off;
};

struct Plan {
  int dtype = 0, eb = 0, B = 0, Hq = 0, Hkv = 0, G = 0, d = 0, w = 0, c = 0;
  int R = 0, R_pad = 0, n_rb = 0, span_chunks = 0;
  int final_span = 0;      // two passes: the final pass's span (its LDS layout's); span_chunks is the statistics pass's
  bool mfma = false;
  bool two_pass = false;   // statistics pass + final-score pass, no chunk partials
  bool u_packed = false;   // chunk partials stored in 24 bits (bf16 problems)
  // exchange mode possible: its longest span (chunks) and the chunks per MFMA group
  int x_max_span = 0, group_chunks = 0;
  std::vector<Seq> seq;
  int64_t scores_elems = 0, index_elems = 0, length_elems = 0, u_elems = 0, st_elems = 0, lse_elems = 0;
  int64_t kv_st = 0, kv_sh = 0, q_ss = 0, q_sr = 0, q_sh = 0;
};

// The exchange kernel (chunk partials kept in LDS, per-row statistics
// exchanged between the spans of a head inside one persistent launch) is
// built and parity-tested but slower than the chunk-partial path on every
// workload measured (its spans wait for the slowest span of their head each
// round and pay several device-scope round trips), so it runs only when
// CHUNKKV_SCORE_PATH=exchange asks for it.
bool exchange_disabled() {
  const char* v = std::getenv("CHUNKKV_SCORE_PATH");
  return !(v && std::strcmp(v, "exchange") == 0);
}

// Polls of a head's ready flag before an exchange-mode span gives up and
// spills its partials (CHUNKKV_SPIN_LIMIT overrides; 0 makes every span spill).
int exchange_spin_limit() {
  const char* v = std::getenv("CHUNKKV_SPIN_LIMIT");
  if (!v || !*v) return 4096;
  const long x = std::strtol(v, nullptr, 10);
  return x < 0 ? 0 : (x > (1 << 24) ? (1 << 24) : static_cast<int>(x));
}

// Score work items per layer that keep a single-layer launch's CUs busy.
constexpr int64_t kMinLayerItems = 192;

// Longest span of the statistics pass of two-pass plans, in final-pass spans
// (a power of two).
#ifndef CKV_STATS_SPAN_MAX
#define CKV_STATS_SPAN_MAX 16
#endif
constexpr int kStatsSpanMax = CKV_STATS_SPAN_MAX;

int make_plan(const chunkkv_problem* p, Plan& pl) {
  if (!p) return fail(CHUNKKV_ERR_INVALID_ARG, "problem is NULL");
  if (p->reserved != 0) return fail(CHUNKKV_ERR_INVALID_ARG, "reserved field must be 0");
  if (p->dtype != CHUNKKV_F32 && p->dtype != CHUNKKV_BF16)
    return fail(CHUNKKV_ERR_INVALID_ARG, "dtype %d is neither CHUNKKV_F32 nor CHUNKKV_BF16", p->dtype);
  if (p->n_seqs < 1) return fail(CHUNKKV_ERR_INVALID_ARG, "n_seqs must be >= 1 (got %d)", p->n_seqs);
  if (!p->seq_start || !p->l_max) return fail(CHUNKKV_ERR_INVALID_ARG, "seq_start and l_max must be non-NULL");
  if (p->n_q_heads < 1 || p->n_kv_heads < 1)
    return fail(CHUNKKV_ERR_INVALID_ARG, "head counts must be >= 1");
  if (p->n_q_heads % p->n_kv_heads != 0)
    return fail(CHUNKKV_ERR_INVALID_ARG, "n_q_heads (%d) must be a multiple of n_kv_heads (%d)",
                p->n_q_heads, p->n_kv_heads);
  if (p->window < 1) return fail(CHUNKKV_ERR_INVALID_ARG, "window must be >= 1 (got %d)", p->window);
  if (p->chunk < 1) return fail(CHUNKKV_ERR_INVALID_ARG, "chunk must be >= 1 (got %d)", p->chunk);
  if (p->head_dim < 1) return fail(CHUNKKV_ERR_INVALID_ARG, "head_dim must be >= 1");
  const int eb = p->dtype == CHUNKKV_F32 ? 4 : 2;
  if (p->head_dim < 8 || p->head_dim > 256 || (p->head_dim * eb) % 16 != 0)
    return fail(CHUNKKV_ERR_UNSUPPORTED, "head_dim %d unsupported (8..256, rows a multiple of 16 bytes)",
                p->head_dim);
  if (p->kv_stride_tok < 1 || p->kv_stride_head < 0 || p->q_stride_seq < 0 || p->q_stride_row < 0 ||
      p->q_stride_head < 0)
    return fail(CHUNKKV_ERR_INVALID_ARG, "strides must be non-negative (kv_stride_tok >= 1)");
  if ((p->kv_stride_tok * eb) % 16 || (p->kv_stride_head * eb) % 16 || (p->q_stride_seq * eb) % 16 ||
      (p->q_stride_row * eb) % 16 || (p->q_stride_head * eb) % 16)
    return fail(CHUNKKV_ERR_UNSUPPORTED, "strides must keep every row 16-byte aligned");
  const int64_t R = static_cast<int64_t>(p->n_q_heads / p->n_kv_heads) * p->window;
  if (R > 4096) return fail(CHUNKKV_ERR_UNSUPPORTED, "G*w = %lld window rows per KV head exceeds 4096",
                            static_cast<long long>(R));
  if (p->seq_start[0] < 0) return fail(CHUNKKV_ERR_INVALID_ARG, "seq_start[0] must be >= 0");

  pl = Plan{};
  pl.dtype = p->dtype;
  pl.eb = eb;
  pl.B = p->n_seqs;
  pl.Hq = p->n_q_heads;
  pl.Hkv = p->n_kv_heads;
  pl.G = p->n_q_heads / p->n_kv_heads;
  pl.d = p->head_dim;
  pl.w = p->window;
  pl.c = p->chunk;
  pl.R = static_cast<int>(R);
  // the MFMA kernel addresses the keys of a group (at most 128 token rows)
  // with 32-bit byte offsets
  pl.mfma = p->dtype == CHUNKKV_BF16 && p->head_dim == 128 && score_mfma_supported(p->chunk) &&
            p->kv_stride_tok * 2 * 128 < (int64_t{1} << 31);
  pl.R_pad = static_cast<int>(pl.mfma ? round_up(R, kMfmaRows) : round_up(R, 4));
  pl.n_rb = pl.mfma ? pl.R_pad / kMfmaRows : 1;
  pl.span_chunks = pl.mfma ? score_mfma_span_chunks(pl.c) : score_generic_span_chunks(pl.R_pad, pl.c);
  // short chunks with one row block: the chunk partials (4*R_pad/c bytes
  // per key token and head, written and read back) would outweigh a second
  // pass over the keys (2*d bytes)
  pl.two_pass = pl.mfma && pl.n_rb == 1 && score_two_pass_supported(pl.c);
  pl.final_span = pl.span_chunks;
  pl.group_chunks = pl.mfma ? score_group_chunks(pl.c) : 0;
  pl.x_max_span = pl.mfma && pl.n_rb == 1 && !pl.two_pass && !exchange_disabled()
                      ? score_exchange_max_span_chunks(pl.c) : 0;
  pl.u_packed = pl.dtype == CHUNKKV_BF16;
  auto layer_items = [&](int64_t span) {
    int64_t n = 0;
    for (int b = 0; b < pl.B; ++b) {
      const int64_t C = std::max<int64_t>(0, p->seq_start[b + 1] - p->seq_start[b] + pl.c - 1) / pl.c;
      n += static_cast<int64_t>(pl.Hkv) * pl.n_rb * ((C + span - 1) / span);
    }
    return n;
  };
  // Two passes: the statistics pass keeps no chunk partials in LDS, so its
  // spans may be several final-pass spans long (fewer span starts, whose
  // first group forms the row maximum, and fewer span statistics), while a
  // layer keeps kMinLayerItems items; the final pass keeps the span its LDS
  // row sums are laid out for.  Measured per call (final spans x 1 / 4 / 8 /
  // 16): 16k tokens at c = 1 98.7 / 86.5 / 86.5 / 95 us, c = 2 62.5 / 57.9 /
  // 65.3 / 81.7, c = 3 60.1 / 60.2 / 71.5 / 95; the 32-layer 32k stack at
  // c = 1 (16 scoring layers) 908-916 / 831 / 803-813 / 795-812 us per step.
  if (pl.two_pass) {
    int f = kStatsSpanMax;
    while (f > 1 && layer_items(static_cast<int64_t>(pl.final_span) * f) < kMinLayerItems) f /= 2;
    pl.span_chunks = pl.final_span * f;
  }
  // A layer with few score work items at the full span (one short sequence:
  // 8 KV heads x 14 spans of an 8k-token layer at c = 10) leaves most CUs
  // idle in a single-layer call, and each span's chain of dependent key
  // groups sets the launch's length: such layers take shorter spans, in whole
  // MFMA groups and at least half the full span, until a layer has
  // kMinLayerItems items.  Measured per single-layer call: 8k tokens at c = 10
  // and 16k at c = 20 (112 items at 60-chunk spans) 30.7 and 33.9 us with
  // 30-chunk spans against 33.9 and 39.1 us; 16k at c = 10 (224 items) is
  // fastest at the full span (36.3 us; 39-41 us with 30-48-chunk spans).
  if (pl.mfma && !pl.two_pass) {
    const int floor_span = std::max(pl.group_chunks, pl.span_chunks / 2 / pl.group_chunks * pl.group_chunks);
    int span = pl.span_chunks;
    while (span - pl.group_chunks >= floor_span && layer_items(span) < kMinLayerItems) span -= pl.group_chunks;
    pl.span_chunks = span;
  }
  pl.kv_st = p->kv_stride_tok;
  pl.kv_sh = p->kv_stride_head;
  pl.q_ss = p->q_stride_seq;
  pl.q_sr = p->q_stride_row;
  pl.q_sh = p->q_stride_head;

  int64_t items = 0;
  for (int b = 0; b < pl.B; ++b) {
    const int64_t T = p->seq_start[b + 1] - p->seq_start[b];
    if (T < 1) return fail(CHUNKKV_ERR_INVALID_ARG, "sequence %d is empty or seq_start decreases", b);
    if (T < p->window)
      return fail(CHUNKKV_ERR_INVALID_ARG, "window %d exceeds sequence %d length %lld", p->window, b,
                  static_cast<long long>(T));
    if (T > 2147483647LL - p->chunk - 64)
      return fail(CHUNKKV_ERR_UNSUPPORTED, "sequence %d longer than 2^31 tokens", b);
    if (p->l_max[b] < 0) return fail(CHUNKKV_ERR_INVALID_ARG, "l_max[%d] must be >= 0", b);
    Seq s{};
    s.tok0 = p->seq_start[b];
    s.T = static_cast<int32_t>(T);
    s.C = static_cast<int32_t>((T + pl.c - 1) / pl.c);
    s.kk = static_cast<int32_t>(std::min<int64_t>(p->l_max[b] / pl.c, s.C));
    s.L_cap = static_cast<int32_t>(std::min<int64_t>(T, static_cast<int64_t>(s.kk) * pl.c + pl.w));
    s.n_span = (s.C + pl.span_chunks - 1) / pl.span_chunks;
    s.n_span_final = (s.C + pl.final_span - 1) / pl.final_span;
    s.score_off = pl.scores_elems;
    s.index_off = pl.index_elems;
    s.u_off = pl.u_elems;
    s.st_off = pl.st_elems;
    s.lse_off = pl.lse_elems;
    pl.scores_elems += static_cast<int64_t>(pl.Hkv) * s.C;
    pl.index_elems += static_cast<int64_t>(pl.Hkv) * s.L_cap;
    if (!pl.two_pass) pl.u_elems += static_cast<int64_t>(pl.Hkv) * s.C * u_row_words(pl.R_pad, pl.u_packed);
    pl.st_elems += static_cast<int64_t>(pl.Hkv) * s.n_span * pl.R_pad;
    pl.lse_elems += static_cast<int64_t>(pl.Hkv) * pl.R_pad;
    items += static_cast<int64_t>(pl.Hkv) * pl.n_rb * std::max(s.n_span, s.n_span_final);
    pl.seq.push_back(s);
  }
  if (items * kMaxLayers > 2000000000LL)
    return fail(CHUNKKV_ERR_UNSUPPORTED, "problem too large for one launch grid");
  pl.length_elems = static_cast<int64_t>(pl.B) * pl.Hkv;
  return CHUNKKV_OK;
}

// ------------------------------------------------------- exchange layout --

// Resident exchange workgroups the span choice assumes (256 CUs x 3); the
// launch packs its rounds with the device's own count.
constexpr int kNominalSlots = 768;

// Span layout of an exchange-mode score launch over nl layers: span length
// (chunks), spans per head of each sequence, statistics offsets.
struct XLayout {
  bool ok = false;
  int span_chunks = 0;
  std::vector<int32_t> n_span;   // per sequence
  std::vector<int64_t> st_off;   // per sequence: float2 offset of head 0, span 0 within a layer
  int64_t st_elems = 0;          // float2 per layer
  int64_t spill_elems = 0;       // spill flags per layer (one per span of every head)
};

// Rounds of one exchange launch (layers [0, nl), sequences [b0, b0 + nb)):
// whole heads in flat item order (layer, sequence, head, span), at most
// `slots` spans per round.  Returns the round count (0 if a head alone has
// more spans than slots); fills round_start[0 .. rounds] (flat item indices,
// the last one the end) when it is non-NULL and rounds <= kMaxRounds, and the
// largest round's span count.
int pack_rounds(const Plan& pl, const std::vector<int32_t>& n_span, int b0, int nb, int nl, int slots,
                int32_t* round_start, int* max_round) {
  int per_layer = 0;
  for (int i = 0; i < nb; ++i) per_layer += pl.Hkv * n_span[b0 + i];
  int rounds = 0, cur = 0, mx = 0, flat = 0;
  for (int li = 0; li < nl; ++li)
    for (int i = 0; i < nb; ++i)
      for (int h = 0; h < pl.Hkv; ++h) {
        const int ns = n_span[b0 + i];
        if (ns > slots) return 0;
        if (rounds == 0 || cur + ns > slots) {
          mx = std::max(mx, cur);
          if (round_start && rounds <= kMaxRounds) round_start[rounds] = flat;
          ++rounds;
          cur = 0;
        }
        cur += ns;
        flat += ns;
      }
  mx = std::max(mx, cur);
  if (round_start && rounds <= kMaxRounds) round_start[rounds] = nl * per_layer;
  if (max_round) *max_round = mx;
  return rounds;
}

// The span length (whole MFMA groups, at most the kernel's LDS ring allows)
// that minimises the sum over launches of rounds x (groups per span + 1),
// the +1 standing for a round's exchange; ties go to longer spans.  The
// choice assumes kNominalSlots resident workgroups, so that workspace sizes
// depend on the problem and the layer count alone.
XLayout xlayout(const Plan& pl, int nl) {
  XLayout xl;
  if (pl.x_max_span <= 0 || pl.group_chunks <= 0 || nl < 1) return xl;
  const int gmax = pl.x_max_span / pl.group_chunks;
  int64_t best = -1;
  int best_g = 0;
  std::vector<int32_t> ns(pl.B);
  for (int g = 1; g <= gmax; ++g) {
    const int span = g * pl.group_chunks;
    for (int b = 0; b < pl.B; ++b) ns[b] = (pl.seq[b].C + span - 1) / span;
    int64_t cost = 0;
    bool ok = true;
    for (int b0 = 0; b0 < pl.B && ok; b0 += kMaxSeqs) {
      const int r = pack_rounds(pl, ns, b0, std::min(kMaxSeqs, pl.B - b0), nl, kNominalSlots, nullptr, nullptr);
      if (r < 1 || r > kMaxRounds) ok = false;
      cost += static_cast<int64_t>(r) * (g + 1);
    }
    if (ok && (best < 0 || cost <= best)) {
      best = cost;
      best_g = g;
    }
  }
  if (!best_g) return xl;
  xl.ok = true;
  xl.span_chunks = best_g * pl.group_chunks;
  xl.n_span.resize(pl.B);
  xl.st_off.resize(pl.B);
  for (int b = 0; b < pl.B; ++b) {
    xl.n_span[b] = (pl.seq[b].C + xl.span_chunks - 1) / xl.span_chunks;
    xl.st_off[b] = xl.st_elems;
    xl.st_elems += static_cast<int64_t>(pl.Hkv) * xl.n_span[b] * pl.R_pad;
    xl.spill_elems += static_cast<int64_t>(pl.Hkv) * xl.n_span[b];
  }
  return xl;
}

// Workspace of nl scoring layers per launch: chunk partials U, span
// statistics (sized for both span layouts), row statistics, then the
// exchange launch's per-head words and per-span spill flags.
struct Work {
  float* U;
  float2* st;
  float2* lse;
  uint32_t* sync;    // sync and spill are contiguous (one clearing launch)
  uint32_t* spill;
};

size_t ws_need(const Plan& pl, int nl, const XLayout& xl) {
  const int64_t st = std::max<int64_t>(pl.st_elems, xl.ok ? xl.st_elems : 0);
  const int64_t flags = xl.ok ? static_cast<int64_t>(pl.B) * pl.Hkv * kSyncWords + xl.spill_elems : 0;
  return align_up(static_cast<size_t>(nl) * pl.u_elems * sizeof(float)) +
         align_up(static_cast<size_t>(nl) * st * sizeof(float2)) +
         align_up(static_cast<size_t>(nl) * pl.lse_elems * sizeof(float2)) +
         align_up(static_cast<size_t>(nl) * flags * sizeof(uint32_t));
}

size_t ws_need(const Plan& pl, int nl) { return ws_need(pl, nl, xlayout(pl, nl)); }

Work carve(const Plan& pl, int nl, const XLayout& xl, void* ws) {
  const int64_t st = std::max<int64_t>(pl.st_elems, xl.ok ? xl.st_elems : 0);
  const size_t u_bytes = align_up(static_cast<size_t>(nl) * pl.u_elems * sizeof(float));
  const size_t st_bytes = align_up(static_cast<size_t>(nl) * st * sizeof(float2));
  const size_t lse_bytes = align_up(static_cast<size_t>(nl) * pl.lse_elems * sizeof(float2));
  char* base = static_cast<char*>(ws);
  Work w;
  w.U = reinterpret_cast<float*>(base);
  w.st = reinterpret_cast<float2*>(base + u_bytes);
  w.lse = reinterpret_cast<float2*>(base + u_bytes + st_bytes);
  w.sync = reinterpret_cast<uint32_t*>(base + u_bytes + st_bytes + lse_bytes);
  w.spill = w.sync + static_cast<int64_t>(nl) * pl.B * pl.Hkv * kSyncWords;
  return w;
}

// ------------------------------------------------------------- launchers --

// ev_start / ev_stop (null, or only with one sequence batch and the MFMA
// kernel) are recorded at the score kernel's start and end.  mode is
// kScorePartials (U and statistics), kScoreStats (statistics only) or
// kScoreFinal (chunk scores from the row statistics lse).
hipError_t run_score(const Plan& pl, int nl, const void* const* q, const void* const* k, float* U,
                     float2* st, hipStream_t s, hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr,
                     int mode = kScorePartials, const float2* lse = nullptr, float* scores = nullptr) {
  for (int b0 = 0; b0 < pl.B; b0 += kMaxSeqs) {
    const int nb = std::min(kMaxSeqs, pl.B - b0);
    ScoreParams P{};
    for (int i = 0; i < nl; ++i) {
      P.q[i] = q[i];
      P.k[i] = k[i];
    }
    P.n_layers = nl;
    P.n_seqs = nb;
    const bool final_pass = mode == kScoreFinal;
    P.span_chunks = final_pass ? pl.final_span : pl.span_chunks;
    int items = 0;
    for (int i = 0; i < nb; ++i) {
      const Seq& sq = pl.seq[b0 + i];
      P.tok0[i] = sq.tok0;
      P.qseq[i] = b0 + i;
      P.T[i] = sq.T;
      P.C[i] = sq.C;
      P.n_span[i] = final_pass ? sq.n_span_final : sq.n_span;
      P.item0[i] = items;
      P.u_off[i] = sq.u_off;
      P.st_off[i] = sq.st_off;
      P.s_off[i] = sq.score_off;
      P.lse_off[i] = sq.lse_off;
      items += pl.Hkv * pl.n_rb * P.n_span[i];
    }
    P.item0[nb] = items;
    P.items_per_layer = items;
    P.u_layer_stride = pl.u_elems;
    P.st_layer_stride = pl.st_elems;
    P.s_layer_stride = pl.scores_elems;
    P.lse_layer_stride = pl.lse_elems;
    P.U = U;
    P.u_packed = pl.u_packed ? 1 : 0;
    P.stats = st;
    P.mode = mode;
    P.S = scores;
    P.lse = lse;
    P.H_q = pl.Hq;
    P.H_kv = pl.Hkv;
    P.G = pl.G;
    P.w = pl.w;
    P.c = pl.c;
    P.d = pl.d;
    P.R = pl.R;
    P.R_pad = pl.R_pad;
    P.n_rb = pl.n_rb;
    P.kv_st = pl.kv_st;
    P.kv_sh = pl.kv_sh;
    P.q_ss = pl.q_ss;
    P.q_sr = pl.q_sr;
    P.q_sh = pl.q_sh;
    P.scale = static_cast<float>(1.4426950408889634 / std::sqrt(static_cast<double>(pl.d)));
    P.rebase_raw = kRebaseLog2 / P.scale;
    const int nblk = nl * items;
    const hipError_t e = pl.mfma ? launch_score_mfma(P, nblk, s, ev_start, ev_stop)
                                 : launch_score_generic(P, pl.dtype, nblk, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Combine blocks a launch should have (2 per CU of a 256-CU part) before
// spans per block are reduced.
constexpr int64_t kCombineMinBlocks = 512;

// Heads whose span statistics take at most this many bytes have every
// combine block form the row statistics itself (no row-statistics launch).
#ifndef CKV_FUSE_LSE_BYTES
#define CKV_FUSE_LSE_BYTES 32768
#endif
constexpr int64_t kFuseLseBytes = CKV_FUSE_LSE_BYTES;

// Spans per combine block: fewer when the launch would otherwise have too
// few blocks to spread over the GPU (a layer or two of short sequences).
int combine_spb(const Plan& pl, int nl) {
  int spb = combine_spans_per_blk(pl.R_pad);
  auto n_blocks = [&](int per) {
    int64_t n = 0;
    for (const Seq& sq : pl.seq) n += static_cast<int64_t>(pl.Hkv) * ((sq.n_span + per - 1) / per);
    return n * nl;
  };
  while (spb > 1 && n_blocks(spb) < kCombineMinBlocks) spb /= 2;
  return spb;
}

// Combine (and row-statistics) parameters of nl scoring layers of sequences
// [b0, b0 + nb), spb spans per block.
CombineParams combine_params(const Plan& pl, int nl, int b0, int nb, int spb, const float* U, const float2* st,
                             float2* lse, float* scores, bool lse_only) {
  CombineParams P{};
  P.n_layers = nl;
  P.n_seqs = nb;
  P.span_chunks = pl.span_chunks;
  P.spans_per_blk = spb;
  int items = 0;
  for (int i = 0; i < nb; ++i) {
    const Seq& sq = pl.seq[b0 + i];
    P.C[i] = sq.C;
    P.n_span[i] = sq.n_span;
    P.n_blk[i] = (sq.n_span + spb - 1) / spb;
    P.item0[i] = items;
    P.u_off[i] = sq.u_off;
    P.st_off[i] = sq.st_off;
    P.score_off[i] = sq.score_off;
    P.lse_off[i] = sq.lse_off;
    P.head0[i] = i * pl.Hkv;
    items += pl.Hkv * P.n_blk[i];
  }
  P.item0[nb] = items;
  P.head0[nb] = nb * pl.Hkv;
  P.items_per_layer = items;
  P.u_layer_stride = pl.u_elems;
  P.st_layer_stride = pl.st_elems;
  P.score_layer_stride = pl.scores_elems;
  P.lse_layer_stride = pl.lse_elems;
  P.U = U;
  P.u_packed = pl.u_packed ? 1 : 0;
  P.stats = st;
  P.lse = lse;
  P.scores = scores;
  P.H_kv = pl.Hkv;
  P.R = pl.R;
  P.R_pad = pl.R_pad;
  P.scale = static_cast<float>(1.4426950408889634 / std::sqrt(static_cast<double>(pl.d)));
  // short heads (span statistics of at most kFuseLseBytes, one round of
  // loads at 128 rows): every combine block forms its head's row statistics
  // itself, which saves a launch (8k layer: 38 -> 35 us per call); with
  // more spans the repeated reads cost more than the launch (32k layers)
  int64_t st_bytes = 0;
  for (int i = 0; i < nb; ++i) st_bytes = std::max<int64_t>(st_bytes, int64_t{8} * P.n_span[i] * pl.R_pad);
  P.fuse_lse = st_bytes <= kFuseLseBytes && !lse_only ? 1 : 0;
  return P;
}

// lse_only: the row statistics alone (the two-pass path's final pass reads them).
hipError_t run_combine(const Plan& pl, int nl, const float* U, const float2* st, float2* lse, float* scores,
                       hipStream_t s, bool lse_only = false) {
  const int spb = combine_spb(pl, nl);
  for (int b0 = 0; b0 < pl.B; b0 += kMaxSeqs) {
    const int nb = std::min(kMaxSeqs, pl.B - b0);
    const CombineParams P = combine_params(pl, nl, b0, nb, spb, U, st, lse, scores, lse_only);
    hipError_t e = P.fuse_lse ? hipSuccess : launch_row_lse(P, nl * nb * pl.Hkv, s);
    if (e != hipSuccess) return e;
    if (lse_only) continue;
    e = launch_combine(P, nl * P.items_per_layer, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Kept rows per decode work item: a multiple of the item's step giving about
// kDecodeBlocks workgroup items (kDecodeWaveItems wave items) over the whole problem (the blocks' partials are
// merged per query head), so short caches still spread over the GPU and long
// ones keep the merge short.
constexpr int64_t kDecodeBlocks = 512;
int decode_rows_per_block(const Plan& pl) {
  int64_t rows = 0;
  for (const Seq& sq : pl.seq) rows += static_cast<int64_t>(pl.Hkv) * sq.L_cap;
  const bool wave = decode_wave_path(pl.d * pl.eb);
  const int64_t items = wave ? kDecodeWaveItems : kDecodeBlocks;
  const int64_t step = wave ? kWaveRows : kDecRows;
  const int64_t per = std::max<int64_t>((rows + items - 1) / items, step);
  return static_cast<int>(std::min<int64_t>(round_up(per, step), int64_t{1} << 30));
}

// Exchange-mode scores of nl scoring layers (one persistent launch per batch
// of at most kMaxSeqs sequences, after one launch that clears the flags).
// Returns hipErrorNotSupported, having launched nothing, when this device
// cannot hold a round's spans at once or the launch would need more than
// kMaxRounds rounds.
hipError_t run_exchange(const Plan& pl, const XLayout& xl, int nl, const void* const* q, const void* const* k,
                        const Work& w, float* scores, hipStream_t s, hipEvent_t ev_start, hipEvent_t ev_stop) {
  int slots = 0;
  hipError_t e = score_exchange_slots(pl.c, &slots);
  if (e != hipSuccess) return e;
  if (slots < 8) return hipErrorNotSupported;
  for (int b0 = 0; b0 < pl.B; b0 += kMaxSeqs) {
    const int r = pack_rounds(pl, xl.n_span, b0, std::min(kMaxSeqs, pl.B - b0), nl, slots, nullptr, nullptr);
    if (r < 1 || r > kMaxRounds) return hipErrorNotSupported;
  }
  // the per-head words of nl layers and the spill flags (which follow the
  // per-head words of the workspace's layer count) in one clearing launch
  const int64_t words = (w.spill - w.sync) + static_cast<int64_t>(nl) * xl.spill_elems;
  if ((e = launch_zero_words(w.sync, words, s)) != hipSuccess) return e;
  const int spin = exchange_spin_limit();
  int64_t spans_before = 0;
  for (int b0 = 0; b0 < pl.B; b0 += kMaxSeqs) {
    const int nb = std::min(kMaxSeqs, pl.B - b0);
    ScoreParams P{};
    for (int i = 0; i < nl; ++i) {
      P.q[i] = q[i];
      P.k[i] = k[i];
    }
    P.n_layers = nl;
    P.n_seqs = nb;
    P.span_chunks = xl.span_chunks;
    int items = 0;
    for (int i = 0; i < nb; ++i) {
      const Seq& sq = pl.seq[b0 + i];
      P.tok0[i] = sq.tok0;
      P.qseq[i] = b0 + i;
      P.T[i] = sq.T;
      P.C[i] = sq.C;
      P.n_span[i] = xl.n_span[b0 + i];
      P.item0[i] = items;
      P.u_off[i] = sq.u_off;
      P.st_off[i] = xl.st_off[b0 + i];
      P.s_off[i] = sq.score_off;
      P.lse_off[i] = sq.lse_off;
      items += pl.Hkv * xl.n_span[b0 + i];
    }
    P.item0[nb] = items;
    P.items_per_layer = items;
    P.u_layer_stride = pl.u_elems;
    P.st_layer_stride = xl.st_elems;
    P.s_layer_stride = pl.scores_elems;
    P.lse_layer_stride = pl.lse_elems;
    P.U = w.U;
    P.u_packed = 1;
    P.stats = w.st;
    P.lse_w = w.lse;
    P.mode = kScoreExchange;
    P.S = scores;
    P.H_q = pl.Hq;
    P.H_kv = pl.Hkv;
    P.G = pl.G;
    P.w = pl.w;
    P.c = pl.c;
    P.d = pl.d;
    P.R = pl.R;
    P.R_pad = pl.R_pad;
    P.n_rb = pl.n_rb;
    P.kv_st = pl.kv_st;
    P.kv_sh = pl.kv_sh;
    P.q_ss = pl.q_ss;
    P.q_sr = pl.q_sr;
    P.q_sh = pl.q_sh;
    P.scale = static_cast<float>(1.4426950408889634 / std::sqrt(static_cast<double>(pl.d)));
    P.rebase_raw = kRebaseLog2 / P.scale;
    int max_round = 0;
    P.n_rounds = pack_rounds(pl, xl.n_span, b0, nb, nl, slots, P.round_start, &max_round);
    P.spin_limit = spin;
    P.sync = w.sync + static_cast<int64_t>(nl) * b0 * pl.Hkv * kSyncWords;
    P.spill = w.spill + static_cast<int64_t>(nl) * spans_before;
    for (int i = 0; i < nb; ++i) spans_before += static_cast<int64_t>(pl.Hkv) * xl.n_span[b0 + i];
    // persistent grid: the largest round, a multiple of 8 (positions are
    // dealt XCD by XCD), at most the resident workgroups
    const int grid = std::min(slots, (max_round + 7) / 8 * 8);
    if ((e = launch_score_mfma(P, grid, s, ev_start, ev_stop)) != hipSuccess) return e;
  }
  return hipSuccess;
}

// Scores of nl scoring layers: the exchange kernel where it applies (xl.ok
// and the device holds a round's spans), else chunk partials then the
// log-sum-exp combine, or (pl.two_pass) statistics, row statistics and a
// final pass over the keys.  ev_start / ev_stop: at the score kernel's own
// start and end (one sequence batch, a single-launch score phase), or null.
hipError_t run_scores(const Plan& pl, const XLayout& xl, int nl, const void* const* q, const void* const* k,
                      const Work& w, float* scores, hipStream_t s, hipEvent_t ev_start = nullptr,
                      hipEvent_t ev_stop = nullptr) {
  hipError_t e;
  if (xl.ok) {
    e = run_exchange(pl, xl, nl, q, k, w, scores, s, ev_start, ev_stop);
    if (e != hipErrorNotSupported) return e;
  }
  if (!pl.two_pass) {
    if ((e = run_score(pl, nl, q, k, w.U, w.st, s, ev_start, ev_stop)) != hipSuccess) return e;
    return run_combine(pl, nl, w.U, w.st, w.lse, scores, s);
  }
  if ((e = run_score(pl, nl, q, k, w.U, w.st, s, nullptr, nullptr, kScoreStats)) != hipSuccess) return e;
  if ((e = run_combine(pl, nl, w.U, w.st, w.lse, scores, s, true)) != hipSuccess) return e;
  return run_score(pl, nl, q, k, w.U, w.st, s, nullptr, nullptr, kScoreFinal, w.lse, scores);
}

// Selection parameters of nl scoring layers of sequences [b0, b0 + nb).
SelectParams select_params(const Plan& pl, int nl, int b0, int nb, const float* scores, int32_t* indices,
                           int32_t* lengths) {
  SelectParams P{};
  P.n_layers = nl;
  P.n_seqs = nb;
  P.H_kv = pl.Hkv;
  P.w = pl.w;
  P.c = pl.c;
  for (int i = 0; i < nb; ++i) {
    const Seq& sq = pl.seq[b0 + i];
    P.T[i] = sq.T;
    P.C[i] = sq.C;
    P.kk[i] = sq.kk;
    P.L_cap[i] = sq.L_cap;
    P.len_off[i] = (b0 + i) * pl.Hkv;
    P.score_off[i] = sq.score_off;
    P.index_off[i] = sq.index_off;
  }
  P.score_layer_stride = pl.scores_elems;
  P.index_layer_stride = pl.index_elems;
  P.len_layer_stride = pl.length_elems;
  P.scores = scores;
  P.indices = indices;
  P.lengths = lengths;
  return P;
}

hipError_t run_select(const Plan& pl, int nl, const float* scores, int32_t* indices, int32_t* lengths,
                      hipStream_t s) {
  for (int b0 = 0; b0 < pl.B; b0 += kMaxSeqs) {
    const int nb = std::min(kMaxSeqs, pl.B - b0);
    const hipError_t e = launch_select(select_params(pl, nl, b0, nb, scores, indices, lengths), nl * nb * pl.Hkv, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Gather parameters of nl layers of sequences [b0, b0 + nb); layer i reads
// index block blocks[i].
GatherParams gather_params(const Plan& pl, int nl, const void* const* k, const void* const* v, void* const* ko,
                           void* const* vo, const int32_t* blocks, const int32_t* indices, const int32_t* lengths,
                           int b0, int nb) {
  GatherParams P{};
  for (int i = 0; i < nl; ++i) {
    P.k[i] = k[i];
    P.v[i] = v[i];
    P.ko[i] = ko[i];
    P.vo[i] = vo[i];
    P.idx_block[i] = blocks[i];
  }
  P.n_layers = nl;
  P.n_seqs = nb;
  P.H_kv = pl.Hkv;
  int items = 0;
  for (int i = 0; i < nb; ++i) {
    const Seq& sq = pl.seq[b0 + i];
    P.tok0[i] = sq.tok0;
    P.T[i] = sq.T;
    P.L_cap[i] = sq.L_cap;
    P.len_off[i] = (b0 + i) * pl.Hkv;
    P.item0[i] = items;
    P.blocks_per_head[i] = (sq.L_cap + kGatherRows - 1) / kGatherRows;
    P.index_off[i] = sq.index_off;
    items += pl.Hkv * P.blocks_per_head[i];
  }
  P.item0[nb] = items;
  P.items_per_layer = items;
  P.index_layer_stride = pl.index_elems;
  P.len_layer_stride = pl.length_elems;
  P.indices = indices;
  P.lengths = lengths;
  P.row_bytes = pl.d * pl.eb;
  P.kv_st_bytes = pl.kv_st * pl.eb;
  P.kv_sh_bytes = pl.kv_sh * pl.eb;
  return P;
}

// Gathers layers [l0, l0 + nl); layer l reads index block blocks[l - l0].
hipError_t run_gather(const Plan& pl, int nl, const void* const* k, const void* const* v,
                      void* const* ko, void* const* vo, const int32_t* blocks, const int32_t* indices,
                      const int32_t* lengths, hipStream_t s, hipEvent_t ev_start = nullptr,
                      hipEvent_t ev_stop = nullptr) {
  for (int b0 = 0; b0 < pl.B; b0 += kMaxSeqs) {
    const int nb = std::min(kMaxSeqs, pl.B - b0);
    const GatherParams P = gather_params(pl, nl, k, v, ko, vo, blocks, indices, lengths, b0, nb);
    const hipError_t e = launch_gather(P, nl * P.items_per_layer, s, ev_start, ev_stop);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

int check_ws(const Plan& pl, const void* ws, size_t ws_bytes, int nl) {
  if (!ws) return fail(CHUNKKV_ERR_WORKSPACE, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(ws) % kAlign)
    return fail(CHUNKKV_ERR_WORKSPACE, "workspace must be %zu-byte aligned", kAlign);
  const size_t need = ws_need(pl, nl);
  if (ws_bytes < need)
    return fail(CHUNKKV_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, need);
  return CHUNKKV_OK;
}

size_t decode_ws_bytes(const Plan& pl) {
  const int rpb = decode_rows_per_block(pl);
  int64_t blocks = 0;
  for (const Seq& sq : pl.seq) blocks += static_cast<int64_t>(pl.Hkv) * ((sq.L_cap + rpb - 1) / rpb);
  return align_up(static_cast<size_t>(blocks) * pl.G * (pl.d + kPartHead) * sizeof(float));
}

int check_decode_args(const void* q_dec, const void* k_out, const void* v_out, const int32_t* lengths,
                      const float* out) {
  if (!q_dec || !k_out || !v_out || !lengths || !out)
    return fail(CHUNKKV_ERR_INVALID_ARG, "q_dec, k_out, v_out, lengths and out must be non-NULL");
  if (!aligned16(q_dec) || !aligned16(k_out) || !aligned16(v_out) || reinterpret_cast<uintptr_t>(out) % 4)
    return fail(CHUNKKV_ERR_UNSUPPORTED, "q_dec, k_out, v_out and the workspace must be 16-byte aligned");
  return CHUNKKV_OK;
}

// Decode attention with the partial records in `part` (at least
// decode_ws_bytes(pl) bytes, 16-byte aligned; every record the merge reads is
// written by the partial kernel of the same call, so its contents on entry
// do not matter).
int run_decode(const Plan& pl, const void* q_dec, const void* k_out, const void* v_out, const int32_t* lengths,
               float* out, float* part, hipStream_t s) {
  const int rpb = decode_rows_per_block(pl);
  int64_t part0 = 0;
  for (int b0 = 0; b0 < pl.B; b0 += kMaxSeqs) {
    const int nb = std::min(kMaxSeqs, pl.B - b0);
    DecodeParams P{};
    P.q = q_dec;
    P.k = k_out;
    P.v = v_out;
    P.lengths = lengths;
    P.out = out;
    P.part = part;
    P.n_seqs = nb;
    P.H_q = pl.Hq;
    P.H_kv = pl.Hkv;
    P.G = pl.G;
    P.d = pl.d;
    P.row_bytes = pl.d * pl.eb;
    P.elem_bytes = pl.eb;
    P.inv_sqrt_d = static_cast<float>(1.0 / std::sqrt(static_cast<double>(pl.d)));
    int items = 0;
    for (int i = 0; i < nb; ++i) {
      const Seq& sq = pl.seq[b0 + i];
      P.qseq[i] = b0 + i;
      P.item0[i] = items;
      P.blocks_per_head[i] = (sq.L_cap + rpb - 1) / rpb;
      P.rows_per_block[i] = rpb;
      P.L_cap[i] = sq.L_cap;
      P.len_off[i] = (b0 + i) * pl.Hkv;
      P.index_off[i] = sq.index_off;
      P.part_off[i] = part0;
      part0 += static_cast<int64_t>(pl.Hkv) * P.blocks_per_head[i];
      items += pl.Hkv * P.blocks_per_head[i];
    }
    P.item0[nb] = items;
    if (decode_lds_bytes(P) > 160 * 1024) return fail(CHUNKKV_ERR_UNSUPPORTED, "head_dim too large for decode");
    const hipError_t e = launch_decode(P, items, nb * pl.Hq, s);
    if (e != hipSuccess) return hip_fail(e, "decode launch");
  }
  return ok();
}

// ------------------------------------------------------- static scratch --
// The scratch of chunkkv_decode_attention_static: one array per GPU, held
// until the process ends.  In host code its name stands for a host-side
// placeholder, not a device address: only the address hipGetSymbolAddress
// returns for the current device (looked up once per device, on the first
// call there) is ever passed to a kernel.
constexpr size_t kStaticScratchBytes = size_t{CHUNKKV_STATIC_SCRATCH_BYTES};
__device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

// One run of consecutive layers that share a chunk size (the hybrid entry
// points): its plan and where its anchors' blocks start in the caller's
// scores / indices / lengths buffers.
struct Run {
  int l0 = 0, n = 0;
  Plan pl;
  int64_t score0 = 0, index0 = 0, length0 = 0;
};

// Splits the layers into runs of equal chunk size and plans each; n_anchor,
// the block totals and the workspace with which every run scores all its
// anchors (at most kMaxLayers) in one launch per phase.
int plan_runs(const chunkkv_problem* p, const int32_t* layer_chunk, int n_layers, int n_reuse,
              std::vector<Run>& runs, int& n_anchor, int64_t tot[3], size_t& ws) {
  if (!p) return fail(CHUNKKV_ERR_INVALID_ARG, "problem is NULL");
  if (!layer_chunk) return fail(CHUNKKV_ERR_INVALID_ARG, "layer_chunk is NULL");
  if (n_layers < 1) return fail(CHUNKKV_ERR_INVALID_ARG, "n_layers must be >= 1 (got %d)", n_layers);
  if (n_reuse < 1) return fail(CHUNKKV_ERR_INVALID_ARG, "n_reuse must be >= 1 (got %d)", n_reuse);
  runs.clear();
  n_anchor = 0;
  tot[0] = tot[1] = tot[2] = 0;
  ws = 0;
  for (int l = 0; l < n_layers;) {
    int e = l + 1;
    while (e < n_layers && layer_chunk[e] == layer_chunk[l]) ++e;
    Run r;
    r.l0 = l;
    r.n = e - l;
    chunkkv_problem q = *p;
    q.chunk = layer_chunk[l];
    const int rc = make_plan(&q, r.pl);
    if (rc) return fail(rc, "layers %d-%d (chunk %d): %s", l, e - 1, layer_chunk[l], g_err.c_str());
    r.score0 = tot[0];
    r.index0 = tot[1];
    r.length0 = tot[2];
    const int na = (r.n + n_reuse - 1) / n_reuse;
    n_anchor += na;
    tot[0] += na * r.pl.scores_elems;
    tot[1] += na * r.pl.index_elems;
    tot[2] += na * r.pl.length_elems;
    ws = std::max(ws, ws_need(r.pl, std::min(na, kMaxLayers)));
    runs.push_back(std::move(r));
    l = e;
  }
  return CHUNKKV_OK;
}

// Records phase event i (if any) on stream s.
hipError_t record_event(void* const* events, int i, hipStream_t s) {
  return events && events[i] ? hipEventRecord(static_cast<hipEvent_t>(events[i]), s) : hipSuccess;
}

// Algorithm 2's scoring half over n_layers layers of one plan: the anchors'
// scores and selections, as many anchors per launch as the workspace holds.
// Phase events 0 and 1 (events may be NULL) bracket the scoring: a scoring
// phase that is one launch of the MFMA score kernel takes them at that
// kernel's own start and end; otherwise they are recorded between kernels
// (entry 1 after the first batch's scores when there is one batch, after the
// last selection when there are several).
hipError_t score_select_run(const Plan& pl, int n_layers, int n_reuse, const void* const* q_win,
                            const void* const* k, float* scores, int32_t* indices, int32_t* lengths,
                            void* workspace, size_t workspace_bytes, hipStream_t s, void* const* events) {
  const int n_anchor = (n_layers + n_reuse - 1) / n_reuse;
  int batch = std::min(n_anchor, kMaxLayers);
  while (batch > 1 && ws_need(pl, batch) > workspace_bytes) --batch;
  const XLayout xl = xlayout(pl, batch);   // the last, shorter launch keeps this span layout
  const Work w = carve(pl, batch, xl, workspace);
  const bool one_batch = n_anchor <= batch;
  const bool score_events = events && one_batch && pl.mfma && !pl.two_pass && pl.B <= kMaxSeqs;
  auto ev = [&](int i) { return events ? static_cast<hipEvent_t>(events[i]) : nullptr; };
  hipError_t e = score_events ? hipSuccess : record_event(events, 0, s);
  if (e != hipSuccess) return e;
  const void* qb[kMaxLayers];
  const void* kb[kMaxLayers];
  for (int a0 = 0; a0 < n_anchor; a0 += batch) {
    const int na = std::min(batch, n_anchor - a0);
    for (int i = 0; i < na; ++i) {
      qb[i] = q_win[(a0 + i) * n_reuse];
      kb[i] = k[(a0 + i) * n_reuse];
    }
    float* sc = scores + a0 * pl.scores_elems;
    // the score phase: the exchange kernel, or chunk partials and their
    // combine, or the two passes over the keys
    e = score_events ? run_scores(pl, xl, na, qb, kb, w, sc, s, ev(0), ev(1)) : run_scores(pl, xl, na, qb, kb, w, sc, s);
    if (e != hipSuccess) return e;
    if (one_batch && !score_events && (e = record_event(events, 1, s)) != hipSuccess) return e;
    e = run_select(pl, na, sc, indices + a0 * pl.index_elems, lengths + a0 * pl.length_elems, s);
    if (e != hipSuccess) return e;
  }
  return one_batch ? hipSuccess : record_event(events, 1, s);
}

// Algorithm 2's gather half: layer l of the run copies its own K/V rows with
// the indices of anchor floor(l / n_reuse).  Phase events 2 and 3 (events may
// be NULL) bracket it, at the kernel's own start and end when the gather is
// one launch.
hipError_t gather_run(const Plan& pl, int n_layers, int n_reuse, const void* const* k, const void* const* v,
                      void* const* ko, void* const* vo, const int32_t* indices, const int32_t* lengths,
                      hipStream_t s, void* const* events) {
  const bool gather_events = events && n_layers <= kMaxLayers && pl.B <= kMaxSeqs;
  auto ev = [&](int i) { return events ? static_cast<hipEvent_t>(events[i]) : nullptr; };
  hipError_t e = gather_events ? hipSuccess : record_event(events, 2, s);
  if (e != hipSuccess) return e;
  int32_t blocks[kMaxLayers];
  for (int l0 = 0; l0 < n_layers; l0 += kMaxLayers) {
    const int nl = std::min(kMaxLayers, n_layers - l0);
    for (int i = 0; i < nl; ++i) blocks[i] = (l0 + i) / n_reuse;
    e = gather_events ? run_gather(pl, nl, k + l0, v + l0, ko + l0, vo + l0, blocks, indices, lengths, s, ev(2), ev(3))
                      : run_gather(pl, nl, k + l0, v + l0, ko + l0, vo + l0, blocks, indices, lengths, s);
    if (e != hipSuccess) return e;
  }
  return gather_events ? hipSuccess : record_event(events, 3, s);
}

hipError_t static_scratch(float** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* ptr = nullptr;
    if ((e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch))) != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    g_scratch_dev[dev] = ptr;
  }
  *out = static_cast<float*>(g_scratch_dev[dev]);
  return hipSuccess;
}

}  // namespace

extern "C" {

int chunkkv_plan(const chunkkv_problem* p, chunkkv_sizes* out, int64_t* score_off, int64_t* index_off,
                 int64_t* l_cap) {
  Plan pl;
  const int rc = make_plan(p, pl);
  if (rc) return rc;
  if (!out) return fail(CHUNKKV_ERR_INVALID_ARG, "sizes output is NULL");
  out->scores_elems = pl.scores_elems;
  out->index_elems = pl.index_elems;
  out->length_elems = pl.length_elems;
  out->workspace_bytes = ws_need(pl, 1);
  for (int b = 0; b < pl.B; ++b) {
    if (score_off) score_off[b] = pl.seq[b].score_off;
    if (index_off) index_off[b] = pl.seq[b].index_off;
    if (l_cap) l_cap[b] = pl.seq[b].L_cap;
  }
  return ok();
}

size_t chunkkv_workspace_bytes(const chunkkv_problem* p, int32_t n_score_layers) {
  Plan pl;
  if (make_plan(p, pl) || n_score_layers < 1) return 0;
  return ws_need(pl, std::min<int32_t>(n_score_layers, kMaxLayers));
}

int chunkkv_score(const chunkkv_problem* p, const void* q_win, const void* k, float* scores, void* workspace,
                  size_t workspace_bytes, void* stream) {
  Plan pl;
  int rc = make_plan(p, pl);
  if (rc) return rc;
  if (!q_win || !k || !scores) return fail(CHUNKKV_ERR_INVALID_ARG, "q_win, k and scores must be non-NULL");
  if (!aligned16(q_win) || !aligned16(k) || reinterpret_cast<uintptr_t>(scores) % 4)
    return fail(CHUNKKV_ERR_UNSUPPORTED, "q_win and k must be 16-byte aligned");
  if ((rc = check_ws(pl, workspace, workspace_bytes, 1))) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const XLayout xl = xlayout(pl, 1);
  hipError_t e = run_scores(pl, xl, 1, &q_win, &k, carve(pl, 1, xl, workspace), scores, s);
  if (e != hipSuccess) return hip_fail(e, "score launch");
  return ok();
}

int chunkkv_select(const chunkkv_problem* p, const float* scores, int32_t* indices, int32_t* lengths,
                   void* stream) {
  Plan pl;
  const int rc = make_plan(p, pl);
  if (rc) return rc;
  if (!scores || !indices || !lengths)
    return fail(CHUNKKV_ERR_INVALID_ARG, "scores, indices and lengths must be non-NULL");
  const hipError_t e = run_select(pl, 1, scores, indices, lengths, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "select launch");
  return ok();
}

int chunkkv_gather(const chunkkv_problem* p, const void* k, const void* v, const int32_t* indices,
                   const int32_t* lengths, void* k_out, void* v_out, void* stream) {
  Plan pl;
  const int rc = make_plan(p, pl);
  if (rc) return rc;
  if (!k || !v || !indices || !lengths || !k_out || !v_out)
    return fail(CHUNKKV_ERR_INVALID_ARG, "k, v, indices, lengths, k_out and v_out must be non-NULL");
  if (!aligned16(k) || !aligned16(v) || !aligned16(k_out) || !aligned16(v_out))
    return fail(CHUNKKV_ERR_UNSUPPORTED, "K/V buffers must be 16-byte aligned");
  const int32_t blk = 0;
  const hipError_t e = run_gather(pl, 1, &k, &v, &k_out, &v_out, &blk, indices, lengths,
                                  static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "gather launch");
  return ok();
}

int chunkkv_gather_paged(const chunkkv_problem* p, const void* k, const void* v, const int32_t* indices,
                         const int32_t* lengths, const int32_t* block_table, int32_t max_pages, int32_t page_rows,
                         int64_t n_pages, void* k_pages, void* v_pages, void* stream) {
  Plan pl;
  const int rc = make_plan(p, pl);
  if (rc) return rc;
  if (!k || !v || !indices || !lengths || !block_table || !k_pages || !v_pages)
    return fail(CHUNKKV_ERR_INVALID_ARG, "k, v, indices, lengths, block_table, k_pages and v_pages must be non-NULL");
  if (page_rows < 1 || max_pages < 1 || n_pages < 1)
    return fail(CHUNKKV_ERR_INVALID_ARG, "page_rows, max_pages and n_pages must be >= 1 (got %d, %d, %lld)",
                page_rows, max_pages, static_cast<long long>(n_pages));
  if (!aligned16(k) || !aligned16(v) || !aligned16(k_pages) || !aligned16(v_pages))
    return fail(CHUNKKV_ERR_UNSUPPORTED, "K/V buffers and pages must be 16-byte aligned");
  for (int b = 0; b < pl.B; ++b) {
    const int64_t need = (static_cast<int64_t>(pl.seq[b].L_cap) + page_rows - 1) / page_rows;
    if (need > max_pages)
      return fail(CHUNKKV_ERR_INVALID_ARG, "sequence %d keeps up to %d rows: needs %lld pages of %d rows, max_pages is %d",
                  b, pl.seq[b].L_cap, static_cast<long long>(need), page_rows, max_pages);
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (int b0 = 0; b0 < pl.B; b0 += kMaxSeqs) {
    const int nb = std::min(kMaxSeqs, pl.B - b0);
    PagedParams P{};
    P.k = k;
    P.v = v;
    P.kp = k_pages;
    P.vp = v_pages;
    P.indices = indices;
    P.lengths = lengths;
    P.block_table = block_table;
    P.n_seqs = nb;
    P.H_kv = pl.Hkv;
    P.page_rows = page_rows;
    P.max_pages = max_pages;
    P.n_pages = n_pages;
    int items = 0;
    for (int i = 0; i < nb; ++i) {
      const Seq& sq = pl.seq[b0 + i];
      P.tok0[i] = sq.tok0;
      P.T[i] = sq.T;
      P.L_cap[i] = sq.L_cap;
      P.len_off[i] = (b0 + i) * pl.Hkv;
      P.item0[i] = items;
      P.blocks_per_head[i] = (sq.L_cap + kGatherRows - 1) / kGatherRows;
      P.index_off[i] = sq.index_off;
      items += pl.Hkv * P.blocks_per_head[i];
    }
    P.item0[nb] = items;
    P.row_bytes = pl.d * pl.eb;
    P.kv_st_bytes = pl.kv_st * pl.eb;
    P.kv_sh_bytes = pl.kv_sh * pl.eb;
    const hipError_t e = launch_gather_paged(P, items, s);
    if (e != hipSuccess) return hip_fail(e, "paged gather launch");
  }
  return ok();
}

int chunkkv_compress_layers(const chunkkv_problem* p, int32_t n_layers, int32_t n_reuse,
                            const void* const* q_win, const void* const* k, const void* const* v,
                            void* const* k_out, void* const* v_out, float* scores, int32_t* indices,
                            int32_t* lengths, void* workspace, size_t workspace_bytes, void* stream,
                            void* const* phase_events) {
  Plan pl;
  int rc = make_plan(p, pl);
  if (rc) return rc;
  if (n_layers < 1) return fail(CHUNKKV_ERR_INVALID_ARG, "n_layers must be >= 1 (got %d)", n_layers);
  if (n_reuse < 1) return fail(CHUNKKV_ERR_INVALID_ARG, "n_reuse must be >= 1 (got %d)", n_reuse);
  if (!q_win || !k || !v || !k_out || !v_out)
    return fail(CHUNKKV_ERR_INVALID_ARG, "pointer tables must be non-NULL");
  if (!scores || !indices || !lengths)
    return fail(CHUNKKV_ERR_INVALID_ARG, "scores, indices and lengths must be non-NULL");
  for (int l = 0; l < n_layers; ++l) {
    if (l % n_reuse == 0 && !q_win[l])
      return fail(CHUNKKV_ERR_INVALID_ARG, "q_win[%d] is NULL on a scoring layer", l);
    if (!k[l] || !v[l] || !k_out[l] || !v_out[l])
      return fail(CHUNKKV_ERR_INVALID_ARG, "a K/V pointer of layer %d is NULL", l);
    if ((l % n_reuse == 0 && !aligned16(q_win[l])) || !aligned16(k[l]) || !aligned16(v[l]) ||
        !aligned16(k_out[l]) || !aligned16(v_out[l]))
      return fail(CHUNKKV_ERR_UNSUPPORTED, "buffers of layer %d must be 16-byte aligned", l);
  }
  if ((rc = check_ws(pl, workspace, workspace_bytes, 1))) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = score_select_run(pl, n_layers, n_reuse, q_win, k, scores, indices, lengths, workspace,
                                  workspace_bytes, s, phase_events);
  if (e != hipSuccess) return hip_fail(e, "score / select launch");
  if ((e = gather_run(pl, n_layers, n_reuse, k, v, k_out, v_out, indices, lengths, s, phase_events)) != hipSuccess)
    return hip_fail(e, "gather launch");
  return ok();
}

int chunkkv_plan_hybrid(const chunkkv_problem* p, const int32_t* layer_chunk, int32_t n_layers, int32_t n_reuse,
                        int32_t* n_anchor, int64_t* score_block_off, int64_t* index_block_off,
                        int64_t* length_block_off, int64_t* kv_out_rows, size_t* workspace_bytes) {
  std::vector<Run> runs;
  int na = 0;
  int64_t tot[3];
  size_t ws = 0;
  const int rc = plan_runs(p, layer_chunk, n_layers, n_reuse, runs, na, tot, ws);
  if (rc) return rc;
  if (n_anchor) *n_anchor = na;
  if (workspace_bytes) *workspace_bytes = ws;
  int a = 0;
  for (const Run& r : runs) {
    for (int i = 0; i < (r.n + n_reuse - 1) / n_reuse; ++i, ++a) {
      if (score_block_off) score_block_off[a] = r.score0 + i * r.pl.scores_elems;
      if (index_block_off) index_block_off[a] = r.index0 + i * r.pl.index_elems;
      if (length_block_off) length_block_off[a] = r.length0 + i * r.pl.length_elems;
    }
    if (kv_out_rows)
      for (int l = r.l0; l < r.l0 + r.n; ++l) kv_out_rows[l] = r.pl.index_elems;
  }
  if (score_block_off) score_block_off[na] = tot[0];
  if (index_block_off) index_block_off[na] = tot[1];
  if (length_block_off) length_block_off[na] = tot[2];
  return ok();
}

int chunkkv_compress_layers_hybrid(const chunkkv_problem* p, const int32_t* layer_chunk, int32_t n_layers,
                                   int32_t n_reuse, const void* const* q_win, const void* const* k,
                                   const void* const* v, void* const* k_out, void* const* v_out, float* scores,
                                   int32_t* indices, int32_t* lengths, void* workspace, size_t workspace_bytes,
                                   void* stream, void* const* phase_events) {
  std::vector<Run> runs;
  int na = 0;
  int64_t tot[3];
  size_t ws = 0;
  int rc = plan_runs(p, layer_chunk, n_layers, n_reuse, runs, na, tot, ws);
  if (rc) return rc;
  if (!q_win || !k || !v || !k_out || !v_out)
    return fail(CHUNKKV_ERR_INVALID_ARG, "pointer tables must be non-NULL");
  if (!scores || !indices || !lengths)
    return fail(CHUNKKV_ERR_INVALID_ARG, "scores, indices and lengths must be non-NULL");
  for (const Run& r : runs)
    for (int l = r.l0; l < r.l0 + r.n; ++l) {
      const bool anchor = (l - r.l0) % n_reuse == 0;
      if (anchor && !q_win[l]) return fail(CHUNKKV_ERR_INVALID_ARG, "q_win[%d] is NULL on a scoring layer", l);
      if (!k[l] || !v[l] || !k_out[l] || !v_out[l])
        return fail(CHUNKKV_ERR_INVALID_ARG, "a K/V pointer of layer %d is NULL", l);
      if ((anchor && !aligned16(q_win[l])) || !aligned16(k[l]) || !aligned16(v[l]) || !aligned16(k_out[l]) ||
          !aligned16(v_out[l]))
        return fail(CHUNKKV_ERR_UNSUPPORTED, "buffers of layer %d must be 16-byte aligned", l);
    }
  for (const Run& r : runs)
    if ((rc = check_ws(r.pl, workspace, workspace_bytes, 1))) return rc;

  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = record_event(phase_events, 0, s);
  if (e != hipSuccess) return hip_fail(e, "phase event");
  for (const Run& r : runs)
    if ((e = score_select_run(r.pl, r.n, n_reuse, q_win + r.l0, k + r.l0, scores + r.score0, indices + r.index0,
                              lengths + r.length0, workspace, workspace_bytes, s, nullptr)) != hipSuccess)
      return hip_fail(e, "score / select launch");
  if ((e = record_event(phase_events, 1, s)) != hipSuccess || (e = record_event(phase_events, 2, s)) != hipSuccess)
    return hip_fail(e, "phase event");
  for (const Run& r : runs)
    if ((e = gather_run(r.pl, r.n, n_reuse, k + r.l0, v + r.l0, k_out + r.l0, v_out + r.l0, indices + r.index0,
                        lengths + r.length0, s, nullptr)) != hipSuccess)
      return hip_fail(e, "gather launch");
  if ((e = record_event(phase_events, 3, s)) != hipSuccess) return hip_fail(e, "phase event");
  return ok();
}

size_t chunkkv_decode_workspace_bytes(const chunkkv_problem* p) {
  Plan pl;
  if (make_plan(p, pl)) return 0;
  return decode_ws_bytes(pl);
}

int chunkkv_decode_attention(const chunkkv_problem* p, const void* q_dec, const void* k_out, const void* v_out,
                             const int32_t* lengths, float* out, void* workspace, size_t workspace_bytes,
                             void* stream) {
  Plan pl;
  int rc = make_plan(p, pl);
  if (rc) return rc;
  if ((rc = check_decode_args(q_dec, k_out, v_out, lengths, out))) return rc;
  if (workspace && !aligned16(workspace))
    return fail(CHUNKKV_ERR_UNSUPPORTED, "q_dec, k_out, v_out and the workspace must be 16-byte aligned");
  const size_t need = decode_ws_bytes(pl);
  if (!workspace || workspace_bytes < need)
    return fail(CHUNKKV_ERR_WORKSPACE, "decode workspace has %zu bytes, needs %zu", workspace ? workspace_bytes : 0,
                need);
  return run_decode(pl, q_dec, k_out, v_out, lengths, out, static_cast<float*>(workspace),
                    static_cast<hipStream_t>(stream));
}

int chunkkv_decode_attention_static(const chunkkv_problem* p, const void* q_dec, const void* k_out,
                                    const void* v_out, const int32_t* lengths, float* out, void* stream) {
  Plan pl;
  int rc = make_plan(p, pl);
  if (rc) return rc;
  if ((rc = check_decode_args(q_dec, k_out, v_out, lengths, out))) return rc;
  const size_t need = decode_ws_bytes(pl);
  if (need > kStaticScratchBytes)
    return fail(CHUNKKV_ERR_WORKSPACE, "decode needs %zu bytes of scratch, the static scratch holds %zu", need,
                kStaticScratchBytes);
  float* ws = nullptr;
  const hipError_t e = static_scratch(&ws);
  if (e != hipSuccess) return hip_fail(e, "static scratch address");
  return run_decode(pl, q_dec, k_out, v_out, lengths, out, ws, static_cast<hipStream_t>(stream));
}

const char* chunkkv_last_error(void) { return g_err.c_str(); }

}  // extern "C"
