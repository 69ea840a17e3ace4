// Internal definitions shared by the HIP kernels and the host side of
// libchunkkv.so (gfx950 / CDNA4).  Not part of the C-ABI.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ckv {

// Per-launch table limits: layer pointers and per-sequence geometry travel in
// kernel arguments; the host splits larger problems into several launches.
constexpr int kMaxLayers = 32;
constexpr int kMaxSeqs = 8;

constexpr int kThreads = 256;            // every kernel: 4 wave64s per workgroup
constexpr int kMfmaRows = 128;           // query rows (G*w) per MFMA score workgroup
#ifndef CKV_GATHER_ROWS
#define CKV_GATHER_ROWS 32
#endif
#ifndef CKV_SPAN_TARGET
#define CKV_SPAN_TARGET 64
#endif
#ifndef CKV_MAX_TILES
#define CKV_MAX_TILES 4
#endif
#ifndef CKV_STAGE_TILES
#define CKV_STAGE_TILES 4
#endif
#ifndef CKV_MIN_WAVES
#define CKV_MIN_WAVES 2
#endif
#ifndef CKV_XCH_WAVES
#define CKV_XCH_WAVES 3
#endif
constexpr int kGatherRows = CKV_GATHER_ROWS;   // output rows per gather workgroup
constexpr int kSpanTarget = CKV_SPAN_TARGET;   // chunks per MFMA score work item (LDS-resident)
constexpr int kMaxTiles = CKV_MAX_TILES;       // 32-slot MFMA tiles per group, at most
constexpr int kStageTiles = CKV_STAGE_TILES;   // key tiles in flight per workgroup (register ring)

// A chunk-partial reference is rebased only when a new maximum exceeds the
// current reference by this many powers of two; below that, exp2 of the
// difference stays far inside fp32 range (2^64 * tokens << FLT_MAX).
constexpr float kRebaseLog2 = 64.0f;

// ------------------------------------------------- chunk-partial storage --
// Chunk partials U (non-negative fp32) of bf16 problems are stored in 24
// bits: the sign bit (always 0) dropped and the mantissa rounded to 16 bits
// (relative error at most 2^-17, far inside the 1e-3 bound of bf16 inputs),
// four values in three 32-bit words.  fp32 problems keep fp32 partials (their
// bound is 1e-5).  A U row of R_pad values (R_pad a multiple of 4) takes
// u_row_words(R_pad, packed) words; U offsets and strides count words.
__host__ __device__ inline int64_t u_row_words(int64_t R_pad, bool packed) { return packed ? R_pad / 4 * 3 : R_pad; }

typedef unsigned int u32x3v __attribute__((ext_vector_type(3)));
// three words at a 4-byte aligned address of U (12-byte accesses)
typedef unsigned int u32x3u __attribute__((ext_vector_type(3), aligned(4)));
__device__ __forceinline__ uint32_t u24_of(float x) { return (__float_as_uint(x) + 0x40u) >> 7; }
__device__ __forceinline__ float f_of_u24(uint32_t v) { return __uint_as_float(v << 7); }
__device__ __forceinline__ float round_u24(float x) { return f_of_u24(u24_of(x)); }
__device__ __forceinline__ u32x3v pack_u24(float a, float b, float c, float d) {
  const uint32_t A = u24_of(a), B = u24_of(b), C = u24_of(c), D = u24_of(d);
  return u32x3v{A | (B << 24), (B >> 8) | (C << 16), (C >> 16) | (D << 8)};
}
__device__ __forceinline__ float4 unpack_u24(u32x3v w) {
  return make_float4(f_of_u24(w.x & 0xFFFFFFu), f_of_u24((w.x >> 24) | ((w.y & 0xFFFFu) << 8)),
                     f_of_u24((w.y >> 16) | ((w.z & 0xFFu) << 16)), f_of_u24(w.z >> 8));
}

// ----------------------------------------------------------------- score --
// One launch scores up to kMaxLayers layers x kMaxSeqs sequences.  Work item
// = (layer, sequence b, KV head h, row block rb, span s); a span is a run of
// span_chunks whole chunks.  In mode kScorePartials each item writes
//   U[layer][u_off[b] + (h*C_b + j)*u_row_words + row r]  chunk partials
//   stats[layer][st_off[b] + (h*n_span_b + s)*R_pad + r] = (m_ref, l)
// where U is sum over the chunk's tokens of exp2((x - m_ref)*scale) and l
// is sum over the span of the same terms.  Short chunks (two passes over the
// keys, one row block): mode kScoreStats writes the statistics only, and
// after the row statistics (M_r, L_r) exist, mode kScoreFinal writes
//   S[layer][s_off[b] + h*C_b + j] = sum_r sum_{t in j} 2^((x - M_r)*scale) / L_r.
constexpr int kScorePartials = 0;
constexpr int kScoreStats = 1;
constexpr int kScoreFinal = 2;
// Mode kScoreExchange (one row block per head): the spans of a head run in
// the same round of a persistent launch; each keeps its chunk partials in
// LDS, publishes (m_ref, l) per row into stats, and the last span of the head
// to arrive forms (M_r, L_r) into lse and raises the head's ready flag; every
// span then writes its own chunk scores S from its LDS partials.  A span
// whose wait for the flag runs out writes its partials to U instead (and
// marks itself in spill); the last span of the head to finish scores the
// marked spans from U with the same arithmetic.
constexpr int kScoreExchange = 3;
constexpr int kMaxRounds = 64;         // rounds of one exchange launch
// Per-head words of an exchange launch: arrivals, finished spans, ready flag.
constexpr int kSyncWords = 4;

struct ScoreParams {
  const void* q[kMaxLayers];
  const void* k[kMaxLayers];
  int32_t n_layers;
  int32_t n_seqs;
  int32_t items_per_layer;
  int32_t span_chunks;
  // MFMA path work split: each unit (layer, b, h, row block) of sequence b
  // is cut into wpu[b] balanced span ranges, one per workgroup
  int32_t wpu[kMaxSeqs];
  int32_t worker0[kMaxSeqs + 1];
  int32_t workers_per_layer;
  // row blocks of one (head, span range) on workgroup ids 8 apart (one XCD),
  // so the blocks' key reads meet in that XCD's L2
  int32_t rb_interleave;
  int64_t tok0[kMaxSeqs];       // first K/V token row of sequence b
  int32_t qseq[kMaxSeqs];       // sequence index for q_stride_seq
  int32_t T[kMaxSeqs];
  int32_t C[kMaxSeqs];
  int32_t n_span[kMaxSeqs];
  int32_t item0[kMaxSeqs + 1];  // first item of sequence b within a layer
  int64_t u_off[kMaxSeqs];       // U offsets and strides in 32-bit words
  int64_t st_off[kMaxSeqs];
  int64_t u_layer_stride;
  int64_t st_layer_stride;
  float* U;                     // 32-bit words: packed 24-bit partials when u_packed
  int32_t u_packed;
  float2* stats;
  int32_t mode;                 // kScorePartials, kScoreStats or kScoreFinal
  float* S;                     // kScoreFinal: chunk scores
  const float2* lse;            // kScoreFinal: row statistics (M_r, L_r), [H_kv][R_pad] per sequence
  int64_t s_off[kMaxSeqs];
  int64_t lse_off[kMaxSeqs];
  int64_t s_layer_stride, lse_layer_stride;
  int32_t H_q, H_kv, G, w, c, d, R, R_pad, n_rb;
  int64_t kv_st, kv_sh, q_ss, q_sr, q_sh;
  float scale;                  // log2(e) / sqrt(d)
  float rebase_raw;             // kRebaseLog2 / scale
  // kScoreExchange: round r holds the items [round_start[r], round_start[r+1])
  // (whole heads); the workgroup at position p takes item round_start[r] + p.
  int32_t n_rounds;
  int32_t round_start[kMaxRounds + 1];
  int32_t spin_limit;           // polls of a head's ready flag before spilling
  float2* lse_w;                // written (M_r, L_r), same layout as lse
  uint32_t* sync;               // [n_layers][n_seqs * H_kv][kSyncWords], zero on entry
  uint32_t* spill;              // [n_layers * items_per_layer], zero on entry
};

// --------------------------------------------------------------- combine --
// Item = (layer, b, h, block of spans_per_blk spans): every item first forms
// the log-sum-exp (M_r, L_r) of all rows from the span statistics, then
//   S_j = sum_r U[j][r] * 2^((m_s,r - M_r)*scale) / L_r
// for the chunks of its spans.
struct CombineParams {
  int32_t n_layers;
  int32_t n_seqs;
  int32_t items_per_layer;
  int32_t span_chunks;
  int32_t spans_per_blk;
  int32_t C[kMaxSeqs];
  int32_t n_span[kMaxSeqs];
  int32_t n_blk[kMaxSeqs];      // span blocks per head
  int32_t item0[kMaxSeqs + 1];
  int64_t u_off[kMaxSeqs];
  int64_t st_off[kMaxSeqs];
  int64_t score_off[kMaxSeqs];
  int64_t lse_off[kMaxSeqs];    // per-row (M, L) of sequence b: [H_kv][R_pad] float2
  int32_t head0[kMaxSeqs + 1];  // first (sequence, head) item of sequence b in the row-statistics launch
  int32_t fuse_lse;             // 1: each combine block forms its head's (M_r, L_r) itself (no row-statistics launch)
  int64_t u_layer_stride, st_layer_stride, score_layer_stride, lse_layer_stride;   // U: 32-bit words
  const float* U;               // packed 24-bit partials when u_packed
  int32_t u_packed;
  const float2* stats;
  float2* lse;
  float* scores;
  int32_t H_kv, R, R_pad;
  float scale;
};

// ---------------------------------------------------------------- select --
// Item = (scoring layer, b, h), one workgroup of kSelectThreads: top-k
// threshold on the fp32 score bit patterns, recent-window merge, ascending
// index list.
constexpr int kSelectThreads = 1024;
constexpr int kSelectKeysPerThread = 16;   // scores held in registers: C <= 16384

struct SelectParams {
  int32_t n_layers;
  int32_t n_seqs;
  int32_t H_kv, w, c;
  int32_t T[kMaxSeqs];
  int32_t C[kMaxSeqs];
  int32_t kk[kMaxSeqs];         // floor(L_max / c)
  int32_t L_cap[kMaxSeqs];
  int32_t len_off[kMaxSeqs];    // b_global * H_kv
  int64_t score_off[kMaxSeqs];
  int64_t index_off[kMaxSeqs];
  int64_t score_layer_stride, index_layer_stride, len_layer_stride;
  const float* scores;
  int32_t* indices;
  int32_t* lengths;
};

// ---------------------------------------------------------------- gather --
// Item = (layer, b, h, block of kGatherRows output rows).
struct GatherParams {
  const void* k[kMaxLayers];
  const void* v[kMaxLayers];
  void* ko[kMaxLayers];
  void* vo[kMaxLayers];
  int32_t idx_block[kMaxLayers];  // scoring-layer block of indices/lengths
  int32_t n_layers;
  int32_t n_seqs;
  int32_t H_kv;
  int32_t items_per_layer;
  int64_t tok0[kMaxSeqs];
  int32_t T[kMaxSeqs];
  int32_t L_cap[kMaxSeqs];
  int32_t len_off[kMaxSeqs];
  int32_t item0[kMaxSeqs + 1];
  int32_t blocks_per_head[kMaxSeqs];
  int64_t index_off[kMaxSeqs];
  int64_t index_layer_stride, len_layer_stride;
  const int32_t* indices;
  const int32_t* lengths;
  int32_t row_bytes;            // head_dim * elem_bytes, multiple of 16
  int64_t kv_st_bytes, kv_sh_bytes;
};

// Host-side launchers (defined next to their kernels).
// MFMA path: bf16, head_dim 128, chunk size with a static layout.
bool score_mfma_supported(int chunk);
// Chunk sizes with the two-pass kernels (statistics, then final scores).
bool score_two_pass_supported(int chunk);
int score_mfma_span_chunks(int chunk);
// Launches min(n_items, resident workgroups) persistent workgroups.
// Launches `kernel` with one by-value argument and returns the launch's own
// status (not a sticky error left by an earlier, unrelated HIP call).
template <typename Arg>
inline hipError_t launch1(void (*kernel)(Arg), dim3 grid, dim3 block, size_t lds, hipStream_t s, Arg arg,
                          hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr) {
  void* args[] = {&arg};
  return hipExtLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, args, lds, s, ev_start, ev_stop, 0);
}

// ev_start / ev_stop (may be null) are recorded at the kernel's start and end.
hipError_t launch_score_mfma(ScoreParams p, int n_items, hipStream_t s, hipEvent_t ev_start = nullptr,
                             hipEvent_t ev_stop = nullptr);
// Exchange mode: the largest span (in chunks) whose partials fit the
// kernel's LDS ring for chunk size c (0: no exchange layout), the chunks per
// MFMA group, and the persistent grid (resident workgroups, a multiple of 8).
int score_exchange_max_span_chunks(int chunk);
int score_group_chunks(int chunk);
hipError_t score_exchange_slots(int chunk, int* slots);
// Zeroes n 32-bit words (the exchange launch's flags) on stream s.
hipError_t launch_zero_words(uint32_t* p, int64_t n, hipStream_t s);
// Generic path: any dtype / head_dim / chunk size (VALU fp32).
int score_generic_span_chunks(int R_pad, int chunk);
size_t score_generic_lds_bytes(int R_pad, int span_chunks, int d);
hipError_t launch_score_generic(const ScoreParams& p, int dtype, int n_blocks, hipStream_t s);
int combine_spans_per_blk(int R_pad);
hipError_t launch_combine(const CombineParams& p, int n_blocks, hipStream_t s);
hipError_t launch_row_lse(const CombineParams& p, int n_blocks, hipStream_t s);
hipError_t launch_select(const SelectParams& p, int n_blocks, hipStream_t s);
hipError_t launch_gather(const GatherParams& p, int n_blocks, hipStream_t s, hipEvent_t ev_start = nullptr,
                         hipEvent_t ev_stop = nullptr);

}  // namespace ckv
