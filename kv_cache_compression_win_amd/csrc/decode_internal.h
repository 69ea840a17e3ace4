// Internal definitions of the decode-attention kernels (not part of the C-ABI).
#pragma once

#include "chunkkv_internal.h"

namespace ckv {

constexpr int kDecRows = 64;         // kept rows per step of a decode work item
constexpr int kDecQ = 8;             // query heads of a group handled per pass
constexpr int kPartHead = 4;         // floats before the value sums in a partial record

// Rows of 16 pieces of 16 bytes (bf16 head_dim 128, fp32 head_dim 64) take
// the one-wave path: work item = one wavefront, kWaveRows kept rows per step,
// no workgroup barriers; about kDecodeWaveItems items over the problem.
constexpr int kWavePieces = 16;
constexpr int kWaveRows = 32;
constexpr int64_t kDecodeWaveItems = 2048;
inline bool decode_wave_path(int row_bytes) { return row_bytes == 16 * kWavePieces; }

// Work item = (sequence b, KV head h, block of rows_per_block[b] kept rows, a
// multiple of the step: kDecRows per workgroup item, kWaveRows per wave item).  Partials
// part[((part_off[b] + h*blocks_per_head[b] + blk)*G + g)*(d + kPartHead) + ...] =
// (block max, block sum of exponentials, 2 unused, d unnormalised value sums):
// records and their value sums start 16-byte aligned.
struct DecodeParams {
  const void* q;                // [n_seqs][H_q][d], element type of the cache
  const void* k;                // compacted caches, rows of row_bytes
  const void* v;
  const int32_t* lengths;       // [n_seqs * H_kv]
  float* out;                   // [n_seqs][H_q][d]
  float* part;
  int32_t n_seqs, H_q, H_kv, G, d, row_bytes, elem_bytes;
  float inv_sqrt_d;
  int32_t qseq[kMaxSeqs];       // global sequence index of launch sequence b
  int32_t item0[kMaxSeqs + 1];
  int32_t blocks_per_head[kMaxSeqs];
  int32_t rows_per_block[kMaxSeqs];
  int32_t L_cap[kMaxSeqs];
  int32_t len_off[kMaxSeqs];    // b_global * H_kv
  int64_t index_off[kMaxSeqs];
  int64_t part_off[kMaxSeqs];
};

size_t decode_lds_bytes(const DecodeParams& p);
// Partial blocks (n_items work items) then the merge (one workgroup per output
// query head).
hipError_t launch_decode(const DecodeParams& p, int n_items, int n_heads_out, hipStream_t s);

}  // namespace ckv
