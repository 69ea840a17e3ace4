// Paged output of the K/V compaction: parameters of the paged gather kernel.
// Not part of the C-ABI.
#pragma once

#include "chunkkv_internal.h"

namespace ckv {

// Item = (sequence b, KV head h, block of kGatherRows kept rows).  Kept row i
// of (b, h) goes to row i % page_rows of pool page
// block_table[(len_off[b] + h) * max_pages + i / page_rows].
struct PagedParams {
  const void* k;
  const void* v;
  void* kp;
  void* vp;
  const int32_t* indices;
  const int32_t* lengths;
  const int32_t* block_table;
  int32_t n_seqs;
  int32_t H_kv;
  int32_t page_rows;
  int32_t max_pages;
  int64_t n_pages;
  int64_t tok0[kMaxSeqs];
  int32_t T[kMaxSeqs];
  int32_t L_cap[kMaxSeqs];
  int32_t len_off[kMaxSeqs];
  int32_t item0[kMaxSeqs + 1];
  int32_t blocks_per_head[kMaxSeqs];
  int64_t index_off[kMaxSeqs];
  int32_t row_bytes;            // head_dim * elem_bytes, multiple of 16
  int64_t kv_st_bytes, kv_sh_bytes;
};

hipError_t launch_gather_paged(const PagedParams& p, int n_blocks, hipStream_t s);

}  // namespace ckv
