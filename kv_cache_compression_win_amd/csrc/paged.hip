// K/V compaction into a paged pool: the index_select of the ChunkKV page
// (section 4.1, Algorithm 1 step 6) written straight into fixed-size pages
// of consecutive KV rows, the block layout PagedAttention engines keep (Kara
// page, section 2), so such an engine takes the compressed cache with no
// further copy.  Kept row i of (sequence b, KV head h) lands in row
// i % page_rows of the page that the block table lists at position
// i / page_rows for (b, h).
//
// Work item = (sequence, KV head, block of kGatherRows kept rows); consecutive
// threads copy consecutive 16-byte pieces of a row, so reads of a source row
// and writes of a page row are contiguous runs.  A page id outside
// [0, n_pages) leaves its rows unwritten; lengths and index values are
// clamped as in the contiguous gather.
#include "paged_internal.h"

namespace ckv {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int kPagedUnroll = 2;

__global__ __launch_bounds__(kThreads) void gather_paged_kernel(const PagedParams P) {
  const int tid = threadIdx.x;
  int item = blockIdx.x;
  int b = 0;
  while (b + 1 < P.n_seqs && item >= P.item0[b + 1]) ++b;
  item -= P.item0[b];
  const int bph = P.blocks_per_head[b];
  const int h = item / bph, blk = item - h * bph;
  const int n = min(max(P.lengths[P.len_off[b] + h], 0), P.L_cap[b]);
  const int t_last = P.T[b] - 1;
  const int i0 = blk * kGatherRows;
  if (i0 >= n) return;
  const int nrows = min(kGatherRows, n - i0);
  const int upr = P.row_bytes >> 4;
  const int total = nrows * upr;

  const int32_t* idx = P.indices + P.index_off[b] + static_cast<int64_t>(h) * P.L_cap[b] + i0;
  const int32_t* table = P.block_table + static_cast<int64_t>(P.len_off[b] + h) * P.max_pages;
  const int64_t src_off = P.tok0[b] * P.kv_st_bytes + static_cast<int64_t>(h) * P.kv_sh_bytes;
  const char* ks = static_cast<const char*>(P.k) + src_off;
  const char* vs = static_cast<const char*>(P.v) + src_off;
  char* kd = static_cast<char*>(P.kp);
  char* vd = static_cast<char*>(P.vp);

  for (int u0 = 0; u0 < total; u0 += kThreads * kPagedUnroll) {
    u32x4 kv[kPagedUnroll], vv[kPagedUnroll];
    int64_t dst[kPagedUnroll];
#pragma unroll
    for (int x = 0; x < kPagedUnroll; ++x) {
      const int u = u0 + x * kThreads + tid;
      dst[x] = -1;
      if (u < total) {
        const int i = u / upr, p = u - i * upr;
        const int r = i0 + i;
        const int64_t page = table[r / P.page_rows];
        if (page >= 0 && page < P.n_pages) {
          const int64_t src = static_cast<int64_t>(min(max(idx[i], 0), t_last)) * P.kv_st_bytes + p * 16;
          kv[x] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(ks + src));
          vv[x] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vs + src));
          dst[x] = (page * P.page_rows + r % P.page_rows) * P.row_bytes + p * 16;
        }
      }
    }
#pragma unroll
    for (int x = 0; x < kPagedUnroll; ++x) {
      if (dst[x] >= 0) {
        __builtin_nontemporal_store(kv[x], reinterpret_cast<u32x4*>(kd + dst[x]));
        __builtin_nontemporal_store(vv[x], reinterpret_cast<u32x4*>(vd + dst[x]));
      }
    }
  }
}

}  // namespace

hipError_t launch_gather_paged(const PagedParams& p, int n_blocks, hipStream_t s) {
  return launch1(gather_paged_kernel, dim3(n_blocks), dim3(kThreads), 0, s, p);
}

}  // namespace ckv
