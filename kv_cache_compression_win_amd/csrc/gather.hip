// K/V compaction: index_select of the kept rows (ChunkKV page, section 4.1,
// Algorithm 1 step 6; under layer-wise index reuse, section 4.2 Algorithm 2,
// a layer reads the index block of its anchor layer).
//
// Work item = (layer, sequence, KV head, block of kGatherRows output rows).
// Rows are copied as 16-byte vectors: consecutive threads take consecutive
// 16-byte pieces of a row, so both the row reads and the compacted writes are
// contiguous runs; every thread issues its K and V loads for up to four
// pieces before storing.  Stores are non-temporal (the compacted cache is
// not re-read by this path).
#include "chunkkv_internal.h"

namespace ckv {
namespace {

#ifndef CKV_GATHER_UNROLL
#define CKV_GATHER_UNROLL 2
#endif
#ifndef CKV_GATHER_NT
#define CKV_GATHER_NT 1
#endif
constexpr int kUnroll = CKV_GATHER_UNROLL;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kThreads) void gather_kernel(const GatherParams P) {
  const int tid = threadIdx.x;
  const int li = blockIdx.x / P.items_per_layer;
  int item = blockIdx.x - li * P.items_per_layer;
  int b = 0;
  while (b + 1 < P.n_seqs && item >= P.item0[b + 1]) ++b;
  item -= P.item0[b];
  const int bph = P.blocks_per_head[b];
  const int h = item / bph, blk = item - h * bph;
  const int blkL = P.idx_block[li];
  // lengths and index values come from the selection (always in range); a
  // caller's own are clamped, so no input reads or writes outside the
  // sequence's rows and the head's L_cap output rows
  const int n = min(max(P.lengths[blkL * P.len_layer_stride + P.len_off[b] + h], 0), P.L_cap[b]);
  const int t_last = P.T[b] - 1;
  const int i0 = blk * kGatherRows;
  if (i0 >= n) return;
  const int nrows = min(kGatherRows, n - i0);
  const int upr = P.row_bytes >> 4;
  const int total = nrows * upr;

  const int64_t out_row0 = P.index_off[b] + static_cast<int64_t>(h) * P.L_cap[b] + i0;
  const int32_t* idx = P.indices + blkL * P.index_layer_stride + out_row0;
  const int64_t src_off = P.tok0[b] * P.kv_st_bytes + static_cast<int64_t>(h) * P.kv_sh_bytes;
  const char* ks = static_cast<const char*>(P.k[li]) + src_off;
  const char* vs = static_cast<const char*>(P.v[li]) + src_off;
  char* kd = static_cast<char*>(P.ko[li]) + out_row0 * P.row_bytes;
  char* vd = static_cast<char*>(P.vo[li]) + out_row0 * P.row_bytes;

  for (int u0 = 0; u0 < total; u0 += kThreads * kUnroll) {
    u32x4 kv[kUnroll], vv[kUnroll];
    int64_t dst[kUnroll];
#pragma unroll
    for (int x = 0; x < kUnroll; ++x) {
      const int u = u0 + x * kThreads + tid;
      dst[x] = -1;
      if (u < total) {
        const int i = u / upr, p = u - i * upr;
        const int64_t src = static_cast<int64_t>(min(max(idx[i], 0), t_last)) * P.kv_st_bytes + p * 16;
#if CKV_GATHER_NT
        kv[x] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(ks + src));
        vv[x] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vs + src));
#else
        kv[x] = *reinterpret_cast<const u32x4*>(ks + src);
        vv[x] = *reinterpret_cast<const u32x4*>(vs + src);
#endif
        dst[x] = static_cast<int64_t>(i) * P.row_bytes + p * 16;
      }
    }
#pragma unroll
    for (int x = 0; x < kUnroll; ++x) {
      if (dst[x] >= 0) {
        __builtin_nontemporal_store(kv[x], reinterpret_cast<u32x4*>(kd + dst[x]));
        __builtin_nontemporal_store(vv[x], reinterpret_cast<u32x4*>(vd + dst[x]));
      }
    }
  }
}

}  // namespace

hipError_t launch_gather(const GatherParams& p, int n_blocks, hipStream_t s, hipEvent_t ev_start,
                         hipEvent_t ev_stop) {
  return launch1(gather_kernel, dim3(n_blocks), dim3(kThreads), 0, s, p, ev_start, ev_stop);
}

}  // namespace ckv
