// Work items of the token-tiled expert FFN kernels (ffn_tiled.hip, ffn_fp4.hip):
// each active row's slots are cut into tiles of kTok, and a workgroup finds
// the row of a tile from an exclusive prefix of the rows' tile counts kept in
// LDS.
#pragma once

#include "internal.h"

namespace moe {
namespace tiles {

// Exclusive prefix over the active rows of their tile counts (kTok slots per
// tile), into tpre[0..na]; wsum: kWaves ints of scratch LDS. Every thread of
// the kWaves-wavefront workgroup calls it; it ends with a barrier.
template <int kTok, int kWaves>
__device__ void build_tile_prefix(const int32_t* __restrict__ row_off, int na, int* tpre,
                                  int* wsum) {
  constexpr int kThreads = 64 * kWaves;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int carry = 0;
  for (int base = 0; base < na; base += kThreads) {
    const int a = base + tid;
    const int v = a < na ? (row_off[a + 1] - row_off[a] + kTok - 1) / kTok : 0;
    int s = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(s, d, 64);
      if (lane >= d) s += o;
    }
    if (lane == 63) wsum[wv] = s;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
      before += i < wv ? wsum[i] : 0;
      total += wsum[i];
    }
    if (a < na) tpre[a] = carry + before + s - v;
    carry += total;
    __syncthreads();
  }
  if (tid == 0) tpre[na] = carry;
  __syncthreads();
}

// Active row holding tile `tile` (every active row has at least one tile).
__device__ __forceinline__ int row_of_tile(const int* tpre, int na, int tile) {
  int lo = 0, hi = na - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (tpre[mid] <= tile) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

}  // namespace tiles
}  // namespace moe
