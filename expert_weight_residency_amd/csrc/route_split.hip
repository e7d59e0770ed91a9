// Residency split of the routed top-k ids with the usage counter fused in.
//
// "vLLM: Pin Hot Experts", section "The one open door": a per-layer int32 row
// map resolves a global expert id to (which tensor, which row); section
// "Results, September 17": each token's ids are split by residency before the
// two bank calls. "We Built the Counter", section 2: the counter is one masked
// relaxed atomic add per routed pick into a fixed table, inside the split
// kernel (no extra launch), and only steps of at most 256 tokens count.
//
// Kernel A (one workgroup of 1024 threads) builds per-bank row histograms and
// a per-expert histogram in LDS, adds the expert histogram to the counter
// table with one relaxed device-scope atomic per touched expert, scans the
// row histograms into CSR offsets and the ascending active-row list, and, for
// at most kSplitSingleMaxPicks picks, places every slot at its row offset plus
// its rank among earlier picks of the same row. Above that size kernel B
// places the slots instead: one wavefront per active row walks the picks in
// order and appends matches with a ballot. Both give the same unique layout.
#include "internal.h"

namespace moe {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;

// Pick s -> packed key: hot row r -> r, cold row r -> n_hot + r, invalid -> -1.
__device__ __forceinline__ int pick_key(const int32_t* __restrict__ ids,
                                        const int32_t* __restrict__ row_map, int E, int n_hot,
                                        int n_cold, int s) {
  const int id = ids[s];
  if (id < 0 || id >= E) return -1;
  const int m = row_map[id];
  if (m >= 0) return m < n_hot ? m : -1;
  const int r = -1 - m;
  return r < n_cold ? n_hot + r : -1;
}

// Block-wide exclusive scan of two ints per thread; also returns the totals.
// `tot` is LDS scratch of kWaves int2. Must be called by all threads.
__device__ __forceinline__ int2 block_scan2(int a, int b, int2* tot, int2& total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  int ia = a, ib = b;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int ta = __shfl_up(ia, d, 64);
    const int tb = __shfl_up(ib, d, 64);
    if (lane >= d) {
      ia += ta;
      ib += tb;
    }
  }
  if (lane == 63) tot[wid] = make_int2(ia, ib);
  __syncthreads();
  int2 pre = make_int2(0, 0), all = make_int2(0, 0);
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const int2 v = tot[w];
    if (w < wid) {
      pre.x += v.x;
      pre.y += v.y;
    }
    all.x += v.x;
    all.y += v.y;
  }
  __syncthreads();
  total = all;
  return make_int2(pre.x + ia - a, pre.y + ib - b);
}

// Scan hist[0..n) (row counts) into CSR offsets + active rows; leaves the
// exclusive start offset of each row in hist[] for slot placement.
__device__ void compact_bank(int* hist, int n, moe_split out, int2* tot) {
  const int per = (n + kThreads - 1) / kThreads;  // <= 4 for n <= 4096
  const int beg = threadIdx.x * per;
  int cnt = 0, act = 0;
  for (int i = 0; i < per; ++i) {
    const int r = beg + i;
    if (r < n) {
      const int c = hist[r];
      cnt += c;
      act += c > 0;
    }
  }
  int2 total;
  const int2 ex = block_scan2(cnt, act, tot, total);
  int off = ex.x, idx = ex.y;
  for (int i = 0; i < per; ++i) {
    const int r = beg + i;
    if (r < n) {
      const int c = hist[r];
      if (c > 0) {
        out.active_rows[idx] = r;
        out.row_off[idx] = off;
        ++idx;
      }
      hist[r] = off;
      off += c;
    }
  }
  if (threadIdx.x == 0) {
    *out.n_active = total.y;
    out.row_off[total.y] = total.x;
  }
}

__global__ __launch_bounds__(kThreads) void route_split_main(
    const int32_t* __restrict__ ids, int n_picks, const int32_t* __restrict__ row_map, int E,
    int n_hot, int n_cold, int32_t* __restrict__ counts, int count_on, moe_split hot,
    moe_split cold, int32_t* __restrict__ n_invalid, int place_slots) {
  __shared__ int hist[2 * MOE_MAX_ROWS];
  __shared__ int idcnt[MOE_MAX_EXPERTS];
  __shared__ int keys[kSplitSingleMaxPicks];
  __shared__ int2 tot[kWaves];
  __shared__ int bad;

  const int nrows = n_hot + n_cold;
  for (int i = threadIdx.x; i < nrows; i += kThreads) hist[i] = 0;
  if (count_on)
    for (int i = threadIdx.x; i < E; i += kThreads) idcnt[i] = 0;
  if (threadIdx.x == 0) bad = 0;
  __syncthreads();

  int my_bad = 0;
  for (int s = threadIdx.x; s < n_picks; s += kThreads) {
    const int key = pick_key(ids, row_map, E, n_hot, n_cold, s);
    if (place_slots) keys[s] = key;
    if (key >= 0)
      atomicAdd(&hist[key], 1);
    else
      ++my_bad;
    if (count_on) {
      const int id = ids[s];
      if (id >= 0 && id < E) atomicAdd(&idcnt[id], 1);
    }
  }
  if (my_bad) atomicAdd(&bad, my_bad);
  __syncthreads();

  if (count_on) {
    for (int i = threadIdx.x; i < E; i += kThreads) {
      const int c = idcnt[i];
      if (c) __hip_atomic_fetch_add(&counts[i], c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  if (threadIdx.x == 0) *n_invalid = bad;

  compact_bank(hist, n_hot, hot, tot);
  compact_bank(hist + n_hot, n_cold, cold, tot);
  __syncthreads();

  if (!place_slots) return;
  // Rank of each pick among earlier picks with the same key (ascending s).
  for (int s = threadIdx.x; s < n_picks; s += kThreads) {
    const int key = keys[s];
    if (key < 0) continue;
    int rank = 0;
    for (int p = 0; p < s; ++p) rank += keys[p] == key;
    if (key < n_hot)
      hot.slots[hist[key] + rank] = s;
    else
      cold.slots[hist[key] + rank] = s;
  }
}

// One wavefront per potential active row: rows [0, cap_hot) of the hot split,
// then [0, cap_cold) of the cold split.
__global__ __launch_bounds__(256) void route_split_place(
    const int32_t* __restrict__ ids, int n_picks, const int32_t* __restrict__ row_map, int E,
    int n_hot, int n_cold, int cap_hot, int cap_cold, moe_split hot, moe_split cold) {
  const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (w >= cap_hot + cap_cold) return;
  const bool is_hot = w < cap_hot;
  const moe_split& sp = is_hot ? hot : cold;
  const int idx = is_hot ? w : w - cap_hot;
  if (idx >= *sp.n_active) return;
  const int want = is_hot ? sp.active_rows[idx] : n_hot + sp.active_rows[idx];
  int base = sp.row_off[idx];
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int s0 = 0; s0 < n_picks; s0 += 64) {
    const int s = s0 + lane;
    const bool hit = s < n_picks && pick_key(ids, row_map, E, n_hot, n_cold, s) == want;
    const uint64_t mask = __ballot(hit);
    if (hit) sp.slots[base + __popcll(mask & below)] = s;
    base += __popcll(mask);
  }
}

}  // namespace

hipError_t launch_route_split(const int32_t* ids, int T, int k, const int32_t* row_map, int E,
                              int n_hot, int n_cold, int32_t* counts, int count_on,
                              const moe_split& hot, const moe_split& cold, int32_t* n_invalid,
                              hipStream_t stream) {
  const int n_picks = T * k;
  const int single = n_picks <= kSplitSingleMaxPicks;
  hipLaunchKernelGGL(route_split_main, dim3(1), dim3(kThreads), 0, stream, ids, n_picks, row_map,
                     E, n_hot, n_cold, counts, count_on, hot, cold, n_invalid, single);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || single) return e;
  const int cap_hot = n_hot < n_picks ? n_hot : n_picks;
  const int cap_cold = n_cold < n_picks ? n_cold : n_picks;
  const int waves = cap_hot + cap_cold;
  if (waves == 0) return hipSuccess;
  hipLaunchKernelGGL(route_split_place, dim3((waves + 3) / 4), dim3(256), 0, stream, ids, n_picks,
                     row_map, E, n_hot, n_cold, cap_hot, cap_cold, hot, cold);
  return hipGetLastError();
}

}  // namespace moe
