// Residency split of the routed top-k ids with the usage counter fused in.
//
// "vLLM: Pin Hot Experts", section "The one open door": a per-layer int32 row
// map resolves a global expert id to (which tensor, which row); section
// "Results, September 17": each token's ids are split by residency before the
// two bank calls. "We Built the Counter", section 2: the counter is one masked
// relaxed atomic add per routed pick into a fixed table, inside the split
// kernel (no extra launch), and only steps of at most 256 tokens count.
//
// Kernel A (one workgroup of 1024 threads) stages a per-expert table of row
// keys in LDS (from the row map), builds per-bank row histograms and a
// per-expert histogram in LDS, adds the expert histogram to the counter table
// with one relaxed device-scope atomic per touched expert, scans the row
// histograms into CSR offsets and the ascending active-row list, and, for at
// most kSplitSingleMaxPicks picks, places every slot at its row offset plus
// its rank among earlier picks of the same row. Above that size kernel B, a
// stable counting scatter spread over many compute units, places the slots
// instead: each of its workgroups owns 16 active rows, counts their picks per
// thread over contiguous pick ranges, scans the counts over the threads and
// writes each pick at its row offset plus its rank. Both give the same unique
// layout.
#include "internal.h"

namespace moe {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;

// Packed key of a pick: hot row r -> r, cold row r -> n_hot + r, invalid -> -1
// (< 2 * MOE_MAX_ROWS: fits int16). ktab[id] holds the packed key of expert id,
// staged in LDS once per workgroup, so a pick's key is one LDS read.
template <int NT>
__device__ __forceinline__ void stage_keys(const int32_t* __restrict__ row_map, int E, int n_hot,
                                           int n_cold, int16_t* ktab) {
  for (int i = threadIdx.x; i < E; i += NT) {
    const int m = row_map[i], cr = -1 - m;
    ktab[i] = (int16_t)(m >= 0 ? (m < n_hot ? m : -1) : (cr < n_cold ? n_hot + cr : -1));
  }
}

// The routed ids as a buffer resource of n entries: a load at or past entry n
// returns 0 and never faults, so no index needs clamping.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t ids_rsrc(const int32_t* ids, int n) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<int32_t*>(ids), (short)0, n * 4,
                                           0x00020000);
}

// Ids of picks s = base + u * NT + threadIdx.x for u < nb (nb uniform; u >= nb:
// -1), every load issued before any is used: one memory round trip per batch
// (a workgroup walking tens of thousands of picks one dependent load at a time
// spends tens of microseconds waiting).
template <int NT, int B>
__device__ __forceinline__ void load_ids(__amdgpu_buffer_rsrc_t ids, int base, int nb,
                                         int (&id)[B]) {
#pragma unroll
  for (int u = 0; u < B; ++u)
    id[u] = u < nb ? __builtin_amdgcn_raw_buffer_load_b32(
                         ids, (base + u * NT + (int)threadIdx.x) * 4, 0, 0)
                   : -1;
}

// Keys of the picks load_ids fetched (past n or u >= nb: -2); id becomes the
// id if it lies in [0, E), else -1.
template <int NT, int B>
__device__ __forceinline__ void resolve_keys(const int16_t* ktab, int E, int n, int base, int nb,
                                             int (&id)[B], int (&key)[B]) {
  // every key-table read is issued before the first use: the empty asm takes
  // the values as operands, so the compiler cannot sink a read into a branch
  // of the selects below and wait on each one in turn
  int kv[B];
#pragma unroll
  for (int u = 0; u < B; ++u) kv[u] = u < nb ? ktab[(uint32_t)id[u] < (uint32_t)E ? id[u] : 0] : 0;
#pragma unroll
  for (int u = 0; u < B; ++u) asm volatile("" : "+v"(kv[u]));
#pragma unroll
  for (int u = 0; u < B; ++u) {
    const int s = base + u * NT + (int)threadIdx.x;
    const bool valid = (uint32_t)id[u] < (uint32_t)E;
    const bool in = u < nb && s < n;
    key[u] = in ? (valid ? kv[u] : -1) : -2;
    id[u] = in && valid ? id[u] : -1;
  }
}

// Block-wide exclusive scan of four ints per thread; also returns the totals.
// `tot` is LDS scratch of kWaves int4. Must be called by all threads.
__device__ __forceinline__ int4 block_scan4(int4 v, int4* tot, int4& total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  int4 in = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int tx = __shfl_up(in.x, d, 64), ty = __shfl_up(in.y, d, 64);
    const int tz = __shfl_up(in.z, d, 64), tw = __shfl_up(in.w, d, 64);
    if (lane >= d) {
      in.x += tx;
      in.y += ty;
      in.z += tz;
      in.w += tw;
    }
  }
  if (lane == 63) tot[wid] = in;
  __syncthreads();
  int4 pre = make_int4(0, 0, 0, 0), all = make_int4(0, 0, 0, 0);
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const int4 t = tot[w];
    if (w < wid) {
      pre.x += t.x;
      pre.y += t.y;
      pre.z += t.z;
      pre.w += t.w;
    }
    all.x += t.x;
    all.y += t.y;
    all.z += t.z;
    all.w += t.w;
  }
  __syncthreads();
  total = all;
  return make_int4(pre.x + in.x - v.x, pre.y + in.y - v.y, pre.z + in.z - v.z, pre.w + in.w - v.w);
}

// Row counts (hist[0..n)) into CSR offsets and the ascending active-row list,
// given this thread's exclusive start offset and active index; leaves the
// exclusive start offset of each row in hist[] for slot placement.
__device__ __forceinline__ void write_bank(int* hist, int n, int beg, int per, int off, int idx,
                                           int n_active, int total, moe_split out) {
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
    *out.n_active = n_active;
    out.row_off[n_active] = total;
  }
}

// Both banks' compaction with one block-wide scan (hist: hot rows, then cold).
__device__ void compact_banks(int* hist, int n_hot, int n_cold, moe_split hot, moe_split cold,
                              int4* tot) {
  const int ph = (n_hot + kThreads - 1) / kThreads;  // <= 4 for n <= 4096
  const int pc = (n_cold + kThreads - 1) / kThreads;
  const int bh = threadIdx.x * ph, bc = threadIdx.x * pc;
  int4 v = make_int4(0, 0, 0, 0);  // hot count, hot active, cold count, cold active
  for (int i = 0; i < ph; ++i) {
    const int r = bh + i;
    if (r < n_hot) {
      const int c = hist[r];
      v.x += c;
      v.y += c > 0;
    }
  }
  for (int i = 0; i < pc; ++i) {
    const int r = bc + i;
    if (r < n_cold) {
      const int c = hist[n_hot + r];
      v.z += c;
      v.w += c > 0;
    }
  }
  int4 total;
  const int4 ex = block_scan4(v, tot, total);
  write_bank(hist, n_hot, bh, ph, ex.x, ex.y, total.y, total.x, hot);
  write_bank(hist + n_hot, n_cold, bc, pc, ex.z, ex.w, total.w, total.z, cold);
}

constexpr int kMainB = 8;  // picks per thread per batch: 8192 per batch

__global__ __launch_bounds__(kThreads) void route_split_main(
    const int32_t* __restrict__ ids, int n_picks, const int32_t* __restrict__ row_map, int E,
    int n_hot, int n_cold, int32_t* __restrict__ counts, int count_on, moe_split hot,
    moe_split cold, int32_t* __restrict__ n_invalid, int place_slots) {
  __shared__ int hist[2 * MOE_MAX_ROWS];
  __shared__ int idcnt[MOE_MAX_EXPERTS];
  __shared__ int keys[kSplitSingleMaxPicks];
  __shared__ int16_t ktab[MOE_MAX_EXPERTS];
  __shared__ int4 tot[kWaves];
  __shared__ int bad;

  const __amdgpu_buffer_rsrc_t rs = ids_rsrc(ids, n_picks);
  stage_keys<kThreads>(row_map, E, n_hot, n_cold, ktab);
  const int nrows = n_hot + n_cold;
  for (int i = threadIdx.x; i < nrows; i += kThreads) hist[i] = 0;
  if (count_on)
    for (int i = threadIdx.x; i < E; i += kThreads) idcnt[i] = 0;
  if (threadIdx.x == 0) bad = 0;
  __syncthreads();

  int my_bad = 0;
  for (int base = 0; base < n_picks; base += kMainB * kThreads) {
    const int nb = min(kMainB, (n_picks - base + kThreads - 1) / kThreads);
    int id[kMainB], key[kMainB];
    load_ids<kThreads, kMainB>(rs, base, nb, id);
    resolve_keys<kThreads, kMainB>(ktab, E, n_picks, base, nb, id, key);
#pragma unroll
    for (int u = 0; u < kMainB; ++u) {
      if (key[u] == -2) continue;  // past the last pick
      const int s = base + u * kThreads + (int)threadIdx.x;
      if (place_slots) keys[s] = key[u];
      if (key[u] >= 0)
        atomicAdd(&hist[key[u]], 1);
      else
        ++my_bad;
      if (count_on && id[u] >= 0) atomicAdd(&idcnt[id[u]], 1);
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

  compact_banks(hist, n_hot, n_cold, hot, cold, tot);
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

// Kernel B. Workgroup g owns the active rows of concatenated index a in
// [16 g, 16 g + 16) (hot active rows first, then cold ones; their packed keys
// ascend with a), so a pick belongs to one of its rows iff the pick's key lies
// between the keys of its first and last row. Per tile of kQTile picks, thread
// t owns the contiguous picks [kQPer t, kQPer t + kQPer) of the tile: their
// keys are computed with coalesced loads, pass through LDS once to reach their
// owner, and stay in its registers. Pass 1 counts the thread's picks of each
// owned row; wavefront r then scans row r's counts over the threads in order,
// which leaves with each thread the rank of its first pick of the row among
// the row's picks in the tile; pass 2 writes each of the thread's picks at its
// row's running base plus that rank, bumping the rank. A row's running base
// starts at its CSR offset and grows by the row's tile total after each tile.
// Only a thread's own picks of owned rows (a small share of all picks) touch
// LDS in the two passes, so the work per workgroup is a few LDS operations
// per pick.
constexpr int kQThreads = 1024;
constexpr int kQRows = kQThreads / 64;     // owned rows: one per wavefront in the scan
constexpr int kQPer = 32;                  // picks per thread per tile (bits of a mask)
constexpr int kQTile = kQThreads * kQPer;  // 32768 picks: ranks and counts fit uint16
// int16 per thread row of the key tile: 80 bytes keeps each row 16-byte
// aligned and puts the 16-byte reads of 8 consecutive threads on distinct banks
constexpr int kQRowStride = kQPer + 8;

__global__ __launch_bounds__(kQThreads) void route_split_place(
    const int32_t* __restrict__ ids, int n_picks, const int32_t* __restrict__ row_map, int E,
    int n_hot, int n_cold, moe_split hot, moe_split cold) {
  __shared__ __align__(16) int16_t lkey[kQThreads * kQRowStride];  // [owner][pick]
  __shared__ __align__(16) uint16_t cnt[kQRows * kQThreads];       // [row][thread]
  __shared__ int16_t ktab[MOE_MAX_EXPERTS];
  __shared__ uint8_t kidx[2 * MOE_MAX_ROWS];  // key - key of the first row -> owned row
  __shared__ int rbase[kQRows], rtot[kQRows];
  __shared__ int32_t* rslots[kQRows];
  __shared__ int32_t* rdst[kQRows];  // rslots[r] + rbase[r] for the current tile

  const __amdgpu_buffer_rsrc_t rs = ids_rsrc(ids, n_picks);
  auto batches = [&](int t0) {
    return (min(kQTile, n_picks - t0) + kQThreads - 1) / kQThreads;
  };
  int id[kQPer];
  const int n_act_hot = *hot.n_active;
  const int n_act = n_act_hot + *cold.n_active;
  const int a0 = (int)blockIdx.x * kQRows;
  if (a0 >= n_act) return;  // whole workgroup, before any barrier
  const int nr = min(kQRows, n_act - a0);
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  auto key_of = [&](int a) {
    return a < n_act_hot ? hot.active_rows[a] : n_hot + cold.active_rows[a - n_act_hot];
  };
  const int klo = key_of(a0), khi = key_of(a0 + nr - 1);
  if (tid < nr) {
    const int a = a0 + tid;
    kidx[key_of(a) - klo] = (uint8_t)tid;
    rbase[tid] = a < n_act_hot ? hot.row_off[a] : cold.row_off[a - n_act_hot];
    rslots[tid] = a < n_act_hot ? hot.slots : cold.slots;
  }
  stage_keys<kQThreads>(row_map, E, n_hot, n_cold, ktab);
  int16_t* const mine = lkey + tid * kQRowStride;
  uint32_t* const cnt32 = reinterpret_cast<uint32_t*>(cnt);
  // the counts of threads 2i and 2i+1 share a 32-bit word (each below 2^16)
  const int cw = tid >> 1, csh = 16 * (tid & 1);

  for (int t0 = 0; t0 < n_picks; t0 += kQTile) {
    const int tn = min(kQTile, n_picks - t0);
    __syncthreads();  // rows and row map staged; the previous tile is done
    {
      // tile pick s = u * kQThreads + tid goes to owner s / kQPer at s % kQPer;
      // batches u >= nb hold no pick below tn and are neither loaded nor
      // written (their owners read nothing)
      const int nb = batches(t0);
      load_ids<kQThreads, kQPer>(rs, t0, nb, id);
      int key[kQPer];
      resolve_keys<kQThreads, kQPer>(ktab, E, n_picks, t0, nb, id, key);
      static_assert(kQThreads % kQPer == 0, "s % kQPer == tid % kQPer");
      int16_t* const dst = lkey + (tid / kQPer) * kQRowStride + tid % kQPer;
#pragma unroll
      for (int u = 0; u < kQPer; ++u)
        if (u < nb) dst[u * (kQThreads / kQPer) * kQRowStride] = (int16_t)key[u];
    }
    if (w < nr) {  // zero row w's counts
      uint4* p = reinterpret_cast<uint4*>(cnt + w * kQThreads + lane * 16);
      p[0] = make_uint4(0, 0, 0, 0);
      p[1] = make_uint4(0, 0, 0, 0);
    }
    __syncthreads();

    // this thread's picks of owned rows, one bit per pick
    uint32_t hits = 0;
    if (tid * kQPer < tn) {
      const uint4* src = reinterpret_cast<const uint4*>(mine);
      uint32_t k2[kQPer / 2];
#pragma unroll
      for (int i = 0; i < kQPer / 8; ++i) {
        const uint4 v = src[i];
        k2[4 * i] = v.x;
        k2[4 * i + 1] = v.y;
        k2[4 * i + 2] = v.z;
        k2[4 * i + 3] = v.w;
      }
#pragma unroll
      for (int j = 0; j < kQPer; ++j) {
        const int key = (int)(int16_t)(k2[j / 2] >> (16 * (j & 1)));
        hits |= (uint32_t)(key >= klo && key <= khi) << j;
      }
    }

    // pass 1: count (no-return atomic add of 1 to this thread's half word)
    for (uint32_t m = hits; m; m &= m - 1) {
      const int j = __builtin_ctz(m);
      const int r = kidx[mine[j] - klo];
      atomicAdd(&cnt32[r * (kQThreads / 2) + cw], 1u << csh);
    }
    __syncthreads();

    if (w < nr) {
      // row w: lane l holds threads [16 l, 16 l + 16)
      uint4* p = reinterpret_cast<uint4*>(cnt + w * kQThreads + lane * 16);
      const uint4 v0 = p[0], v1 = p[1];
      const uint32_t q[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
      uint32_t ex[8];
      int sum = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int lo = (int)(q[i] & 0xffffu), hi = (int)(q[i] >> 16);
        ex[i] = (uint32_t)sum | ((uint32_t)(sum + lo) << 16);
        sum += lo + hi;
      }
      int incl = sum;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int t = __shfl_up(incl, d, 64);
        if (lane >= d) incl += t;
      }
      const uint32_t pre = (uint32_t)(incl - sum) * 0x10001u;  // add to both halves
      p[0] = make_uint4(ex[0] + pre, ex[1] + pre, ex[2] + pre, ex[3] + pre);
      p[1] = make_uint4(ex[4] + pre, ex[5] + pre, ex[6] + pre, ex[7] + pre);
      if (lane == 63) {
        rtot[w] = incl;
        rdst[w] = rslots[w] + rbase[w];
      }
    }
    __syncthreads();

    // pass 2: place, in pick order within the thread
    for (uint32_t m = hits; m; m &= m - 1) {
      const int j = __builtin_ctz(m);
      const int r = kidx[mine[j] - klo];
      uint16_t* const c = cnt + r * kQThreads + tid;
      const int rank = *c;
      *c = (uint16_t)(rank + 1);
      rdst[r][rank] = t0 + tid * kQPer + j;
    }
    __syncthreads();
    if (tid < nr) rbase[tid] += rtot[tid];
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
  // at most one active row per pick in each bank
  const int cap_hot = n_hot < n_picks ? n_hot : n_picks;
  const int cap_cold = n_cold < n_picks ? n_cold : n_picks;
  const int rows = cap_hot + cap_cold;
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(route_split_place, dim3((rows + kQRows - 1) / kQRows), dim3(kQThreads), 0,
                     stream, ids, n_picks, row_map, E, n_hot, n_cold, hot, cold);
  return hipGetLastError();
}

}  // namespace moe
