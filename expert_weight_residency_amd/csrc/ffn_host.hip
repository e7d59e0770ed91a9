// Expert FFN kernels for a bank in pinned host memory, read in place over the
// host link at decode-sized steps (gfx950). Same operations as the other bf16
// kernel families: gate/up + SwiGLU, and the down GEMM into unweighted bf16
// rows ("We Built the Counter", section 1: cold experts are read in place from
// host memory whenever the router picks one; "vLLM: Pin Hot Experts",
// section "Results, September 17": the routed expert FFN per bank).
//
// The host link wants long contiguous reads: one stream of 16-byte pieces, or
// pieces of 512 bytes per row, reach its ceiling (~56 GB/s), while the MFMA
// operand layout (16 rows x 128 bytes per load) reaches ~40 GB/s. Reads of
// host memory in that linear pattern also leave the device-bank kernels
// running beside them almost untouched (measured: +2-3 us on the hot gate/up
// and down at a full link; a copy of the same rows into HBM costs them ~17 us
// through its HBM writes). So these kernels copy each work item's weight bytes
// from host memory in the linear pattern (each load instruction reads 1 KB
// contiguous: lane L its 16-byte granule L), holds it in registers while the
// wavefront multiplies the previous item out of LDS, then writes it to the
// wavefront's LDS item buffer and feeds the MFMA A operand from there. (A
// global-to-LDS copy would save the registers, but the compiler cannot tell
// its LDS writes from the LDS reads of the arithmetic and waits for every copy
// in flight before each read, which serializes the stream.) Each output element sees the same MFMA sequence (same
// 256-element chunks, same lane-to-element map, same order from zero) and the
// same epilogue as in the other families, so a pick gives the same bits from
// either bank.
#include <type_traits>

#include "internal.h"
#include "mxfp4_common.h"

namespace moe {
namespace {

using namespace mx;

// Native vector type for the staged pieces (an array of HIP's uint4 struct,
// copied through memcpy, is not promoted to registers and lands in scratch).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---- down -------------------------------------------------------------------
//
// Work item = 16 output rows of one active expert: 16 x I/2 contiguous weight
// bytes and 16 x I/32 contiguous scale bytes, loaded whole (kDLoads loads of
// 1 KB; pieces past the item's bytes read its first granule, one request for
// the whole wavefront, so every load is unconditional) while the wavefront
// computes its previous item. Items are ordered (expert, row block);
// workgroup b takes one equal contiguous run and its wavefronts take every
// kDW-th item of it; the run's h rows are staged into LDS once (in phases
// when they exceed it), and a wavefront runs all 16-slot passes of an item
// from the same buffer.

constexpr int kDW = 4;                    // wavefronts per workgroup (one per SIMD)
constexpr int kDThreads = 64 * kDW;
constexpr int kDMaxI = 3072;              // largest I an item buffer holds
constexpr int kDWLoads = kDMaxI / 128;    // weight loads per item (16 rows x I/2 bytes)
constexpr int kDSLoads = 2;               // scale loads per item (16 rows x I/32 <= 1.5 KB)
constexpr int kDLoads = kDWLoads + kDSLoads;
constexpr int kDBuf = kDLoads * 1024;     // bytes of one item buffer
// h rows of the run's slots, staged once per phase: a static array (reads of
// dynamically sized LDS would count, for the compiler, as possibly aliasing the
// item buffers' pending copies, and it would wait for every copy in flight)
constexpr int kDMaxKpad = kDMaxI;         // I padded to whole 256-element chunks
constexpr int kDHElems = 9 * kDMaxKpad;   // 9 rows at I = 3072 (more at smaller I)
constexpr int kDHRowsMax = kDHElems / kChunkElems;

__global__ __launch_bounds__(kDThreads, 1) void ffn_down_host(
    const uint8_t* __restrict__ w2, const uint8_t* __restrict__ s2,
    const int32_t* __restrict__ n_active, const int32_t* __restrict__ active_rows,
    const int32_t* __restrict__ row_off, const int32_t* __restrict__ slots,
    const __bf16* __restrict__ h, int H, int I, int max_rows, uint16_t* __restrict__ Y) {
  __shared__ __align__(16) unsigned char dbuf[kDW][kDBuf];
  __shared__ __align__(16) __bf16 hs[kDHElems];
  __shared__ int l_slot[kDHRowsMax];
  const int nchunk = (I + kChunkElems - 1) / kChunkElems, kpad = nchunk * kChunkElems;
  const int nblk = I / 32, sbr = I / 32;
  const uint32_t wib = 8u * (uint32_t)I, sib = (uint32_t)I / 2u;  // item weight / scale bytes

  const int tid = threadIdx.x, lane = tid & 63, r = lane & 15, q = lane >> 4;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int na = __builtin_amdgcn_readfirstlane(*n_active);
  const int per = H / 16;
  const int n = na * per;
  if (n == 0) return;
  const int qb = (n + gridDim.x - 1) / gridDim.x;
  const int g0 = blockIdx.x * qb;
  if (g0 >= n) return;  // the whole workgroup, before any barrier
  const int g1 = min(n, g0 + qb);
  const int s_lo = __builtin_amdgcn_readfirstlane(row_off[g0 / per]);
  const int s_hi = __builtin_amdgcn_readfirstlane(row_off[(g1 - 1) / per + 1]);
  const bool lane_in_last = (nchunk - 1) * kChunkBlocks + 2 * q < nblk;

  for (int ph0 = s_lo; ph0 < s_hi; ph0 += max_rows) {
    const int ph1 = min(s_hi, ph0 + max_rows);
    if (ph0 != s_lo) __syncthreads();  // the previous phase is done with the rows
    {
      const int gpr = kpad / 8, nr = ph1 - ph0;
      for (int gi = tid; gi < nr * gpr; gi += kDThreads) {
        const int m = gi / gpr, g = gi - m * gpr;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (g * 8 < I)
          v = *reinterpret_cast<const uint4*>(h + (size_t)slots[ph0 + m] * I + g * 8);
        *reinterpret_cast<uint4*>(hs + lds_elem(m, kpad, g * 8)) = v;
      }
      for (int i = tid; i < nr; i += kDThreads) l_slot[i] = slots[ph0 + i];
    }
    __syncthreads();

    auto lo_of = [&](int a) { return max(__builtin_amdgcn_readfirstlane(row_off[a]), ph0); };
    auto ncols = [&](int a) {
      return min(__builtin_amdgcn_readfirstlane(row_off[a + 1]), ph1) - lo_of(a);
    };
    // this wavefront's next item with slots in the phase after `it` (g1: none)
    auto next_item = [&](int it) {
      for (it += kDW; it < g1; it += kDW)
        if (ncols(it / per) > 0) return it;
      return g1;
    };
    unsigned char* buf = dbuf[wv];
    // the next item, on its way from host memory (plain unrolled loops in
    // the kernel body: the array stays in registers)
    u32x4 stg[kDLoads];
#define DOWN_HOST_ISSUE(IT)                                                              \
  do {                                                                                   \
    const int a_ = (IT) / per, o0_ = ((IT) - a_ * per) * 16;                              \
    const uint64_t row_ = (uint32_t)__builtin_amdgcn_readfirstlane(active_rows[a_]);      \
    const uint8_t* wsrc_ = w2 + (row_ * H + o0_) * (uint64_t)(I / 2);                     \
    const uint8_t* ssrc_ = s2 + (row_ * H + o0_) * (uint64_t)sbr;                         \
    _Pragma("unroll") for (int u = 0; u < kDWLoads; ++u) {                                \
      const uint32_t off = u * 1024u + lane * 16u;                                        \
      stg[u] = *reinterpret_cast<const u32x4*>(wsrc_ + (off < wib ? off : 0u));           \
    }                                                                                     \
    _Pragma("unroll") for (int u = 0; u < kDSLoads; ++u) {                                \
      const uint32_t off = u * 1024u + lane * 16u;                                        \
      stg[kDWLoads + u] = *reinterpret_cast<const u32x4*>(ssrc_ + (off < sib ? off : 0u)); \
    }                                                                                     \
  } while (0)
#define DOWN_HOST_STORE()                                                                \
  do {                                                                                   \
    _Pragma("unroll") for (int u = 0; u < kDLoads; ++u)                                   \
      *reinterpret_cast<u32x4*>(buf + u * 1024 + lane * 16) = stg[u];                     \
  } while (0)
    auto compute = [&](int it) __attribute__((always_inline)) {
      const unsigned char* sbuf = buf + kDWLoads * 1024;
      const int a = it / per, o0 = (it - a * per) * 16;
      const int lo = lo_of(a), nt = ncols(a);
      const unsigned char* wrow = buf + r * (I / 2) + 32 * q;
      for (int pass = 0; pass * 16 < nt; ++pass) {
        const int j = pass * 16 + r;
        const bool has = j < nt;
        const int lrow = (has ? lo + j : lo) - ph0;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int c = 0; c < nchunk; ++c) {
          const bool ok = c != nchunk - 1 || lane_in_last;
          const uint32_t raw =
              *reinterpret_cast<const uint16_t*>(sbuf + (ok ? r * sbr + c * 8 + 2 * q : 0));
          const uint32_t b = ok ? raw : 0x7f7fu;
          const float s0 = e8m0_to_f32(b & 0xffu), s1 = e8m0_to_f32(b >> 8);
          AChunk w;
          w.lo = *reinterpret_cast<const uint4*>(wrow + c * 128);
          w.hi = *reinterpret_cast<const uint4*>(wrow + c * 128 + 16);
          const int e0 = c * kChunkElems + 64 * q;
#pragma unroll
          for (int m = 0; m < 8; ++m) {
            const bf16x8 bv =
                *reinterpret_cast<const bf16x8*>(hs + lds_elem(lrow, kpad, e0 + 8 * m));
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                dequant8(word_of(w, m), m < 4 ? s0 : s1), bv, acc, 0, 0, 0);
          }
        }
        // lane (r, q) holds output rows o0 + 4q + v of the pass's column r
        if (has) {
          const size_t sl = (uint32_t)l_slot[lrow];
          uint32_t yb[4];
#pragma unroll
          for (int v = 0; v < 4; ++v) yb[v] = f32_to_bf16_bits(acc[v]);
          *reinterpret_cast<uint2*>(Y + sl * H + o0 + 4 * q) =
              make_uint2(yb[0] | (yb[1] << 16), yb[2] | (yb[3] << 16));
        }
      }
    };
    // a wavefront only reads and writes its own item buffer, and LDS accesses
    // of one wavefront are ordered: no barrier between items
    int it = g0 + wv;
    if (it < g1 && ncols(it / per) == 0) it = next_item(it);
    if (it < g1) {
      DOWN_HOST_ISSUE(it);
      DOWN_HOST_STORE();
    }
    while (it < g1) {
      const int nx = next_item(it);
      if (nx < g1) DOWN_HOST_ISSUE(nx);
      compute(it);
      if (nx < g1) DOWN_HOST_STORE();
      it = nx;
    }
#undef DOWN_HOST_ISSUE
#undef DOWN_HOST_STORE
  }
}

int down_host_rows_that_fit(int I, int want) {
  const int kpad = (I + kChunkElems - 1) / kChunkElems * kChunkElems;
  const int fit = kDHElems / kpad;
  return fit < want ? fit : want;
}

// ---- gate/up ----------------------------------------------------------------
//
// Work item = 8 i-columns of one active expert: its 8 gate rows and 8 up rows
// (each run of 8 rows is 8 x H/2 contiguous bytes) make the 16 rows of one
// MFMA tile, gate in tile rows 0-7 and up in 8-15 (an output element depends
// only on its own row and column, so its bits do not depend on where the row
// sits in the tile). The item streams in windows of 4 chunks: 16 rows x 512
// bytes, 8 loads of 2 rows x 512 bytes each (the pattern the host link serves
// at full rate); the item's 16 scale rows come with its first window. A
// wavefront holds the next window in registers while it multiplies the
// current one out of its LDS window buffer; the prefetch runs straight across
// item boundaries. In LDS, granule j of row n sits at granule j ^ (n & 15)
// of the row, so the 16 rows of one operand read hit different banks.
// SwiGLU: lane (r, q) holds tile rows 4q..4q+3 of token column r, so gate
// columns are in lanes 0-31 and the matching up columns in lanes 32-63; one
// lane-half swap brings them together.

constexpr int kGW = 4;                       // wavefronts per workgroup (one per SIMD)
constexpr int kGThreads = 64 * kGW;
constexpr int kGMaxH = 4096;                 // largest H (scale rows of 8 x H/32 <= 1 KB)
constexpr int kGWinLoads = 8;                // loads per window (16 rows x 512 B)
constexpr int kGLoads = kGWinLoads + 2;      // + the two scale loads (first window only)
constexpr int kGWinBytes = kGWinLoads * 1024;
constexpr int kGXElems = 14 * kGMaxH;        // staged x rows (14 at H = 4096)

__global__ __launch_bounds__(kGThreads, 1) void ffn_gate_up_host(
    const uint8_t* __restrict__ w13, const uint8_t* __restrict__ s13,
    const int32_t* __restrict__ n_active, const int32_t* __restrict__ active_rows,
    const int32_t* __restrict__ row_off, const int32_t* __restrict__ slots,
    const __bf16* __restrict__ x, int k, int H, int I, int max_rows, uint16_t* __restrict__ h_ws) {
  __shared__ __align__(16) unsigned char wbuf[kGW][kGWinBytes];
  __shared__ __align__(16) unsigned char sbuf[kGW][2048];
  __shared__ __align__(16) __bf16 xs[kGXElems];
  __shared__ int l_slot[kGXElems / kChunkElems];
  const int kpad = H;                          // H is a multiple of 1024
  const int nwin = H / 1024;                   // windows of 4 chunks per row
  const uint32_t wrb = (uint32_t)H / 2u, srb = (uint32_t)H / 32u;
  const uint32_t shb = 8u * srb;               // scale bytes of 8 rows

  const int tid = threadIdx.x, lane = tid & 63, r = lane & 15, q = lane >> 4;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int na = __builtin_amdgcn_readfirstlane(*n_active);
  const int per = I / 8;
  const int n = na * per;
  if (n == 0) return;
  const int qb = (n + gridDim.x - 1) / gridDim.x;
  const int g0 = blockIdx.x * qb;
  if (g0 >= n) return;  // the whole workgroup, before any barrier
  const int g1 = min(n, g0 + qb);
  const int s_lo = __builtin_amdgcn_readfirstlane(row_off[g0 / per]);
  const int s_hi = __builtin_amdgcn_readfirstlane(row_off[(g1 - 1) / per + 1]);
  unsigned char* buf = wbuf[wv];
  unsigned char* sb = sbuf[wv];

  for (int ph0 = s_lo; ph0 < s_hi; ph0 += max_rows) {
    const int ph1 = min(s_hi, ph0 + max_rows);
    if (ph0 != s_lo) __syncthreads();  // the previous phase is done with the rows
    {
      const int gpr = kpad / 8, nr = ph1 - ph0;
      for (int gi = tid; gi < nr * gpr; gi += kGThreads) {
        const int m = gi / gpr, g = gi - m * gpr;
        const int sl = slots[ph0 + m];
        *reinterpret_cast<uint4*>(xs + lds_elem(m, kpad, g * 8)) =
            *reinterpret_cast<const uint4*>(x + (size_t)(sl / k) * H + g * 8);
      }
      for (int i = tid; i < nr; i += kGThreads) l_slot[i] = slots[ph0 + i];
    }
    __syncthreads();

    auto lo_of = [&](int a) { return max(__builtin_amdgcn_readfirstlane(row_off[a]), ph0); };
    auto ncols = [&](int a) {
      return min(__builtin_amdgcn_readfirstlane(row_off[a + 1]), ph1) - lo_of(a);
    };
    auto next_item = [&](int it) {
      for (it += kGW; it < g1; it += kGW)
        if (ncols(it / per) > 0) return it;
      return g1;
    };
    // A step = (item, 16-slot pass, window); the prefetch cursor runs one
    // step ahead of the arithmetic.
    struct Step { int it, pass, w; };
    auto next_step = [&](Step s) {
      if (++s.w < nwin) return s;
      s.w = 0;
      if (++s.pass * 16 < ncols(s.it / per)) return s;
      s.pass = 0;
      s.it = next_item(s.it);
      return s;
    };
    u32x4 stg[kGLoads];
    auto issue = [&](const Step& s) __attribute__((always_inline)) {
      const int a = s.it / per, i0 = (s.it - a * per) * 8;
      const uint64_t row = (uint32_t)__builtin_amdgcn_readfirstlane(active_rows[a]);
      const uint64_t e0 = row * 2 * (uint64_t)I;     // the expert's first w13 row
      // load u: tile rows 2u (lanes 0-31) and 2u + 1 (lanes 32-63)
#pragma unroll
      for (int u = 0; u < kGWinLoads; ++u) {
        const int tr = 2 * u + (lane >> 5);
        const uint64_t wr = e0 + (tr < 8 ? i0 + tr : I + i0 + tr - 8);
        stg[u] = *reinterpret_cast<const u32x4*>(w13 + wr * wrb + s.w * 512u + (lane & 31) * 16u);
      }
      // scale rows of the 8 gate rows, then of the 8 up rows (H/32 bytes each,
      // contiguous); after the first window the loads read one granule
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const uint32_t off = lane * 16u;
        const uint64_t sr = e0 + (u == 0 ? i0 : I + i0);
        stg[kGWinLoads + u] =
            *reinterpret_cast<const u32x4*>(s13 + sr * srb + (s.w == 0 && off < shb ? off : 0u));
      }
    };
    auto store = [&](const Step& s) __attribute__((always_inline)) {
#pragma unroll
      for (int u = 0; u < kGWinLoads; ++u) {
        const int tr = 2 * u + (lane >> 5), j = lane & 31;
        *reinterpret_cast<u32x4*>(buf + tr * 512 + 16 * (j ^ (tr & 15))) = stg[u];
      }
      if (s.w == 0) {
#pragma unroll
        for (int u = 0; u < 2; ++u)
          if (lane * 16u < shb) *reinterpret_cast<u32x4*>(sb + u * shb + lane * 16) = stg[kGWinLoads + u];
      }
    };
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    auto compute = [&](const Step& s) __attribute__((always_inline)) {
      const int a = s.it / per, i0 = (s.it - a * per) * 8;
      const int lo = lo_of(a), nt = ncols(a);
      const int j = s.pass * 16 + r;
      const bool has = j < nt;
      const int lrow = (has ? lo + j : lo) - ph0;
      if (s.w == 0) acc = f32x4{0.f, 0.f, 0.f, 0.f};
      const unsigned char* wrow = buf + r * 512;
#pragma unroll
      for (int cw = 0; cw < 4; ++cw) {
        const int c = 4 * s.w + cw;
        const uint32_t raw = *reinterpret_cast<const uint16_t*>(sb + r * srb + 8 * c + 2 * q);
        const float s0 = e8m0_to_f32(raw & 0xffu), s1 = e8m0_to_f32(raw >> 8);
        const int g = 8 * cw + 2 * q;
        AChunk wc;
        wc.lo = *reinterpret_cast<const uint4*>(wrow + 16 * (g ^ r));
        wc.hi = *reinterpret_cast<const uint4*>(wrow + 16 * ((g + 1) ^ r));
        const int e0 = c * kChunkElems + 64 * q;
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          const bf16x8 bv = *reinterpret_cast<const bf16x8*>(xs + lds_elem(lrow, kpad, e0 + 8 * m));
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dequant8(word_of(wc, m), m < 4 ? s0 : s1),
                                                        bv, acc, 0, 0, 0);
        }
      }
      if (s.w == nwin - 1) {
        // lanes 0-31 hold gate columns i0 + 4q + v, lanes 32-63 the same up
        // columns: bring the up values to the low half
        uint32_t hb[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[v]),
                                                           __float_as_uint(acc[v]), false, false);
          const float u = __uint_as_float(sw[1]);
          hb[v] = f32_to_bf16_bits(silu_f32(acc[v]) * u);
        }
        if (has && q < 2) {
          const size_t sl = (uint32_t)l_slot[lrow];
          *reinterpret_cast<uint2*>(h_ws + sl * I + i0 + 4 * q) =
              make_uint2(hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16));
        }
      }
    };
    Step cur{g0 + wv, 0, 0};
    if (cur.it < g1 && ncols(cur.it / per) == 0) cur.it = next_item(cur.it);
    if (cur.it < g1) issue(cur);
    while (cur.it < g1) {
      store(cur);
      const Step nx = next_step(cur);
      if (nx.it < g1) issue(nx);
      compute(cur);
      cur = nx;
    }
  }
}

int gate_up_host_rows_that_fit(int H, int want) {
  const int fit = kGXElems / H;
  return fit < want ? fit : want;
}

}  // namespace

bool ffn_use_down_host(int T, int k, int H, int I, const void* s2) {
  return T >= 1 && T <= kHostMaxTokens && I <= kDMaxI && I % 64 == 0 && H % 16 == 0 &&
         (reinterpret_cast<uintptr_t>(s2) & 15u) == 0 &&
         device_lds_per_block() >= 160 * 1024;
}

bool ffn_use_gate_up_host(int T, int k, int H, int I, const void* s13) {
  return T >= 1 && T <= kHostMaxTokens && H % 1024 == 0 && H <= kGMaxH && I % 8 == 0 &&
         (reinterpret_cast<uintptr_t>(s13) & 15u) == 0 &&
         device_lds_per_block() >= 160 * 1024;
}

hipError_t launch_gate_up_host(const uint8_t* w13, const uint8_t* s13, const moe_split& sp, int T,
                               int k, int H, int I, const uint16_t* x, uint16_t* h_ws,
                               hipStream_t stream) {
  const int max_rows = gate_up_host_rows_that_fit(H, T * k);
  hipLaunchKernelGGL(ffn_gate_up_host, dim3(kHostBankCUs), dim3(kGThreads), 0, stream, w13, s13,
                     sp.n_active, sp.active_rows, sp.row_off, sp.slots,
                     reinterpret_cast<const __bf16*>(x), k, H, I, max_rows, h_ws);
  return hipGetLastError();
}

hipError_t launch_down_host(const uint8_t* w2, const uint8_t* s2, const moe_split& sp, int T,
                            int k, int H, int I, const uint16_t* h_ws, uint16_t* Y,
                            hipStream_t stream) {
  const int max_rows = down_host_rows_that_fit(I, T * k);
  hipLaunchKernelGGL(ffn_down_host, dim3(kHostBankCUs), dim3(kDThreads), 0, stream, w2, s2,
                     sp.n_active, sp.active_rows, sp.row_off, sp.slots,
                     reinterpret_cast<const __bf16*>(h_ws), H, I, max_rows, Y);
  return hipGetLastError();
}

}  // namespace moe
