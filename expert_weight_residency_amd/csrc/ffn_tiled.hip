// Token-tiled MXFP4 expert FFN for steps with many tokens per expert (gfx950).
//
// Same operation as the decode kernels in ffn_mxfp4.hip (gate/up GEMM +
// SwiGLU into h, then the down GEMM into unweighted bf16 rows of Y; "vLLM: Pin
// Hot Experts", section "Results, September 17"), organised for calls where
// an expert has tens of tokens ("We Built the Counter", section 7: bigger
// steps want larger tiles than decode's 8 tokens). It runs below 256 tokens
// per step, when a bank averages 2 or more picks per row; from 256 tokens
// (prefill) the FP4 kernels of ffn_fp4.hip take over.
//
//  - Work item = (tile of up to 64 of one expert's slots, block of 512 weight
//    rows). A workgroup of 8 wavefronts runs one item; each wavefront owns 64
//    weight rows (4 MFMA groups of 16) and the 64 tokens (4 MFMA column groups
//    of 16), so every dequantized weight fragment feeds up to 4 MFMAs and the
//    weights are read once per 64 tokens instead of once per 8.
//  - The reduction axis streams in 256-element chunks. Activation chunks are
//    staged into two LDS buffers: while the wavefronts compute chunk c from
//    one buffer, their loads for chunk c+1 are in flight and land in the other
//    buffer before the one barrier per chunk. Weight chunks run kP ahead in a
//    register ring, issued after the activation loads so that waiting for the
//    activations never waits for the newest weights.
//  - Column groups with no valid token are skipped (uniform per tile).
//  - Each output element sees exactly the MFMA sequence of the decode kernel
//    (same chunks, same lane-to-element map, same order, from zero), and the
//    epilogues are the same code, so a pick gives the same bits from either
//    kernel family; which family runs is purely a speed choice.
//  - A persistent grid strides over the items. Items are ordered (expert,
//    weight block, tile) and handed out so that the workgroups of one XCD
//    (dispatch is round-robin over the 8 XCDs) take consecutive items: the
//    tiles of a heavy expert read each weight block from HBM once and share
//    it in that XCD's L2; for an expert with one tile, its blocks share the
//    activation chunks.
#include <type_traits>

#include "internal.h"
#include "mxfp4_common.h"
#include "tile_items.h"

namespace moe {
namespace {

using namespace mx;
using namespace tiles;

constexpr int kTok = 64;                         // tokens per tile
constexpr int kTokGroups = kTok / 16;            // MFMA column groups per tile
constexpr int kWaves = 8;                        // wavefronts per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kGroups = 4;                       // 16-row MFMA groups per wavefront
constexpr int kP = 1;                            // weight chunks in flight per wavefront
constexpr int kBufElems = kTok * kChunkElems;    // bf16 elements of one LDS buffer
constexpr int kGranules = kChunkElems / 8;       // 16-byte granules per row chunk
constexpr int kStage = kTok * kGranules / kThreads;  // granules staged per thread per chunk
constexpr int kXcds = 8;
static_assert(kStage * kThreads == kTok * kGranules, "staging must cover the tile");
static_assert(kThreads / kGranules * kStage == kTok, "staging rows");

// kGateUp: gate/up GEMM + SwiGLU (src = x rows by token, dst = h by slot).
// Otherwise: down GEMM (src = h rows by slot, dst = Y by slot).
template <bool kGateUp>
__global__ __launch_bounds__(kThreads, 2) void ffn_tiled(
    const uint8_t* __restrict__ w, const uint8_t* __restrict__ s,
    const int32_t* __restrict__ n_active, const int32_t* __restrict__ active_rows,
    const int32_t* __restrict__ row_off, const int32_t* __restrict__ slots,
    const __bf16* __restrict__ src, int k, int H, int I, int blocks_per_tile,
    uint16_t* __restrict__ dst) {
  extern __shared__ __align__(16) unsigned char smem[];
  __bf16* xs = reinterpret_cast<__bf16*>(smem);          // [2][kTok][256]
  int* tpre = reinterpret_cast<int*>(xs + 2 * kBufElems);  // [na + 1]
  __shared__ int wsum[kWaves];

  const int K = kGateUp ? H : I;       // reduction length
  const int ncols = kGateUp ? I : H;   // output columns per slot
  const int nblk = K / 32, nchunk = (K + kChunkElems - 1) / kChunkElems;
  const size_t wrb = K / 2, srb = K / 32;
  const size_t rows_per_expert = kGateUp ? 2 * (size_t)I : (size_t)H;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int r = lane & 15, q = lane >> 4;

  const int na = *n_active;
  build_tile_prefix<kTok, kWaves>(row_off, na, tpre, wsum);
  const int items = tpre[na] * blocks_per_tile;

  // Workgroup b runs on XCD b % 8 (dispatch is round-robin over the XCDs):
  // give the workgroups of one XCD consecutive logical indices.
  const int G = gridDim.x;
  const int G8 = G - G % kXcds;
  const int b = blockIdx.x;
  const int lb = b < G8 ? (b % kXcds) * (G8 / kXcds) + b / kXcds : b;

  // This thread's staging granule and its kStage tile rows.
  const int sg = tid % kGranules;
  const int sn0 = tid / kGranules;  // rows sn0 + (kThreads / kGranules) * u

  for (int item = lb; item < items; item += G) {
    // Items of active row a occupy [blocks * tpre[a], blocks * tpre[a+1]),
    // ordered (block, tile): the tiles of one weight block are consecutive,
    // so they run side by side on one XCD and read the block's weights from
    // HBM once.
    const int a = row_of_tile(tpre, na, item / blocks_per_tile);
    const int ntl = tpre[a + 1] - tpre[a];
    const int li = item - blocks_per_tile * tpre[a];
    const int blk = li / ntl, tl = li - blk * ntl;
    const int t0 = row_off[a] + tl * kTok;
    const int nvalid = min(kTok, row_off[a + 1] - t0);
    const int ntg = (nvalid + 15) / 16;

    // Rows of this wavefront: 4 groups of 16. Gate/up: gate i0, i0+16 and up
    // I+i0, I+i0+16 for i-columns i0..i0+31. Down: output rows c0..c0+63.
    const int c0 = (blk * kWaves + wv) * (kGateUp ? 32 : 64);
    const bool busy = c0 < ncols;
    const size_t row = active_rows[a];
    const uint8_t* wexp = w + row * rows_per_expert * wrb;
    const uint8_t* sexp = s + row * rows_per_expert * srb;
    const uint8_t* wrow[kGroups];
    const uint8_t* srow[kGroups];
#pragma unroll
    for (int g = 0; g < kGroups; ++g) {
      size_t wr;
      if (kGateUp) wr = (g < 2 ? 0 : (size_t)I) + c0 + 16 * (g & 1) + r;
      else wr = (size_t)c0 + 16 * g + r;
      if (!busy) wr = r;
      wrow[g] = wexp + wr * wrb;
      srow[g] = sexp + wr * srb;
    }

    // Staging: this thread's kStage tile rows. Every load is issued
    // unconditionally from an in-bounds address (a missing token reads the
    // tile's first row, a granule past K reads the row's first granule) and zeroed when it
    // is written to LDS, so the loads never sit under a branch: the in-order
    // vector-memory counter then lets a wavefront wait for one load without
    // draining the ones issued after it.
    const __bf16* sp[kStage];
    uint32_t svalid = 0;
#pragma unroll
    for (int u = 0; u < kStage; ++u) {
      const int n = sn0 + (kThreads / kGranules) * u;
      const int sl = slots[t0 + (n < nvalid ? n : 0)];
      sp[u] = kGateUp ? src + (size_t)(sl / k) * H : src + (size_t)sl * I;
      svalid |= (n < nvalid ? 1u : 0u) << u;
    }
    uint4 stg[kStage];
    int stage_e = 0;
    auto stage_load = [&](int c) {
      stage_e = c * kChunkElems + 8 * sg;
      const int e = stage_e < K ? stage_e : 0;
#pragma unroll
      for (int u = 0; u < kStage; ++u) stg[u] = *reinterpret_cast<const uint4*>(sp[u] + e);
    };
    auto stage_store = [&](int buf) {
      const bool in_k = stage_e < K;
#pragma unroll
      for (int u = 0; u < kStage; ++u) {
        const int n = sn0 + (kThreads / kGranules) * u;
        const bool keep = in_k && ((svalid >> u) & 1u);
        *reinterpret_cast<uint4*>(xs + buf * kBufElems + lds_elem(n, kChunkElems, 8 * sg)) =
            keep ? stg[u] : make_uint4(0, 0, 0, 0);
      }
    };

    f32x4 acc[kGroups][kTokGroups];
#pragma unroll
    for (int g = 0; g < kGroups; ++g)
#pragma unroll
      for (int t = 0; t < kTokGroups; ++t) acc[g][t] = f32x4{0.f, 0.f, 0.f, 0.f};

    // The chunk loop, specialised on the number of column groups with a token.
    auto run = [&](auto ntc) {
      constexpr int NT = decltype(ntc)::value;
      // Chunk indices past the end read block 0 of the row (load_a clamps), so
      // the prefetch is unconditional too.
      AChunk ring[kP + 1][kGroups];
#pragma unroll
      for (int p = 0; p < kP; ++p)
#pragma unroll
        for (int g = 0; g < kGroups; ++g) load_a(ring[p][g], wrow[g], srow[g], p, q, nblk);
      stage_load(0);
      stage_store(0);
      __syncthreads();
      for (int c = 0; c < nchunk; c += kP + 1) {
#pragma unroll
        for (int u = 0; u <= kP; ++u) {
          const int cc = c + u;
          if (cc >= nchunk) break;
          stage_load(cc + 1);
#pragma unroll
          for (int g = 0; g < kGroups; ++g)
            load_a(ring[(u + kP) % (kP + 1)][g], wrow[g], srow[g], cc + kP, q, nblk);
          const bool ok = cc * kChunkBlocks + 2 * q < nblk;
          float sc[kGroups][2];
#pragma unroll
          for (int g = 0; g < kGroups; ++g) chunk_scales(ring[u][g], ok, sc[g][0], sc[g][1]);
          const __bf16* xb = xs + (cc & 1) * kBufElems;
#pragma unroll
          for (int m = 0; m < 8; ++m) {
            bf16x8 bv[NT];
#pragma unroll
            for (int t = 0; t < NT; ++t)
              bv[t] = *reinterpret_cast<const bf16x8*>(
                  xb + lds_elem(16 * t + r, kChunkElems, 64 * q + 8 * m));
#pragma unroll
            for (int g = 0; g < kGroups; ++g) {
              const bf16x8 av = dequant8(word_of(ring[u][g], m), sc[g][m >> 2]);
#pragma unroll
              for (int t = 0; t < NT; ++t)
                acc[g][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv[t], acc[g][t], 0, 0, 0);
            }
          }
          // The buffer written here was last read in the previous chunk, which
          // every wavefront finished before the last barrier.
          stage_store((cc + 1) & 1);
          __syncthreads();
        }
      }
    };

    if (busy) {
      switch (ntg) {
        case 1: run(std::integral_constant<int, 1>{}); break;
        case 2: run(std::integral_constant<int, 2>{}); break;
        case 3: run(std::integral_constant<int, 3>{}); break;
        default: run(std::integral_constant<int, 4>{}); break;
      }
    } else {
      // A wavefront past the last weight row only helps stage.
      stage_load(0);
      stage_store(0);
      __syncthreads();
      for (int cc = 0; cc < nchunk; ++cc) {
        stage_load(cc + 1);
        stage_store((cc + 1) & 1);
        __syncthreads();
      }
    }

    // Epilogue: lane (r, q) holds rows 4q + v of each group for token 16t + r.
    if (busy) {
#pragma unroll
      for (int t = 0; t < kTokGroups; ++t) {
        const int n = 16 * t + r;
        if (t < ntg && n < nvalid) {
          const size_t sl = slots[t0 + n];
          if (kGateUp) {
#pragma unroll
            for (int half = 0; half < 2; ++half) {
              uint32_t hb[4];
#pragma unroll
              for (int v = 0; v < 4; ++v)
                hb[v] = f32_to_bf16_bits(silu_f32(acc[half][t][v]) * acc[2 + half][t][v]);
              *reinterpret_cast<uint2*>(dst + sl * I + c0 + 16 * half + 4 * q) =
                  make_uint2(hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16));
            }
          } else {
#pragma unroll
            for (int g = 0; g < kGroups; ++g) {
              uint32_t yb[4];
#pragma unroll
              for (int v = 0; v < 4; ++v) yb[v] = f32_to_bf16_bits(acc[g][t][v]);
              *reinterpret_cast<uint2*>(dst + sl * H + c0 + 16 * g + 4 * q) =
                  make_uint2(yb[0] | (yb[1] << 16), yb[2] | (yb[3] << 16));
            }
          }
        }
      }
    }
  }
}

size_t tiled_lds_bytes(int cap) {
  return 2 * (size_t)kBufElems * sizeof(uint16_t) + ((size_t)cap + 1) * sizeof(int);
}

// Workgroups for a launch (items are grid-strided). A device bank gets one
// workgroup per CU less the CUs a concurrent host-bank launch holds: a
// workgroup that cannot be placed would run its share of the items after
// everyone else (one workgroup per item instead measured ~20% slower from
// workgroup turnover). A host-resident bank gets kTiledHostWaves wavefronts.
unsigned tiled_grid(int cap, int T, int k, int blocks, int on_host) {
  const long long max_tiles = (long long)T * k / kTok + cap;
  const long long max_items = max_tiles * blocks;
  const int host_wgs = kTiledHostWaves / kWaves;
  static_assert(kTiledHostWaves / kWaves == kHostBankCUs, "host-bank launch width");
  long long g = on_host ? host_wgs : device_cus() - host_wgs;
  if (g > max_items) g = max_items;
  return (unsigned)(g < 1 ? 1 : g);
}

}  // namespace

bool ffn_use_tiled(int T, int k, int cap) {
  return (long long)T * k >= (long long)kTiledMinPicksPerRow * cap;
}

hipError_t launch_gate_up_tiled(const uint8_t* w13, const uint8_t* s13, int cap, int on_host,
                                const moe_split& sp, const uint16_t* x, int T, int k, int H, int I,
                                uint16_t* h_ws, hipStream_t stream) {
  const int blocks = (I / 32 + kWaves - 1) / kWaves;
  hipLaunchKernelGGL(ffn_tiled<true>, dim3(tiled_grid(cap, T, k, blocks, on_host)),
                     dim3(kThreads), tiled_lds_bytes(cap), stream, w13, s13, sp.n_active,
                     sp.active_rows, sp.row_off, sp.slots, reinterpret_cast<const __bf16*>(x), k,
                     H, I, blocks, h_ws);
  return hipGetLastError();
}

hipError_t launch_down_tiled(const uint8_t* w2, const uint8_t* s2, int cap, int on_host,
                             const moe_split& sp, int T, int k, int H, int I,
                             const uint16_t* h_ws, uint16_t* Y, hipStream_t stream) {
  const int blocks = (H / 64 + kWaves - 1) / kWaves;
  hipLaunchKernelGGL(ffn_tiled<false>, dim3(tiled_grid(cap, T, k, blocks, on_host)),
                     dim3(kThreads), tiled_lds_bytes(cap), stream, w2, s2, sp.n_active,
                     sp.active_rows, sp.row_off, sp.slots,
                     reinterpret_cast<const __bf16*>(h_ws), k, H, I, blocks, Y);
  return hipGetLastError();
}

}  // namespace moe
