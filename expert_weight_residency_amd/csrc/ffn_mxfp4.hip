// Grouped MXFP4 expert FFN over one residency bank (gfx950).
//
// Computes, for every active bank row r and every slot s routed to it, the
// unweighted expert row Y[s] = bf16(Wdown[r] . (silu(Wgate[r] . x) * (Wup[r] . x)))
// ("vLLM: Pin Hot Experts", section "Results, September 17": the routed MXFP4
// MoE called once per bank with finalization deferred; "Where the experts live
// today": MXFP4 weights with ue8m0 block scales). The same kernels read the
// hot bank from HBM and the cold bank from pinned host memory in place ("We
// Built the Counter", section 1).
//
// Design for decode, where the layer is bound by streaming expert weights:
//  - A workgroup of 8 wavefronts owns one active row (expert) and a block of
//    its weight rows; each wavefront owns 2 groups of 16 rows and walks the
//    whole reduction axis, so each weight byte is read from HBM once per step
//    (the pages' kernel re-reads an expert for every extra 8-token tile: "We
//    Built the Counter", section 6).
//  - The activation rows of up to kTT of the expert's tokens are staged once in
//    LDS (XOR-swizzled 16-byte granules, zero-padded to whole chunks), and the
//    MFMA B operand is read from there. Only weight loads remain in the
//    vector-memory queue, which completes in order, so each wavefront can keep
//    kP chunks of weights in flight in a register ring without waiting on
//    activation traffic.
//  - A lane (r, q) = (lane % 16, lane / 16) loads 32 contiguous bytes of row r
//    per 256-element chunk (two E8M0 blocks), so the four lanes of a row cover a
//    full 128-byte line; the chunk's two scale bytes come with it.
//  - E2M1 codes become bf16 with v_cvt_scalef32_pk_bf16_fp4 (the E8M0 scale is
//    applied in the convert; exact for scale bytes below 253) and accumulate in
//    fp32 on v_mfma_f32_16x16x32_bf16: no activation quantization, and the
//    VALU work per weight byte does not grow with the tokens per expert.
//  - Loads past the end of the reduction axis read a clamped in-bounds address
//    with unit scale; the matching activations are the LDS zero padding.
//  - The reduction order of an output element depends only on K and the chunk
//    constants, never on the bank, the row, the grid or the other tokens, so a
//    pick gives the same bits from either bank.
//  - Kernel 1 pairs gate rows i0..i0+15 with up rows I+i0..I+i0+15 in one
//    wavefront and applies SwiGLU in registers; h goes to the workspace as
//    bf16. Kernel 2 (down) reads h for the expert's slots and writes Y rows.
//  - Experts with more than kTT tokens take several passes; a pass re-reads the
//    workgroup's weight block right after the previous one, mostly from L2.
//  - Work items are (active row, row block); a grid-stride loop lets a bank in
//    host memory run on a capped number of wavefronts (see kHostReadWaves).
#include "internal.h"
#include "mxfp4_common.h"

namespace moe {
namespace {

using namespace mx;

constexpr int kWavesDevice = 8;   // wavefronts per workgroup (device bank)
constexpr int kWavesHost = 8;     // ... and for a host-resident bank
constexpr int kTT = 8;            // most tokens staged per pass
constexpr int kLdsTile = 65536;   // LDS bytes of the activation tile
constexpr int kPDevice = 2;       // weight chunks in flight per wavefront (device bank)
constexpr int kPHost = 4;         // ... and for a host-resident bank (few wavefronts)
constexpr int kNG = 2;            // 16-row MFMA groups per wavefront
// (Device banks: 4 waves per SIMD, two 8-wave workgroups per CU, no spills.)
// Wavefronts that read a host-resident bank at once. Host-link reads in flight
// beyond what saturates the link only back up the memory path that concurrent
// HBM-bound kernels use, so the count is capped; with 4 chunks in flight per
// wavefront, 64 wavefronts on 8 CUs reach ~42 GB/s while a concurrent hot-bank
// kernel keeps ~95% of its speed. (Spreading the same wavefronts over 32 CUs
// reads the link slightly faster but slows the hot bank 2.5x.)
constexpr int kHostReadWaves = 64;
static_assert(kHostReadWaves / kWavesHost == kHostBankCUs, "host-bank launch width");

// Stage rows src_row(n) for n < nvalid into the LDS tile, zero past K.
template <typename RowFn>
__device__ __forceinline__ void stage_rows(__bf16* xs, int nvalid, int K, int kpad, RowFn src_row) {
  const int gpr = kpad / 8;  // granules per row
  for (int gi = threadIdx.x; gi < nvalid * gpr; gi += blockDim.x) {
    const int n = gi / gpr, g = gi - n * gpr;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (g * 8 < K) v = *reinterpret_cast<const uint4*>(src_row(n) + g * 8);
    *reinterpret_cast<uint4*>(xs + lds_elem(n, kpad, g * 8)) = v;
  }
}

// acc[g] += W[group g] (16 x K, MXFP4) . B (K x 16 tokens, bf16 in LDS) over
// the whole reduction axis, with P chunks of weights in flight in a register
// ring (indexed statically: the chunk loop is unrolled by P + 1). P does not
// change the arithmetic, only how far ahead the loads run. nrow: LDS
// row this lane's token column reads (its token, or row 0 when it has none).
template <int kP>
__device__ __forceinline__ void mx_gemm(const uint8_t* const* wrow, const uint8_t* const* srow,
                                        int nblk, const __bf16* xs, int kpad, int nrow, int q,
                                        f32x4 (&acc)[kNG]) {
  const int nchunk = (nblk + kChunkBlocks - 1) / kChunkBlocks;
  AChunk ring[kP + 1][kNG];
#pragma unroll
  for (int p = 0; p < kP; ++p)
    if (p < nchunk)
#pragma unroll
      for (int g = 0; g < kNG; ++g) load_a(ring[p][g], wrow[g], srow[g], p, q, nblk);
  for (int c = 0; c < nchunk; c += kP + 1) {
#pragma unroll
    for (int u = 0; u <= kP; ++u) {
      const int cc = c + u;
      if (cc >= nchunk) break;
      if (cc + kP < nchunk) {
#pragma unroll
        for (int g = 0; g < kNG; ++g)
          load_a(ring[(u + kP) % (kP + 1)][g], wrow[g], srow[g], cc + kP, q, nblk);
      }
      const bool ok = cc * kChunkBlocks + 2 * q < nblk;
      const int e0 = cc * kChunkElems + 64 * q;
      float sc[kNG][2];
#pragma unroll
      for (int g = 0; g < kNG; ++g) chunk_scales(ring[u][g], ok, sc[g][0], sc[g][1]);
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const bf16x8 bv = *reinterpret_cast<const bf16x8*>(xs + lds_elem(nrow, kpad, e0 + 8 * m));
#pragma unroll
        for (int g = 0; g < kNG; ++g)
          acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              dequant8(word_of(ring[u][g], m), sc[g][m >> 2]), bv, acc[g], 0, 0, 0);
      }
    }
  }
}


// Kernel 1: h[s][i] = silu(gate_i . x_t) * (up_i . x_t) for the slots of each
// active row. Work item = kW wavefronts of one active row; wavefront w of
// block b owns i-rows i0 = (b * kW + w) * 16 .. i0 + 15 (gate and up).
template <int kP, int kW>
__global__ __launch_bounds__(64 * kW, kP <= 2 ? 4 : 2) void ffn_gate_up(
    const uint8_t* __restrict__ w13, const uint8_t* __restrict__ s13,
    const int32_t* __restrict__ n_active, const int32_t* __restrict__ active_rows,
    const int32_t* __restrict__ row_off, const int32_t* __restrict__ slots,
    const __bf16* __restrict__ x, int k, int H, int I, int blocks_per_row, int tt,
    uint16_t* __restrict__ h_ws) {
  extern __shared__ __align__(16) unsigned char smem[];
  __bf16* xs = reinterpret_cast<__bf16*>(smem);
  const int kpad = (H + kChunkElems - 1) / kChunkElems * kChunkElems;
  const int items = *n_active * blocks_per_row;
  const int lane = threadIdx.x & 63, r = lane & 15, q = lane >> 4;
  const size_t wrb = H / 2, srb = H / 32;
  const int nblk = H / 32;
  for (int item = blockIdx.x; item < items; item += gridDim.x) {
    const int a = item / blocks_per_row;
    const int i0 = ((item % blocks_per_row) * kW + (threadIdx.x >> 6)) * 16;
    const bool busy = i0 < I;
    const size_t row = active_rows[a];
    const uint8_t* wexp = w13 + row * (2 * (size_t)I) * wrb;
    const uint8_t* sexp = s13 + row * (2 * (size_t)I) * srb;
    const size_t ri = busy ? i0 + r : r;
    const uint8_t* const wrow[kNG] = {wexp + ri * wrb, wexp + (I + ri) * wrb};
    const uint8_t* const srow[kNG] = {sexp + ri * srb, sexp + (I + ri) * srb};
    const int s_beg = row_off[a], s_end = row_off[a + 1];
    for (int t0 = s_beg; t0 < s_end; t0 += tt) {
      const int nvalid = min(tt, s_end - t0);
      __syncthreads();  // previous pass done with the tile
      stage_rows(xs, nvalid, H, kpad,
                 [&](int n) { return x + (size_t)(slots[t0 + n] / k) * H; });
      __syncthreads();
      if (busy) {
        f32x4 acc[kNG] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
        mx_gemm<kP>(wrow, srow, nblk, xs, kpad, r < nvalid ? r : 0, q, acc);
        // lane (r, q) holds i-rows i0 + 4q + v of token r
        if (r < nvalid) {
          uint32_t hb[4];
#pragma unroll
          for (int v = 0; v < 4; ++v) hb[v] = f32_to_bf16_bits(silu_f32(acc[0][v]) * acc[1][v]);
          *reinterpret_cast<uint2*>(h_ws + (size_t)slots[t0 + r] * I + i0 + 4 * q) =
              make_uint2(hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16));
        }
      }
    }
  }
}

// Kernel 2: Y[s][o] = bf16(down_o . h_s). Work item = kW wavefronts of one
// active row; wavefront w of block b owns output rows o0 = (b * kW + w) *
// 32 .. o0 + 31.
template <int kP, int kW>
__global__ __launch_bounds__(64 * kW, kP <= 2 ? 4 : 2) void ffn_down(
    const uint8_t* __restrict__ w2, const uint8_t* __restrict__ s2,
    const int32_t* __restrict__ n_active, const int32_t* __restrict__ active_rows,
    const int32_t* __restrict__ row_off, const int32_t* __restrict__ slots,
    const uint16_t* __restrict__ h_ws, int H, int I, int blocks_per_row, int tt,
    uint16_t* __restrict__ Y) {
  extern __shared__ __align__(16) unsigned char smem[];
  __bf16* xs = reinterpret_cast<__bf16*>(smem);
  const int kpad = (I + kChunkElems - 1) / kChunkElems * kChunkElems;
  const int items = *n_active * blocks_per_row;
  const int lane = threadIdx.x & 63, r = lane & 15, q = lane >> 4;
  const size_t wrb = I / 2, srb = I / 32;
  const int nblk = I / 32;
  const __bf16* hb = reinterpret_cast<const __bf16*>(h_ws);
  for (int item = blockIdx.x; item < items; item += gridDim.x) {
    const int a = item / blocks_per_row;
    const int o0 = ((item % blocks_per_row) * kW + (threadIdx.x >> 6)) * 16 * kNG;
    const bool busy = o0 < H;
    const size_t row = active_rows[a];
    const uint8_t* wexp = w2 + row * (size_t)H * wrb;
    const uint8_t* sexp = s2 + row * (size_t)H * srb;
    const size_t ro = busy ? o0 + r : r;
    const uint8_t* const wrow[kNG] = {wexp + ro * wrb, wexp + (ro + 16) * wrb};
    const uint8_t* const srow[kNG] = {sexp + ro * srb, sexp + (ro + 16) * srb};
    const int s_beg = row_off[a], s_end = row_off[a + 1];
    for (int t0 = s_beg; t0 < s_end; t0 += tt) {
      const int nvalid = min(tt, s_end - t0);
      __syncthreads();
      stage_rows(xs, nvalid, I, kpad, [&](int n) { return hb + (size_t)slots[t0 + n] * I; });
      __syncthreads();
      if (busy) {
        f32x4 acc[kNG] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
        mx_gemm<kP>(wrow, srow, nblk, xs, kpad, r < nvalid ? r : 0, q, acc);
        if (r < nvalid) {
          const size_t ybase = (size_t)slots[t0 + r] * H + o0 + 4 * q;
#pragma unroll
          for (int g = 0; g < kNG; ++g) {
            uint32_t yb[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) yb[v] = f32_to_bf16_bits(acc[g][v]);
            *reinterpret_cast<uint2*>(Y + ybase + 16 * g) =
                make_uint2(yb[0] | (yb[1] << 16), yb[2] | (yb[3] << 16));
          }
        }
      }
    }
  }
}

// Blocks launched for `items` work items: all of them for a device bank, at
// most kHostReadWaves wavefronts' worth for a host-resident bank.
unsigned grid_for(int items, int on_host) {
  const int cap = kHostReadWaves / kWavesHost;
  return (unsigned)(on_host && items > cap ? cap : items);
}

// Tokens per pass for reduction length K: as many as fit the LDS tile, at most kTT.
int tokens_per_pass(int K) {
  const int row = (K + kChunkElems - 1) / kChunkElems * kChunkElems * (int)sizeof(uint16_t);
  const int t = kLdsTile / row;
  return t < kTT ? t : kTT;
}

size_t lds_bytes(int K) {
  return (size_t)tokens_per_pass(K) * ((K + kChunkElems - 1) / kChunkElems * kChunkElems) *
         sizeof(uint16_t);
}

}  // namespace

int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0) {
    (void)hipGetLastError();
    return 256;
  }
  return cus;
}

size_t device_lds_per_block() {
  int dev = 0, v = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess ||
      v <= 0) {
    (void)hipGetLastError();
    return 64 * 1024;
  }
  return (size_t)v;
}

int ffn_max_reduction() { return kLdsTile / (int)sizeof(uint16_t); }

hipError_t launch_gate_up(const uint8_t* w13, const uint8_t* s13, int cap, int on_host,
                          const moe_split& sp, const uint16_t* x, int T, int k, int H, int I,
                          uint16_t* h_ws, hipStream_t stream) {
  if (ffn_use_fp4(T))
    return launch_gate_up_fp4(w13, s13, cap, on_host, sp, x, T, k, H, I, h_ws, stream);
  if (on_host && ffn_use_gate_up_host(T, k, H, I, s13))
    return launch_gate_up_host(w13, s13, sp, T, k, H, I, x, h_ws, stream);
  if (ffn_use_resident(T, k, H, cap, s13))
    return launch_gate_up_resident(w13, s13, cap, on_host, sp, x, T, k, H, I, h_ws, stream);
  if (ffn_use_tiled(T, k, cap))
    return launch_gate_up_tiled(w13, s13, cap, on_host, sp, x, T, k, H, I, h_ws, stream);
  const int w = on_host ? kWavesHost : kWavesDevice;
  const int blocks = (I / 16 + w - 1) / w;
  auto kern = on_host ? ffn_gate_up<kPHost, kWavesHost> : ffn_gate_up<kPDevice, kWavesDevice>;
  hipLaunchKernelGGL(kern, dim3(grid_for(cap * blocks, on_host)), dim3(64 * w), lds_bytes(H),
                     stream, w13, s13, sp.n_active, sp.active_rows, sp.row_off, sp.slots,
                     reinterpret_cast<const __bf16*>(x), k, H, I, blocks, tokens_per_pass(H),
                     h_ws);
  return hipGetLastError();
}

constexpr int kSmallBankRows = 96;        // banks this small prefer the persistent down kernel
constexpr int kSmallBankPicksPerRow = 8;  // ... below this many picks per row

hipError_t launch_down(const uint8_t* w2, const uint8_t* s2, int cap, int on_host,
                       const moe_split& sp, int T, int k, int H, int I, const uint16_t* h_ws,
                       uint16_t* Y, hipStream_t stream) {
  if (ffn_use_fp4(T))
    return launch_down_fp4(w2, s2, cap, on_host, sp, T, k, H, I, h_ws, Y, stream);
  if (on_host && ffn_use_down_host(T, k, H, I, s2))
    return launch_down_host(w2, s2, sp, T, k, H, I, h_ws, Y, stream);
  // A device bank of few rows (the step's staged cold rows) holds few active
  // experts: the token-tiled kernel then runs one workgroup per 512 weight
  // rows per 64-token tile and leaves most CUs idle, while the persistent
  // kernel spreads 16-row items over all of them (89-row stage at T = 32, 64,
  // 112: 2.1, 1.7, 1.2% less per layer). From kSmallBankPicksPerRow picks per
  // row the tiled kernel's one weight read per 64 tokens counts for more.
  const bool small = !on_host && cap <= kSmallBankRows &&
                     (long long)T * k < (long long)kSmallBankPicksPerRow * cap;
  if (!small && ffn_use_tiled(T, k, cap))
    return launch_down_tiled(w2, s2, cap, on_host, sp, T, k, H, I, h_ws, Y, stream);
  if (ffn_use_down_resident(T, k, H, I, w2, s2, on_host))
    return launch_down_resident(w2, s2, cap, on_host, sp, T, k, H, I, h_ws, Y, stream);
  if (ffn_use_tiled(T, k, cap))
    return launch_down_tiled(w2, s2, cap, on_host, sp, T, k, H, I, h_ws, Y, stream);
  const int w = on_host ? kWavesHost : kWavesDevice;
  const int blocks = (H / (16 * kNG) + w - 1) / w;
  auto kern = on_host ? ffn_down<kPHost, kWavesHost> : ffn_down<kPDevice, kWavesDevice>;
  hipLaunchKernelGGL(kern, dim3(grid_for(cap * blocks, on_host)), dim3(64 * w), lds_bytes(I),
                     stream, w2, s2, sp.n_active, sp.active_rows, sp.row_off, sp.slots, h_ws, H, I,
                     blocks, tokens_per_pass(I), Y);
  return hipGetLastError();
}

}  // namespace moe
