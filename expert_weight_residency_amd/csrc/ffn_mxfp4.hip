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
//  - One wavefront owns 16 output rows x (up to) 16 tokens per MFMA tile and
//    walks the whole reduction axis, so every weight byte is read once per
//    step for up to 16*NT tokens of an expert (the pages' kernel re-reads an
//    expert per extra 8-token tile: "We Built the Counter", section 6).
//  - A lane (r, q) = (lane % 16, lane / 16) loads 32 contiguous bytes of row r
//    per 256-element chunk (two E8M0 blocks), so the four lanes of a row cover
//    a full 128-byte line; the chunk's two scale bytes come with it.
//  - E2M1 codes become bf16 with v_cvt_scalef32_pk_bf16_fp4 (scale applied in
//    the convert, exact for E8M0 bytes < 253), and the products accumulate in
//    fp32 on v_mfma_f32_16x16x32_bf16 with the bf16 activations (or h) as the
//    B operand: no activation quantization, and the VALU cost per weight byte
//    stays constant as tokens per expert grow.
//  - The reduction order of an output element depends only on K and the chunk
//    constants, never on the bank, the row, the grid or the other tokens, so a
//    pick gives the same bits from either bank.
//  - The next chunk's weights are loaded before the current chunk's MFMAs.
//  - Kernel 1 pairs gate rows i0..i0+15 with up rows I+i0.. in one wavefront and
//    applies SwiGLU in registers; h goes to the workspace as bf16.
//    Kernel 2 (down) reads h for the expert's slots and writes bf16 Y rows.
#include "internal.h"

namespace moe {
namespace {

constexpr int kWavesPerBlock = 4;
constexpr int kChunkElems = 256;  // reduction elements per chunk per row
constexpr int kChunkBlocks = 8;   // E8M0 blocks per chunk

__device__ __forceinline__ float e8m0_to_f32(uint32_t b) {
  // 2^(b-127) as an fp32 bit pattern; b = 0 is the subnormal 2^-127, 255 is NaN.
  const uint32_t bits = b == 0 ? 0x00400000u : (b == 255 ? 0x7fc00000u : (b << 23));
  return __uint_as_float(bits);
}

struct AChunk {
  uint4 lo, hi;  // 32 bytes = 64 E2M1 codes of one row: blocks 2q and 2q+1 of the chunk
  float s0, s1;  // their scales
};

// Whole chunk in range: no checks.
__device__ __forceinline__ void load_a(AChunk& a, const uint8_t* __restrict__ wrow,
                                       const uint8_t* __restrict__ srow, int c, int q) {
  const int b0 = c * kChunkBlocks + 2 * q;
  const uint4* p = reinterpret_cast<const uint4*>(wrow + b0 * 16);
  a.lo = p[0];
  a.hi = p[1];
  const uint32_t sc = *reinterpret_cast<const uint16_t*>(srow + b0);
  a.s0 = e8m0_to_f32(sc & 0xffu);
  a.s1 = e8m0_to_f32(sc >> 8);
}

// Tail chunk: blocks at or past nblk read as zero codes.
__device__ __forceinline__ void load_a_tail(AChunk& a, const uint8_t* __restrict__ wrow,
                                            const uint8_t* __restrict__ srow, int c, int q,
                                            int nblk) {
  const int b0 = c * kChunkBlocks + 2 * q;
  a.lo = make_uint4(0, 0, 0, 0);
  a.hi = make_uint4(0, 0, 0, 0);
  a.s0 = 1.0f;
  a.s1 = 1.0f;
  if (b0 < nblk) {
    a.lo = *reinterpret_cast<const uint4*>(wrow + b0 * 16);
    a.s0 = e8m0_to_f32(srow[b0]);
  }
  if (b0 + 1 < nblk) {
    a.hi = *reinterpret_cast<const uint4*>(wrow + b0 * 16 + 16);
    a.s1 = e8m0_to_f32(srow[b0 + 1]);
  }
}

__device__ __forceinline__ uint32_t word_of(const AChunk& a, int m) {
  const uint4& v = m < 4 ? a.lo : a.hi;
  switch (m & 3) {
    case 0: return v.x;
    case 1: return v.y;
    case 2: return v.z;
    default: return v.w;
  }
}

// 8 E2M1 codes (one dword, low nibble first) times a power-of-two scale -> 8 bf16.
__device__ __forceinline__ bf16x8 dequant8(uint32_t w, float s) {
  const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 0);
  const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 1);
  const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 2);
  const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 3);
  return bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

__device__ __forceinline__ bf16x8 load_b(const __bf16* __restrict__ row, int off) {
  return *reinterpret_cast<const bf16x8*>(row + off);
}

// acc[j][g] += W[g rows] (16 x K, MXFP4) . B[j] (K x 16 tokens, bf16) over the
// whole reduction axis. wrow/srow: this lane's row (lane % 16) of group g.
// brow[j]: this lane's token row (token lane % 16 of tile j), or null.
template <int NT, int NG>
__device__ __forceinline__ void mx_gemm(const uint8_t* const* wrow, const uint8_t* const* srow,
                                        int nblk, const __bf16* const* brow, int ntile, int q,
                                        f32x4 (&acc)[NT][NG]) {
  const int nfull = nblk / kChunkBlocks;
  const int nchunk = (nblk + kChunkBlocks - 1) / kChunkBlocks;
  const bf16x8 zero8 = {};
  AChunk cur[NG], nxt[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    if (nfull > 0)
      load_a(cur[g], wrow[g], srow[g], 0, q);
    else
      load_a_tail(cur[g], wrow[g], srow[g], 0, q, nblk);
  }
  for (int c = 0; c < nchunk; ++c) {
    if (c + 1 < nfull) {
#pragma unroll
      for (int g = 0; g < NG; ++g) load_a(nxt[g], wrow[g], srow[g], c + 1, q);
    } else if (c + 1 < nchunk) {
#pragma unroll
      for (int g = 0; g < NG; ++g) load_a_tail(nxt[g], wrow[g], srow[g], c + 1, q, nblk);
    }
    const int base = c * kChunkElems + 64 * q;
    const bool tail = c >= nfull;
    const int b0 = c * kChunkBlocks + 2 * q;
    const bool v0 = !tail || b0 < nblk, v1 = !tail || b0 + 1 < nblk;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const bool valid = m < 4 ? v0 : v1;
      bf16x8 av[NG];
#pragma unroll
      for (int g = 0; g < NG; ++g) av[g] = dequant8(word_of(cur[g], m), m < 4 ? cur[g].s0 : cur[g].s1);
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        if (j < ntile) {
          const bf16x8 bv = (brow[j] != nullptr && valid) ? load_b(brow[j], base + 8 * m) : zero8;
#pragma unroll
          for (int g = 0; g < NG; ++g)
            acc[j][g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[g], bv, acc[j][g], 0, 0, 0);
        }
      }
    }
    if (c + 1 < nchunk) {
#pragma unroll
      for (int g = 0; g < NG; ++g) cur[g] = nxt[g];
    }
  }
}

__device__ __forceinline__ float silu_f32(float z) { return z / (1.0f + __expf(-z)); }

// Kernel 1: h[s][i] = silu(gate_i . x_t) * (up_i . x_t) for the slots of each
// active row. Wave = one 16-row i-block (gate + up) of one active row.
template <int NT>
__global__ __launch_bounds__(64 * kWavesPerBlock) void ffn_gate_up(
    const uint8_t* __restrict__ w13, const uint8_t* __restrict__ s13,
    const int32_t* __restrict__ n_active, const int32_t* __restrict__ active_rows,
    const int32_t* __restrict__ row_off, const int32_t* __restrict__ slots,
    const __bf16* __restrict__ x, int k, int H, int I, int blocks_per_row,
    uint16_t* __restrict__ h_ws) {
  const int a = blockIdx.x / blocks_per_row;
  if (a >= *n_active) return;
  const int ib = (blockIdx.x % blocks_per_row) * kWavesPerBlock + (threadIdx.x >> 6);
  const int i0 = ib * 16;
  if (i0 >= I) return;
  const int lane = threadIdx.x & 63, r = lane & 15, q = lane >> 4;
  const size_t wrb = H / 2, srb = H / 32;
  const size_t row = active_rows[a];
  const uint8_t* wexp = w13 + row * (2 * (size_t)I) * wrb;
  const uint8_t* sexp = s13 + row * (2 * (size_t)I) * srb;
  const uint8_t* const wrow[2] = {wexp + (i0 + r) * wrb, wexp + (I + i0 + r) * wrb};
  const uint8_t* const srow[2] = {sexp + (i0 + r) * srb, sexp + (I + i0 + r) * srb};
  const int nblk = H / 32;
  const int s_beg = row_off[a], s_end = row_off[a + 1];

  for (int t0 = s_beg; t0 < s_end; t0 += 16 * NT) {
    const int ntile = min(NT, (s_end - t0 + 15) / 16);
    int slot[NT];
    const __bf16* brow[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int idx = t0 + 16 * j + r;
      slot[j] = idx < s_end ? slots[idx] : -1;
      brow[j] = slot[j] >= 0 ? x + (size_t)(slot[j] / k) * H : nullptr;
    }
    f32x4 acc[NT][2];
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[j][0] = acc[j][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    mx_gemm<NT, 2>(wrow, srow, nblk, brow, ntile, q, acc);
    // lane (r, q) holds rows i0 + 4q + v of token r of each tile
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      if (j < ntile && slot[j] >= 0) {
        uint32_t hb[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) hb[v] = f32_to_bf16_bits(silu_f32(acc[j][0][v]) * acc[j][1][v]);
        uint2 pk = make_uint2(hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16));
        *reinterpret_cast<uint2*>(h_ws + (size_t)slot[j] * I + i0 + 4 * q) = pk;
      }
    }
  }
}

// Kernel 2: Y[s][o] = bf16(down_o . h_s). Wave = 16*NG output rows of one active row.
template <int NT, int NG>
__global__ __launch_bounds__(64 * kWavesPerBlock) void ffn_down(
    const uint8_t* __restrict__ w2, const uint8_t* __restrict__ s2,
    const int32_t* __restrict__ n_active, const int32_t* __restrict__ active_rows,
    const int32_t* __restrict__ row_off, const int32_t* __restrict__ slots,
    const uint16_t* __restrict__ h_ws, int H, int I, int blocks_per_row,
    uint16_t* __restrict__ Y) {
  const int a = blockIdx.x / blocks_per_row;
  if (a >= *n_active) return;
  const int ob = (blockIdx.x % blocks_per_row) * kWavesPerBlock + (threadIdx.x >> 6);
  const int o0 = ob * 16 * NG;
  if (o0 >= H) return;
  const int lane = threadIdx.x & 63, r = lane & 15, q = lane >> 4;
  const size_t wrb = I / 2, srb = I / 32;
  const size_t row = active_rows[a];
  const uint8_t* wexp = w2 + row * (size_t)H * wrb;
  const uint8_t* sexp = s2 + row * (size_t)H * srb;
  const uint8_t* wrow[NG];
  const uint8_t* srow[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    wrow[g] = wexp + (o0 + 16 * g + r) * wrb;
    srow[g] = sexp + (o0 + 16 * g + r) * srb;
  }
  const int nblk = I / 32;
  const int s_beg = row_off[a], s_end = row_off[a + 1];
  const __bf16* hb = reinterpret_cast<const __bf16*>(h_ws);

  for (int t0 = s_beg; t0 < s_end; t0 += 16 * NT) {
    const int ntile = min(NT, (s_end - t0 + 15) / 16);
    int slot[NT];
    const __bf16* brow[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int idx = t0 + 16 * j + r;
      slot[j] = idx < s_end ? slots[idx] : -1;
      brow[j] = slot[j] >= 0 ? hb + (size_t)slot[j] * I : nullptr;
    }
    f32x4 acc[NT][NG];
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int g = 0; g < NG; ++g) acc[j][g] = f32x4{0.f, 0.f, 0.f, 0.f};
    mx_gemm<NT, NG>(wrow, srow, nblk, brow, ntile, q, acc);
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      if (j < ntile && slot[j] >= 0) {
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          uint32_t yb[4];
#pragma unroll
          for (int v = 0; v < 4; ++v) yb[v] = f32_to_bf16_bits(acc[j][g][v]);
          uint2 pk = make_uint2(yb[0] | (yb[1] << 16), yb[2] | (yb[3] << 16));
          *reinterpret_cast<uint2*>(Y + (size_t)slot[j] * H + o0 + 16 * g + 4 * q) = pk;
        }
      }
    }
  }
}

constexpr int kDownGroups = 2;

template <int NT>
hipError_t launch_nt(const uint8_t* w13, const uint8_t* s13, const uint8_t* w2, const uint8_t* s2,
                     int cap, const moe_split& sp, const uint16_t* x, int k, int H, int I,
                     uint16_t* h_ws, uint16_t* Y, hipStream_t stream) {
  const int gu_blocks = (I / 16 + kWavesPerBlock - 1) / kWavesPerBlock;
  hipLaunchKernelGGL(ffn_gate_up<NT>, dim3(cap * gu_blocks), dim3(64 * kWavesPerBlock), 0, stream,
                     w13, s13, sp.n_active, sp.active_rows, sp.row_off, sp.slots,
                     reinterpret_cast<const __bf16*>(x), k, H, I, gu_blocks, h_ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int rows_per_wave = 16 * kDownGroups;
  const int dn_blocks = (H / rows_per_wave + kWavesPerBlock - 1) / kWavesPerBlock;
  hipLaunchKernelGGL((ffn_down<NT, kDownGroups>), dim3(cap * dn_blocks),
                     dim3(64 * kWavesPerBlock), 0, stream, w2, s2, sp.n_active, sp.active_rows,
                     sp.row_off, sp.slots, h_ws, H, I, dn_blocks, Y);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_ffn(const uint8_t* w13, const uint8_t* s13, const uint8_t* w2,
                      const uint8_t* s2, int cap, const moe_split& split, const uint16_t* x, int T,
                      int k, int H, int I, uint16_t* h_ws, uint16_t* Y, hipStream_t stream) {
  if (T <= 16) return launch_nt<1>(w13, s13, w2, s2, cap, split, x, k, H, I, h_ws, Y, stream);
  if (T <= 32) return launch_nt<2>(w13, s13, w2, s2, cap, split, x, k, H, I, h_ws, Y, stream);
  return launch_nt<4>(w13, s13, w2, s2, cap, split, x, k, H, I, h_ws, Y, stream);
}

}  // namespace moe
