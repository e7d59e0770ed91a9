// MXFP4 operand helpers shared by the two expert-FFN kernel families (decode
// and token-tiled). Both take the reduction axis in the same 256-element
// chunks and the same lane-to-element assignment, and run the same MFMA
// sequence per output element, so a pick gives the same bits from either.
#pragma once

#include "internal.h"

namespace moe {
namespace mx {

constexpr int kChunkElems = 256;  // reduction elements per chunk per row
constexpr int kChunkBlocks = 8;   // E8M0 blocks per chunk

struct AChunk {
  uint4 lo, hi;  // 64 E2M1 codes of one row: blocks 2q and 2q+1 of the chunk
  uint16_t sc;   // their two E8M0 scale bytes (widened where used)
};

__device__ __forceinline__ float e8m0_to_f32(uint32_t b) {
  // 2^(b-127) as an fp32 bit pattern; b = 0 is the subnormal 2^-127, 255 is NaN.
  const uint32_t bits = b == 0 ? 0x00400000u : (b == 255 ? 0x7fc00000u : (b << 23));
  return __uint_as_float(bits);
}

// Chunk c of this lane's weight row. K is a multiple of 64, so the lane's two
// blocks are both in range or both past the end; past the end the lane reads
// block 0 instead (in bounds). Nothing here inspects the loaded values, so
// issuing a load never waits for it; the consumer substitutes unit scales for
// out-of-range lanes, whose activations are LDS zero padding.
__device__ __forceinline__ void load_a(AChunk& a, const uint8_t* __restrict__ wrow,
                                       const uint8_t* __restrict__ srow, int c, int q, int nblk) {
  const int b0 = c * kChunkBlocks + 2 * q;
  const int bb = b0 < nblk ? b0 : 0;
  const uint4* p = reinterpret_cast<const uint4*>(wrow + bb * 16);
  a.lo = p[0];
  a.hi = p[1];
  a.sc = *reinterpret_cast<const uint16_t*>(srow + bb);
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

// LDS activation tiles: rows of kpad elements; 16-byte granule g of row n is
// stored at granule g ^ (n & 7), so the lanes of one MFMA operand read (which
// differ in row and sit at the same column) hit different banks.
__device__ __forceinline__ int lds_elem(int n, int kpad, int elem) {
  return n * kpad + ((((elem >> 3) ^ (n & 7))) << 3);
}

// Scales of a lane's two blocks in a chunk; unit (byte 127) past the end of
// the axis (the lane then read an in-bounds block whose activations are zero).
// The byte is selected before the conversion so that no branch forms around
// the loaded value (a branch there makes the compiler wait for every load in
// flight, not just this chunk's).
__device__ __forceinline__ void chunk_scales(const AChunk& a, bool ok, float& s0, float& s1) {
  const uint32_t b = ok ? (uint32_t)a.sc : 0x7f7fu;
  s0 = e8m0_to_f32(b & 0xffu);
  s1 = e8m0_to_f32(b >> 8);
}

__device__ __forceinline__ float silu_f32(float z) { return z / (1.0f + __expf(-z)); }

}  // namespace mx
}  // namespace moe
