// MXFP4 operand helpers shared by the bf16 expert-FFN kernels (resident
// gate/up, persistent down, decode and token-tiled). All take the reduction
// axis in the same 256-element chunks and the same lane-to-element assignment,
// and run the same MFMA sequence per output element, so a pick gives the same
// bits from any of them. (The FP4 kernels of ffn_fp4.hip share the chunk
// constants and AChunk; their arithmetic is their own.)
#pragma once

#include "internal.h"

namespace moe {
namespace mx {

constexpr int kChunkElems = 256;  // reduction elements per chunk per row
constexpr int kChunkBlocks = 8;   // E8M0 blocks per chunk

// Weight loads over whole 128-byte lines. In the MFMA operand layout lane
// (r, q) needs bytes 32q .. 32q+31 of chunk c of row r; two 16-byte loads of
// that layout would each touch 16 rows x half a line. Instead, for one group
// of 16 rows: load A reads rows 0-7 whole (lane r < 8: bytes 32q .. +15 of
// row r, its own; lane r >= 8: bytes 32q+16 .. +31 of row r-8, its partner's)
// and load B rows 8-15 (lane r >= 8: its own first half of row r; lane r < 8:
// the second half of row r+8). Each load is then 8 full lines, which the
// memory system streams faster, also with the streaming cache policy. After
// arrival, lo_word / hi_word give the dwords of the lane's own 32 bytes: the
// first half is in A or B, the second half is in partner lane r^8's other
// load, fetched with a DPP row rotation by 8 (bank-masked: lanes 0-7 of a
// row take lane r+8's A, lanes 8-15 take lane r-8's B). The bytes each lane
// ends with are exactly those of the row-per-lane loads.
__device__ __forceinline__ uint4 ld_stream16(const void* p) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// Byte offsets, from the group's first row, of this lane's two loads.
__device__ __forceinline__ size_t line_load_a(int r, int q, size_t row_bytes) {
  return (size_t)(r & 7) * row_bytes + 32 * q + (r >= 8 ? 16 : 0);
}
__device__ __forceinline__ size_t line_load_b(int r, int q, size_t row_bytes) {
  return (size_t)(8 + (r & 7)) * row_bytes + 32 * q + (r < 8 ? 16 : 0);
}

constexpr int kDppRowRor8 = 0x128;  // DPP row_ror:8 (lane r of a row reads lane (r+8) mod 16)

__device__ __forceinline__ uint32_t lo_word(uint32_t a, uint32_t b, bool upper) {
  return upper ? b : a;
}
__device__ __forceinline__ uint32_t hi_word(uint32_t a, uint32_t b) {
  const int t = __builtin_amdgcn_update_dpp(0, (int)a, kDppRowRor8, 0xf, 0x3, false);
  return (uint32_t)__builtin_amdgcn_update_dpp(t, (int)b, kDppRowRor8, 0xf, 0xc, false);
}

struct AChunk {
  uint4 lo, hi;  // 64 E2M1 codes of one row: blocks 2q and 2q+1 of the chunk
                 // (kernels with whole-line loads keep loads A and B here; own_word
                 // turns them into these codes)
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

// Word m (0..7) of this lane's own 32 bytes of a chunk held as the two
// whole-line loads A (in lo) and B (in hi); upper: r >= 8.
__device__ __forceinline__ uint32_t own_word(const AChunk& a, int m, bool upper) {
  const uint32_t wa = word_of(a, m & 3), wb = word_of(a, 4 + (m & 3));
  return m < 4 ? lo_word(wa, wb, upper) : hi_word(wa, wb);
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
