// Expert FFN for prefill-sized steps on gfx950's block-scaled FP4 matrix
// instruction (v_mfma_scale_f32_16x16x128_f8f6f4).
//
// Same operation as the other kernel families (gate/up GEMM + SwiGLU, then the
// down GEMM into unweighted bf16 rows; "vLLM: Pin Hot Experts", section
// "Results, September 17"), for steps large enough that an expert's weights
// meet many tokens at once ("We Built the Counter", section 7: prefill wants
// bigger tiles than decode). The E2M1 weights and their E8M0 block scales go
// into the instruction as stored; nothing is dequantized in registers.
//
// The instruction multiplies two MX operands, so the bf16 activations (x for
// gate/up, h for down) are carried as two E4M3 terms with their own E8M0
// per-32 scales: hi = e4m3(v / 2^e_hi), lo = e4m3((v - hi * 2^e_hi) / 2^e_lo),
// e chosen per block so nothing saturates. A bf16 value has 8 significant bits
// and each term 4, so hi + lo carries v to within 2^-9 of its magnitude (exact
// for most values), and every product with a weight runs as two MFMAs, one per
// term, into the same fp32 accumulator.
//
// Quantized rows are stored per slot (so two banks never write the same row),
// per 256-element chunk, as 512 data bytes (hi 256, lo 256) in the order the
// instruction's B operand wants, plus 16 scale bytes:
//  - MFMA j (0, 1) of a chunk takes chunk blocks 2q + j in its K-block q
//    (lane quarter q of the A operand holds weight block 2q + j: the 16 bytes
//    the weight row stores there, with its scale byte j);
//  - B lane (c, q) holds, for MFMA j, bytes 0-15 = elements 16(q&1)..+15 of
//    chunk block 2(q>>1) + j and bytes 16-31 = the same elements of chunk
//    block 4 + 2(q>>1) + j; those 32 bytes sit at (4j + q) * 32 of a term;
//  - the B scale of K-block q is read from lane quarter q: scale dword q of a
//    chunk holds [hi(2q), hi(2q+1), lo(2q), lo(2q+1)] and the instruction's
//    byte select picks j (hi) or 2 + j (lo).
// (These operand placements were measured on the device with one-hot and
// random operands; they are what the instruction computes, not a choice.)
//
// Work items, tiles and the XCD-aware order follow ffn_tiled.hip: item =
// (tile of up to 64 slots of one expert, block of weight rows), 8 wavefronts
// each own 64 weight rows x the tile's 64 tokens. The tile's quantized
// activation chunks reach LDS by 16-byte global-to-LDS copies into two static
// buffers (no registers held across the chunk's arithmetic), each step naming
// its buffer at compile time so that the compiler need not wait for the copy
// into one buffer before reading the other; the barrier between steps waits
// for the copy only, not for the weight loads issued after it.
// The gate/up epilogue applies SwiGLU, rounds h to bf16 exactly as the other
// families do, and writes it already split into the two terms for the down
// kernel. Per output element the accumulation order (chunks in order; per
// chunk MFMA 0 hi, 0 lo, 1 hi, 1 lo) does not depend on the tile, the bank
// or the grid, so split and unsplit steps agree bit for bit; the bits differ
// from the bf16 families (which run below kFp4MinTokens), within the
// tolerance the parity tests check against the oracle.
#include <type_traits>

#include "internal.h"
#include "mxfp4_common.h"
#include "tile_items.h"

namespace moe {
namespace {

using namespace mx;
using namespace tiles;

typedef int v8i __attribute__((ext_vector_type(8)));

constexpr int kTok = 64;                 // tokens per tile
constexpr int kTokGroups = kTok / 16;    // MFMA column groups per tile
constexpr int kWaves = 8;                // wavefronts per workgroup (two per SIMD)
constexpr int kThreads = 64 * kWaves;
constexpr int kWavesPerSimd = kWaves / 4;  // register budget: 256 per wavefront
constexpr int kGroups = 4;               // 16-row MFMA groups per wavefront
constexpr int kP = 1;                    // weight chunks in flight per wavefront
// Steps per unrolled cycle: a whole number of ring turns and of the two LDS
// buffers, so each step's ring slot and buffer are compile-time constants.
constexpr int kCycle = (kP + 1) % 2 == 0 ? kP + 1 : 2 * (kP + 1);
constexpr int kQData = 512;              // quantized data bytes per row per chunk (hi, lo)
constexpr int kQScale = 16;              // quantized scale bytes per row per chunk
constexpr int kXcds = 8;
constexpr int kFmtFp4 = 4, kFmtFp8 = 0;  // the instruction's operand format codes
constexpr int kLoadsPerChunk = 3 * kGroups;  // a chunk of weights: per group 2 x 16 B + scales

// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wavefront are outstanding and all of its LDS reads have returned (the
// export counter untouched).
constexpr int vmcnt_lds_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4); }

// Workgroup barrier after an explicit wait (waitcnt immediate W), with an
// acquire fence after it so no later memory access moves above it, and
// scheduling barriers so nothing moves across the wait.
#define wg_barrier(W)                                   \
  do {                                                  \
    __builtin_amdgcn_sched_barrier(0);                  \
    __builtin_amdgcn_s_waitcnt(W);                      \
    __builtin_amdgcn_s_barrier();                       \
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup"); \
    __builtin_amdgcn_sched_barrier(0);                  \
  } while (0)
// Chunk c of this lane's weight row in group g: the group's first row at
// `gb` (wave-uniform), this lane's row at gb + lw, its scales at sb + ls.
// As load_a: past the end of the axis the lane reads block 0 (in bounds).
__device__ __forceinline__ void load_w(AChunk& a, const uint8_t* __restrict__ gb,
                                       const uint8_t* __restrict__ sb, uint32_t lw, uint32_t ls,
                                       int c, int q, int nblk) {
  const int b0 = c * kChunkBlocks + 2 * q;
  const uint32_t bb = b0 < nblk ? (uint32_t)b0 : 0u;
  const uint4* p = reinterpret_cast<const uint4*>(gb + (lw + 16u * bb));
  a.lo = p[0];
  a.hi = p[1];
  a.sc = *reinterpret_cast<const uint16_t*>(sb + (ls + bb));
}

// ---- the two-term E4M3 split ----------------------------------------------

// Smallest e with amax * 2^-e <= 448 (the largest E4M3 value), clamped to the
// E8M0 range; 0 for an all-zero block.
__device__ __forceinline__ int block_exp(float amax) {
  if (!(amax > 0.f)) return 0;
  const uint32_t u = __float_as_uint(amax);
  const int ea = (int)((u >> 23) & 0xffu) - 127;
  const int e = ea - 8 + ((u & 0x7fffffu) > 0x600000u ? 1 : 0);  // 448 = 1.75 * 2^8
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

typedef short v2s __attribute__((ext_vector_type(2)));
typedef float v2f __attribute__((ext_vector_type(2)));

// Four finite values with |v| <= 448 -> their E4M3 codes, value i in byte i,
// rounded to nearest even with the sign kept for -0: gfx950's conversion at
// scale 1. (On the device it gave the codes of a software round-to-nearest-
// even on every E4M3 value, every midpoint between neighbours and the f32
// values on either side of it, +-0, subnormal codes and 4M random values.)
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  v2s r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(v2s{0, 0}, a, b, 1.0f, false);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, c, d, 1.0f, true);
  return __builtin_bit_cast(uint32_t, r);
}
// The exact values of the E4M3 codes in bytes 2*Hi and 2*Hi + 1 of c.
template <bool Hi>
__device__ __forceinline__ v2f e4m3x2_value(uint32_t c) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(c, 1.0f, Hi);
}
// The two terms of four values v sharing a block exponent e (|v| 2^-e <= 448):
// returns the four hi codes and leaves in v what they leave over, exactly
// (v and the rounded term are close).
__device__ __forceinline__ uint32_t split_hi(float& v0, float& v1, float& v2, float& v3, int e) {
  const uint32_t c = e4m3x4(__builtin_ldexpf(v0, -e), __builtin_ldexpf(v1, -e),
                            __builtin_ldexpf(v2, -e), __builtin_ldexpf(v3, -e));
  const v2f a = e4m3x2_value<false>(c), b = e4m3x2_value<true>(c);
  v0 -= __builtin_ldexpf(a.x, e);
  v1 -= __builtin_ldexpf(a.y, e);
  v2 -= __builtin_ldexpf(b.x, e);
  v3 -= __builtin_ldexpf(b.y, e);
  return c;
}

// Byte offset, inside a chunk's 256 bytes of one term, of element w (0..31)
// of chunk block b (0..7).
__device__ __forceinline__ int term_offset(int b, int w) {
  const int j = b & 1, bb = b >> 1;
  const int q = 2 * (bb & 1) + (w >> 4);
  return (4 * j + q) * 32 + 16 * (bb >> 1) + (w & 15);
}
// Byte offsets of block b's hi and lo scale inside a chunk's 16 scale bytes.
__device__ __forceinline__ int scale_offset_hi(int b) { return 4 * (b >> 1) + (b & 1); }
__device__ __forceinline__ int scale_offset_lo(int b) { return 4 * (b >> 1) + 2 + (b & 1); }

// ---- activations -> two terms, one thread per 32-element block --------------

// x rows of the bank's slots: row s of (qd, qs) = x[slots[i] / k] for the
// slots s = slots[i] of the split. Blocks past H are written as zeros.
__global__ __launch_bounds__(256) void quant_x_slots(
    const __bf16* __restrict__ x, const int32_t* __restrict__ n_active,
    const int32_t* __restrict__ row_off, const int32_t* __restrict__ slots, int k, int H, int nch,
    uint8_t* __restrict__ qd, uint8_t* __restrict__ qs) {
  const int na = *n_active;
  const int nslots = na > 0 ? row_off[na] : 0;
  const int bpr = nch * 8;  // blocks per row
  const long long total = (long long)nslots * bpr;
  for (long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (long long)gridDim.x * blockDim.x) {
    const int i = (int)(idx / bpr), bi = (int)(idx - (long long)i * bpr);
    const int c = bi >> 3, b = bi & 7;
    const size_t sl = (uint32_t)slots[i];
    const int k0 = c * kChunkElems + 32 * b;
    float v[32];
    if (k0 < H) {
      const uint4* src = reinterpret_cast<const uint4*>(x + (sl / k) * H + k0);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const uint4 w = src[g];
        const uint32_t d[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          v[8 * g + 2 * h] = bf16_bits_to_f32(d[h] & 0xffffu);
          v[8 * g + 2 * h + 1] = bf16_bits_to_f32(d[h] >> 16);
        }
      }
    } else {
#pragma unroll
      for (int w = 0; w < 32; ++w) v[w] = 0.f;
    }
    float amax = 0.f;
#pragma unroll
    for (int w = 0; w < 32; ++w) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[w]));
    const int eh = block_exp(amax);
    uint32_t hi[8], lo[8];
#pragma unroll
    for (int d = 0; d < 8; ++d) hi[d] = split_hi(v[4 * d], v[4 * d + 1], v[4 * d + 2], v[4 * d + 3], eh);
    float ramax = 0.f;
#pragma unroll
    for (int w = 0; w < 32; ++w) ramax = __builtin_fmaxf(ramax, __builtin_fabsf(v[w]));
    const int el = block_exp(ramax);
#pragma unroll
    for (int d = 0; d < 8; ++d)
      lo[d] = e4m3x4(__builtin_ldexpf(v[4 * d], -el), __builtin_ldexpf(v[4 * d + 1], -el),
                     __builtin_ldexpf(v[4 * d + 2], -el), __builtin_ldexpf(v[4 * d + 3], -el));
    uint8_t* d = qd + (sl * nch + c) * kQData;
    // elements 0-15 and 16-31 of the block are 16 contiguous bytes each
    *reinterpret_cast<uint4*>(d + term_offset(b, 0)) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
    *reinterpret_cast<uint4*>(d + term_offset(b, 16)) = make_uint4(hi[4], hi[5], hi[6], hi[7]);
    *reinterpret_cast<uint4*>(d + 256 + term_offset(b, 0)) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
    *reinterpret_cast<uint4*>(d + 256 + term_offset(b, 16)) =
        make_uint4(lo[4], lo[5], lo[6], lo[7]);
    uint8_t* s = qs + (sl * nch + c) * kQScale;
    s[scale_offset_hi(b)] = (uint8_t)(eh + 127);
    s[scale_offset_lo(b)] = (uint8_t)(el + 127);
  }
}

// The B operand of one (token group T, MFMA J) step: both terms (8 dwords
// each) from the LDS data buffer `bd` and the scale dword from the LDS scale
// buffer `bs`. Row n = 16T + r of a buffer stores its granule G at granule
// G ^ (n & 7) (the copy's bank swizzle); n & 7 = r & 7 for every T, and lane
// (r, q)'s granules 8J + 2q + {0, 1} (hi term; lo: 16 more) keep J's bit out
// of the swizzle, so each address is a per-lane offset fixed for the kernel
// (BOff) plus a compile-time constant the LDS read carries as its immediate.
struct BOff {
  uint32_t d0, d1, s;  // granules 2q and 2q + 1 of row r; scale dword q of row r
};
__device__ __forceinline__ BOff b_offsets(int r, int q) {
  BOff o;
  o.d0 = (uint32_t)(r * kQData + 16 * ((2 * q) ^ (r & 7)));
  o.d1 = (uint32_t)(r * kQData + 16 * ((2 * q + 1) ^ (r & 7)));
  o.s = (uint32_t)(r * kQScale + 4 * q);
  return o;
}
struct BFrag {
  v8i h, l;
  int sc;
};
template <int T, int J>
__device__ __forceinline__ BFrag load_b(const unsigned char* bd, const unsigned char* bs,
                                        const BOff& o) {
  constexpr uint32_t kRow = 16u * T * kQData + 16u * 8u * J;  // token group T, granule 8J
  const uint4 h0 = *reinterpret_cast<const uint4*>(bd + (o.d0 + kRow));
  const uint4 h1 = *reinterpret_cast<const uint4*>(bd + (o.d1 + kRow));
  const uint4 l0 = *reinterpret_cast<const uint4*>(bd + (o.d0 + (kRow + 256u)));
  const uint4 l1 = *reinterpret_cast<const uint4*>(bd + (o.d1 + (kRow + 256u)));
  BFrag b;
  b.h = v8i{(int)h0.x, (int)h0.y, (int)h0.z, (int)h0.w, (int)h1.x, (int)h1.y, (int)h1.z, (int)h1.w};
  b.l = v8i{(int)l0.x, (int)l0.y, (int)l0.z, (int)l0.w, (int)l1.x, (int)l1.y, (int)l1.z, (int)l1.w};
  b.sc = *reinterpret_cast<const int*>(bs + (o.s + 16u * T * kQScale));
  return b;
}

// Steps S .. 2*NT-1 of one chunk, step S = (token group S/2, MFMA S%2): the
// hi MFMAs of the 4 row groups, then their lo MFMAs (4 independent
// accumulators between dependent ones), with the next step's B operand
// loaded from LDS meanwhile. The scheduling barrier keeps one step's
// operands in flight instead of the whole chunk's. (The instruction's byte
// selects are compile-time constants, hence the templates.)
template <int S, int NT>
__device__ __forceinline__ void chunk_steps(f32x4 (&acc)[kGroups][kTokGroups],
                                            const AChunk (&a)[kGroups], const int (&sca)[kGroups],
                                            const unsigned char* bd, const unsigned char* bs,
                                            const BOff& bo, const BFrag& cur) {
  constexpr int T = S / 2, J = S % 2;
  // the first step's operand reads stay ahead of its scheduling region
  if constexpr (S == 0) __builtin_amdgcn_sched_barrier(0);
  BFrag nxt;
  if constexpr (S + 1 < 2 * NT) nxt = load_b<(S + 1) / 2, (S + 1) % 2>(bd, bs, bo);
#pragma unroll
  for (int g = 0; g < kGroups; ++g) {
    const uint4 a4 = J ? a[g].hi : a[g].lo;
    const v8i av = {(int)a4.x, (int)a4.y, (int)a4.z, (int)a4.w, 0, 0, 0, 0};
    acc[g][T] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, cur.h, acc[g][T], kFmtFp4,
                                                                 kFmtFp8, J, sca[g], J, cur.sc);
  }
#pragma unroll
  for (int g = 0; g < kGroups; ++g) {
    const uint4 a4 = J ? a[g].hi : a[g].lo;
    const v8i av = {(int)a4.x, (int)a4.y, (int)a4.z, (int)a4.w, 0, 0, 0, 0};
    acc[g][T] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
        av, cur.l, acc[g][T], kFmtFp4, kFmtFp8, J, sca[g], 2 + J, cur.sc);
  }
  // The next step's LDS reads go out right after this step's first MFMA, so
  // the other seven cover their latency. (Left alone, the scheduler issues
  // them after most of the MFMAs, reusing the current operand's registers,
  // and the next step waits for them. The wait before the first MFMA counts
  // all LDS reads, so reads issued before it would be waited for at once.)
  if constexpr (S + 1 < 2 * NT) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    // 4 x 16 B, and the scale dword when the next step starts a token group
    __builtin_amdgcn_sched_group_barrier(0x100, S % 2 == 0 ? 4 : 5, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 2 * kGroups - 1, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (S + 1 < 2 * NT) chunk_steps<S + 1, NT>(acc, a, sca, bd, bs, bo, nxt);
}

// f(integral_constant<int, I>) for I = B .. E-1, unrolled at compile time.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// ---- the GEMM ---------------------------------------------------------------

// kGateUp: gate/up GEMM + SwiGLU (B = quantized x rows by slot, output = h
// split into two terms by slot). Otherwise: down GEMM (B = quantized h rows by
// slot, output = Y bf16 by slot).
template <bool kGateUp>
__global__ __launch_bounds__(kThreads, kWavesPerSimd) void ffn_fp4(
    const uint8_t* __restrict__ w, const uint8_t* __restrict__ s,
    const int32_t* __restrict__ n_active, const int32_t* __restrict__ active_rows,
    const int32_t* __restrict__ row_off, const int32_t* __restrict__ slots,
    const uint8_t* __restrict__ bq_d, const uint8_t* __restrict__ bq_s, int H, int I,
    int blocks_per_tile, uint8_t* __restrict__ hq_d, uint8_t* __restrict__ hq_s,
    uint16_t* __restrict__ Y) {
  // Two activation buffers as separate objects: with the ring unrolled by an
  // even count, every access names one of them statically, so the compiler
  // can tell a copy into one buffer from reads of the other and need not
  // wait for the copy before those reads.
  __shared__ __align__(16) unsigned char buf0[kTok * kQData];
  __shared__ __align__(16) unsigned char buf1[kTok * kQData];
  __shared__ __align__(16) unsigned char sbuf0[kTok * kQScale];
  __shared__ __align__(16) unsigned char sbuf1[kTok * kQScale];
  extern __shared__ __align__(16) unsigned char smem[];
  int* tpre = reinterpret_cast<int*>(smem);                          // [na + 1]
  __shared__ int wsum[kWaves];

  const int K = kGateUp ? H : I;       // reduction length
  const int ncols = kGateUp ? I : H;   // output columns per slot
  const int nblk = K / 32, nchunk = (K + kChunkElems - 1) / kChunkElems;
  const int nch_out = (I + kChunkElems - 1) / kChunkElems;  // chunks of an h row
  const size_t wrb = K / 2, srb = K / 32;
  const size_t rows_per_expert = kGateUp ? 2 * (size_t)I : (size_t)H;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int r = lane & 15, q = lane >> 4;
  const uint32_t lw = (uint32_t)r * (uint32_t)wrb, ls = (uint32_t)r * (uint32_t)srb;
  const BOff bo = b_offsets(r, q);

  const int na = *n_active;
  build_tile_prefix<kTok, kWaves>(row_off, na, tpre, wsum);
  const int items = tpre[na] * blocks_per_tile;

  // Workgroup b runs on XCD b % 8 (dispatch is round-robin over the XCDs):
  // give the workgroups of one XCD consecutive logical indices.
  const int G = gridDim.x;
  const int G8 = G - G % kXcds;
  const int b = blockIdx.x;
  const int lb = b < G8 ? (b % kXcds) * (G8 / kXcds) + b / kXcds : b;

  for (int item = lb; item < items; item += G) {
    const int a = row_of_tile(tpre, na, item / blocks_per_tile);
    const int ntl = tpre[a + 1] - tpre[a];
    const int li = item - blocks_per_tile * tpre[a];
    const int blk = li / ntl, tl = li - blk * ntl;
    const int t0 = row_off[a] + tl * kTok;
    const int nvalid = min(kTok, row_off[a + 1] - t0);
    const int ntg = (nvalid + 15) / 16;

    // Rows of this wavefront: 4 groups of 16. Gate/up: gate c0, c0+16 and up
    // I+c0, I+c0+16 for i-columns c0..c0+31 (one 32-block of h). Down: output
    // rows c0..c0+63.
    const int c0 = (blk * kWaves + wv) * (kGateUp ? 32 : 64);
    const bool busy = c0 < ncols;
    const size_t row = active_rows[a];
    const uint8_t* wexp = w + row * rows_per_expert * wrb;
    const uint8_t* sexp = s + row * rows_per_expert * srb;
    // first row of each group (wave-uniform); a lane adds r rows
    const uint8_t* wgb[kGroups];
    const uint8_t* sgb[kGroups];
#pragma unroll
    for (int g = 0; g < kGroups; ++g) {
      size_t wr;
      if (kGateUp) wr = (g < 2 ? 0 : (size_t)I) + c0 + 16 * (g & 1);
      else wr = (size_t)c0 + 16 * g;
      if (!busy) wr = 0;
      wgb[g] = wexp + wr * wrb;
      sgb[g] = sexp + wr * srb;
    }

    // Staging of one chunk of the tile's quantized rows straight into LDS
    // (16-byte global-to-LDS loads: lane L of a wavefront's load lands at
    // granule L of the wavefront's 1 KB destination, from any address). Load
    // u of wavefront w fills LDS granules p = (kWaves*u + w) * 64 + L: row
    // n = p / 32, stored granule L%32, which holds the row's granule
    // (L%32) ^ (n & 7) (the read side's bank swizzle); every wavefront also
    // copies the 64 scale granules (the same bytes to the same place). The
    // copies are unconditional, so the compiler sees each one followed by
    // exactly one chunk of weight loads: rows past the tile's last slot copy
    // its first slot (their token columns compute values that are never
    // written out: the MFMA's output columns are independent), and the chunk
    // index is clamped. Source offsets are 32-bit (a 64-bit copy of each
    // costs registers this kernel does not have): the entry points refuse
    // steps whose quantized rows reach 4 GB (ffn_fp4_fits).
    constexpr int kU = kTok * 32 / kThreads;  // copies per wavefront per chunk
    uint32_t src_row[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int n = 2 * (kWaves * u + wv) + (lane >> 5);
      const uint32_t sl = (uint32_t)slots[t0 + (n < nvalid ? n : 0)];
      src_row[u] = sl * (uint32_t)(nchunk * kQData) + 16u * (uint32_t)((lane & 31) ^ (n & 7));
    }
    const uint32_t src_sc =
        (uint32_t)slots[t0 + (lane < nvalid ? lane : 0)] * (uint32_t)(nchunk * kQScale);
    // stage(integral_constant<int, b>, c): chunk c into buffer b (named
    // statically, so each copy targets one of the two objects)
    auto stage = [&](auto bufc, int c) __attribute__((always_inline)) {
      const uint32_t cc = (uint32_t)(c < nchunk ? c : nchunk - 1);
      unsigned char* bd = decltype(bufc)::value ? buf1 : buf0;
      unsigned char* bs = decltype(bufc)::value ? sbuf1 : sbuf0;
#pragma unroll
      for (int u = 0; u < kU; ++u)
        __builtin_amdgcn_global_load_lds(bq_d + (src_row[u] + cc * kQData),
                                         bd + (kWaves * u + wv) * 64 * 16, 16, 0, 0);
      __builtin_amdgcn_global_load_lds(bq_s + (src_sc + cc * kQScale), bs, 16, 0, 0);
      // keep the copies ahead of the weight loads issued next: the waits
      // below count those loads to know the copies are done
      __builtin_amdgcn_sched_barrier(0);
    };

    f32x4 acc[kGroups][kTokGroups];
#pragma unroll
    for (int g = 0; g < kGroups; ++g)
#pragma unroll
      for (int t = 0; t < kTokGroups; ++t) acc[g][t] = f32x4{0.f, 0.f, 0.f, 0.f};

    using B0 = std::integral_constant<int, 0>;
    auto run = [&](auto ntc) __attribute__((always_inline)) {
      constexpr int NT = decltype(ntc)::value;
      AChunk ring[kP + 1][kGroups];
      stage(B0{}, 0);
#pragma unroll
      for (int p = 0; p < kP; ++p)
#pragma unroll
        for (int g = 0; g < kGroups; ++g) load_w(ring[p][g], wgb[g], sgb[g], lw, ls, p, q, nblk);
      // the copy of chunk 0 is done once at most the kP chunks of weight
      // loads issued after it are outstanding
      wg_barrier(vmcnt_lds_imm(kP * kLoadsPerChunk));
      for (int c = 0; c < nchunk; c += kCycle) {
        // step u of this cycle is chunk c + u; c is a multiple of the cycle,
        // so chunk c + u is in ring slot u % (kP + 1) and LDS buffer u & 1
        static_for<0, kCycle>([&](auto uc) __attribute__((always_inline)) {
          constexpr int u = decltype(uc)::value;
          const int cc = c + u;
          // Copies, weight loads and the wait run for every step of the cycle
          // (past the last chunk they re-read clamped, in-bounds data), so the
          // compiler counts exactly one chunk of weight loads after each copy;
          // only the arithmetic is skipped past the last chunk.
          // Chunk cc's weights (loaded kP steps ago) are waited for here,
          // before the next copies and loads are issued (the kP - 1 chunks
          // issued after them may stay in flight). Left to the compiler, the
          // wait lands at the first use of those registers, after the copy
          // just issued; a global-to-LDS copy makes it wait for every
          // outstanding load there, the next chunk's just issued included,
          // and no weight load would overlap the arithmetic.
          __builtin_amdgcn_sched_barrier(0);
          __builtin_amdgcn_s_waitcnt(vmcnt_lds_imm((kP - 1) * kLoadsPerChunk));
          __builtin_amdgcn_sched_barrier(0);
          // The buffer filled here was last read in chunk cc - 1, which every
          // wavefront finished before the last barrier.
          stage(std::integral_constant<int, (u + 1) & 1>{}, cc + 1);
#pragma unroll
          for (int g = 0; g < kGroups; ++g)
            load_w(ring[(u + kP) % (kP + 1)][g], wgb[g], sgb[g], lw, ls, cc + kP, q, nblk);
          constexpr int slot = u % (kP + 1);
          if (busy && cc < nchunk) {
            // a lane past the end of the axis has weight block 0 in its
            // registers: unit scales (the activations there are zero)
            const bool ok = cc * kChunkBlocks + 2 * q < nblk;
            int sca[kGroups];
#pragma unroll
            for (int g = 0; g < kGroups; ++g) sca[g] = ok ? (int)ring[slot][g].sc : 0x7f7f;
            const unsigned char* bd = (u & 1) ? buf1 : buf0;
            const unsigned char* bs = (u & 1) ? sbuf1 : sbuf0;
            chunk_steps<0, NT>(acc, ring[slot], sca, bd, bs, bo, load_b<0, 0>(bd, bs, bo));
          }
          // The copy of chunk cc + 1 is done once at most the one chunk of
          // weight loads issued after it is outstanding, and this buffer's
          // reads are done once the LDS counter is zero; then the barrier
          // hands both buffers over. (No release fence before it: that would
          // also wait for the weight loads, and the only LDS writes in the
          // loop are these copies, complete by the wait. The acquire fence
          // after it keeps the next step's LDS reads below it.)
          wg_barrier(vmcnt_lds_imm(kLoadsPerChunk));
        });
      }
    };

    // Every wavefront runs the same steps (copies, weight loads, waits and
    // barriers); one past the last weight row loads rows of group 0 and
    // skips the arithmetic.
    switch (ntg) {
      case 1: run(std::integral_constant<int, 1>{}); break;
      case 2: run(std::integral_constant<int, 2>{}); break;
      case 3: run(std::integral_constant<int, 3>{}); break;
      default: run(std::integral_constant<int, 4>{}); break;
    }

    // Epilogue: lane (r, q) holds rows 4q + v of each group for token 16t + r.
    if (kGateUp) {
      // h for i-columns c0..c0+31 is one 32-block of the h row: the lane's 8
      // values are elements 16*half + 4q + v; the block's magnitude comes from
      // the 4 lanes of the token. A wavefront past I but inside the last chunk
      // writes its block as zeros (the down kernel reads whole chunks).
      const int kpad_i = nch_out * kChunkElems;
      if (c0 < kpad_i) {
        const int cc = c0 / kChunkElems, bb = (c0 % kChunkElems) / 32;
#pragma unroll
        for (int t = 0; t < kTokGroups; ++t) {
          const int n = 16 * t + r;
          float hv[2][4];
#pragma unroll
          for (int half = 0; half < 2; ++half)
#pragma unroll
            for (int v = 0; v < 4; ++v)
              hv[half][v] = busy ? bf16_bits_to_f32(f32_to_bf16_bits(
                                       silu_f32(acc[half][t][v]) * acc[2 + half][t][v]))
                                 : 0.f;
          float m = 0.f;
#pragma unroll
          for (int half = 0; half < 2; ++half)
#pragma unroll
            for (int v = 0; v < 4; ++v) m = __builtin_fmaxf(m, __builtin_fabsf(hv[half][v]));
          m = __builtin_fmaxf(m, __shfl_xor(m, 16, 64));
          m = __builtin_fmaxf(m, __shfl_xor(m, 32, 64));
          const int eh = block_exp(m);
          uint32_t hw[2], lw[2];
          float rm = 0.f;
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            hw[half] = split_hi(hv[half][0], hv[half][1], hv[half][2], hv[half][3], eh);
#pragma unroll
            for (int v = 0; v < 4; ++v) rm = __builtin_fmaxf(rm, __builtin_fabsf(hv[half][v]));
          }
          rm = __builtin_fmaxf(rm, __shfl_xor(rm, 16, 64));
          rm = __builtin_fmaxf(rm, __shfl_xor(rm, 32, 64));
          const int el = block_exp(rm);
#pragma unroll
          for (int half = 0; half < 2; ++half)
            lw[half] = e4m3x4(__builtin_ldexpf(hv[half][0], -el), __builtin_ldexpf(hv[half][1], -el),
                              __builtin_ldexpf(hv[half][2], -el), __builtin_ldexpf(hv[half][3], -el));
          if (t < ntg && n < nvalid) {
            const size_t sl = (uint32_t)slots[t0 + n];
            uint8_t* d = hq_d + (sl * nch_out + cc) * kQData;
#pragma unroll
            for (int half = 0; half < 2; ++half) {
              const int off = term_offset(bb, 16 * half + 4 * q);
              *reinterpret_cast<uint32_t*>(d + off) = hw[half];
              *reinterpret_cast<uint32_t*>(d + 256 + off) = lw[half];
            }
            if (q == 0) {
              uint8_t* sp = hq_s + (sl * nch_out + cc) * kQScale;
              sp[scale_offset_hi(bb)] = (uint8_t)(eh + 127);
              sp[scale_offset_lo(bb)] = (uint8_t)(el + 127);
            }
          }
        }
      }
    } else if (busy) {
#pragma unroll
      for (int t = 0; t < kTokGroups; ++t) {
        const int n = 16 * t + r;
        if (t < ntg && n < nvalid) {
          const size_t sl = (uint32_t)slots[t0 + n];
#pragma unroll
          for (int g = 0; g < kGroups; ++g) {
            uint32_t yb[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) yb[v] = f32_to_bf16_bits(acc[g][t][v]);
            *reinterpret_cast<uint2*>(Y + sl * H + c0 + 16 * g + 4 * q) =
                make_uint2(yb[0] | (yb[1] << 16), yb[2] | (yb[3] << 16));
          }
        }
      }
    }
  }
}

// Dynamic LDS of a launch: the tile prefix (the two activation buffers are static).
size_t fp4_lds_bytes(int cap) { return ((size_t)cap + 1) * sizeof(int); }

// Workgroups for a launch (items are grid-strided): one per CU less the CUs a
// concurrent host-bank launch holds for a device bank; kHostBankCUs for a bank
// in host memory.
unsigned fp4_grid(int cap, int T, int k, int blocks, int on_host) {
  const long long max_items = ((long long)T * k / kTok + cap) * blocks;
  long long g = on_host ? kHostBankCUs : device_cus() - kHostBankCUs;
  if (g > max_items) g = max_items;
  return (unsigned)(g < 1 ? 1 : g);
}

// Workspace regions of an FP4 step (all offsets multiples of 16).
struct Fp4Ws {
  uint8_t *hq_d, *hq_s, *xq_d, *xq_s;
};
Fp4Ws fp4_ws(void* ws, int T, int k, int H, int I) {
  const size_t P = (size_t)T * k;
  const size_t nI = (I + kChunkElems - 1) / kChunkElems, nH = (H + kChunkElems - 1) / kChunkElems;
  uint8_t* p = static_cast<uint8_t*>(ws);
  Fp4Ws r;
  r.hq_d = p;
  r.hq_s = r.hq_d + P * nI * kQData;
  r.xq_d = r.hq_s + P * nI * kQScale;
  r.xq_s = r.xq_d + P * nH * kQData;
  return r;
}

}  // namespace

bool ffn_use_fp4(int T) { return T >= kFp4MinTokens; }

bool ffn_fp4_fits(int T, int k, int H, int I) {
  const uint64_t P = (uint64_t)T * k;
  const uint64_t nI = (I + kChunkElems - 1) / kChunkElems, nH = (H + kChunkElems - 1) / kChunkElems;
  return P * (nI > nH ? nI : nH) * kQData < ((uint64_t)1 << 32);
}

size_t ffn_fp4_workspace_bytes(int T, int k, int H, int I) {
  const size_t P = (size_t)T * k;
  const size_t nI = (I + kChunkElems - 1) / kChunkElems, nH = (H + kChunkElems - 1) / kChunkElems;
  return P * (nI + nH) * (kQData + kQScale);
}

hipError_t launch_gate_up_fp4(const uint8_t* w13, const uint8_t* s13, int cap, int on_host,
                              const moe_split& sp, const uint16_t* x, int T, int k, int H, int I,
                              void* ws, hipStream_t stream) {
  const Fp4Ws r = fp4_ws(ws, T, k, H, I);
  const int nH = (H + kChunkElems - 1) / kChunkElems;
  hipLaunchKernelGGL(quant_x_slots, dim3(device_cus() * 4), dim3(256), 0, stream,
                     reinterpret_cast<const __bf16*>(x), sp.n_active, sp.row_off, sp.slots, k, H,
                     nH, r.xq_d, r.xq_s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // wavefronts of 32 i-columns, up to the end of I's last chunk (the
  // wavefronts past I write that chunk's zero blocks)
  const int blocks = (I + kChunkElems - 1) / kChunkElems * (kChunkElems / 32) / kWaves;
  hipLaunchKernelGGL(ffn_fp4<true>, dim3(fp4_grid(cap, T, k, blocks, on_host)), dim3(kThreads),
                     fp4_lds_bytes(cap), stream, w13, s13, sp.n_active, sp.active_rows,
                     sp.row_off, sp.slots, r.xq_d, r.xq_s, H, I, blocks, r.hq_d, r.hq_s,
                     (uint16_t*)nullptr);
  return hipGetLastError();
}

hipError_t launch_down_fp4(const uint8_t* w2, const uint8_t* s2, int cap, int on_host,
                           const moe_split& sp, int T, int k, int H, int I, const void* ws,
                           uint16_t* Y, hipStream_t stream) {
  const Fp4Ws r = fp4_ws(const_cast<void*>(ws), T, k, H, I);
  const int blocks = (H + 64 * kWaves - 1) / (64 * kWaves);
  hipLaunchKernelGGL(ffn_fp4<false>, dim3(fp4_grid(cap, T, k, blocks, on_host)), dim3(kThreads),
                     fp4_lds_bytes(cap), stream, w2, s2, sp.n_active, sp.active_rows, sp.row_off,
                     sp.slots, r.hq_d, r.hq_s, H, I, blocks, (uint8_t*)nullptr,
                     (uint8_t*)nullptr, Y);
  return hipGetLastError();
}

}  // namespace moe
