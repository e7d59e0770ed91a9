// Copy a bank's active rows into a compact device bank (gfx950).
//
// For a bank in host memory, the expert FFN's reads over the host link are
// rows interleaved 16 at a time (what the MFMA operand layout wants), and the
// link delivers those at ~42 GB/s, against ~55 GB/s for one contiguous
// stream. This kernel reads each active row of each tensor as one contiguous
// stream of 64 KB pieces (consecutive lanes on consecutive 16-byte granules)
// and writes it to row a of a device bank, so the FFN can
// then read HBM ("Should a GB300 Prefetch Its Cold Experts?": bringing a cold
// expert into HBM before its use instead of reading it in place).
//
// It runs on kHostBankCUs workgroups, like the in-place host-bank kernels, so
// it leaves the device-bank launches beside it their CUs.
#include "internal.h"

namespace moe {
namespace {

constexpr int kThreads = 1024;
constexpr int kUnroll = 4;                          // granules in flight per thread
constexpr uint64_t kPiece = kThreads * kUnroll;     // granules per piece (64 KB)

// The copy is cut into pieces of 64 KB (the last piece of a tensor row may be
// shorter): per active row, ceil(row bytes / 64 KB) pieces of each tensor in
// turn (none for a tensor passed with zero row bytes: not copied). Workgroup b takes pieces b, b + G, ...; in a piece each thread moves
// 4 granules, consecutive lanes on consecutive granules. (The compiler keeps
// the 4 granules in LDS and issues their loads one after another, so a
// workgroup has 16 KB in flight. Variants with all 4, or two pieces' 8, in
// flight in registers copied at the same rate beside the hot FFN and slowed
// the hot kernels a little more: the link, not the copy, sets the rate.
// 256-thread workgroups fall short.)
__global__ __launch_bounds__(kThreads) void stage_rows_kernel(
    const uint8_t* __restrict__ s0, const uint8_t* __restrict__ s1,
    const uint8_t* __restrict__ s2, const uint8_t* __restrict__ s3, uint8_t* __restrict__ d0,
    uint8_t* __restrict__ d1, uint8_t* __restrict__ d2, uint8_t* __restrict__ d3, uint64_t b0,
    uint64_t b1, uint64_t b2, uint64_t b3, const int32_t* __restrict__ n_active,
    const int32_t* __restrict__ active_rows, int32_t* __restrict__ dst_rows) {
  const int na = *n_active;
  for (int i = blockIdx.x * kThreads + threadIdx.x; i < na; i += gridDim.x * kThreads)
    dst_rows[i] = i;

  const uint8_t* const src[4] = {s0, s1, s2, s3};
  uint8_t* const dst[4] = {d0, d1, d2, d3};
  const uint64_t rb[4] = {b0, b1, b2, b3};
  uint64_t np[4], per_row = 0;  // pieces per tensor row, per active row
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    np[t] = (rb[t] / 16 + kPiece - 1) / kPiece;
    per_row += np[t];
  }
  const uint64_t total = (uint64_t)na * per_row;
  for (uint64_t p = blockIdx.x; p < total; p += gridDim.x) {
    const int a = (int)(p / per_row);
    uint64_t j = p - (uint64_t)a * per_row;
    int t = 0;
    while (j >= np[t]) j -= np[t++];
    const uint64_t row = (uint32_t)active_rows[a];
    const uint4* __restrict__ sp = reinterpret_cast<const uint4*>(src[t] + row * rb[t]);
    uint4* __restrict__ dp = reinterpret_cast<uint4*>(dst[t] + (uint64_t)a * rb[t]);
    const uint64_t g0 = j * kPiece, n = rb[t] / 16;
    uint4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint64_t i = g0 + u * kThreads + threadIdx.x;
      if (i < n) v[u] = sp[i];
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint64_t i = g0 + u * kThreads + threadIdx.x;
      if (i < n) dp[i] = v[u];
    }
  }
}

}  // namespace

hipError_t launch_stage_rows(const uint8_t* const src[4], uint8_t* const dst[4],
                             const uint64_t row_bytes[4], const moe_split& split,
                             int32_t* dst_rows, hipStream_t stream) {
  hipLaunchKernelGGL(stage_rows_kernel, dim3(kHostBankCUs), dim3(kThreads), 0, stream, src[0],
                     src[1], src[2], src[3], dst[0], dst[1], dst[2], dst[3], row_bytes[0],
                     row_bytes[1], row_bytes[2], row_bytes[3], split.n_active, split.active_rows,
                     dst_rows);
  return hipGetLastError();
}

}  // namespace moe
