// Ordered fp32 FMA finalize and the row-map write of a swap.
//
// Finalize: "vLLM: Pin Hot Experts", section "Results, September 17" (one
// finalize accumulates the six bf16 rows in fp32 with fma in the original k
// order and casts once) and "Update, September 17 afternoon" (this makes the
// split bit-identical to the unsplit call by construction). Each thread owns 8
// consecutive outputs of one token: a 16-byte load of each of the k rows, k
// fused multiply-adds per output starting from +0.0f, one round-to-nearest-even
// cast, one 16-byte store. The layer is tiny next to the expert FFN; the
// kernel is bound by reading Y once.
#include "internal.h"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void finalize_kernel(const uint16_t* __restrict__ Y,
                                                       const float* __restrict__ w, int T, int k,
                                                       int H, uint16_t* __restrict__ out) {
  const int per_tok = H / 8;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)T * per_tok) return;
  const int t = (int)(idx / per_tok);
  const int o = (int)(idx % per_tok) * 8;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
  for (int j = 0; j < k; ++j) {
    const float wj = w[(int64_t)t * k + j];
    const uint4 v = *reinterpret_cast<const uint4*>(Y + ((int64_t)t * k + j) * H + o);
    const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] = __builtin_fmaf(wj, bf16_bits_to_f32(d[e] & 0xffffu), acc[2 * e]);
      acc[2 * e + 1] = __builtin_fmaf(wj, bf16_bits_to_f32(d[e] >> 16), acc[2 * e + 1]);
    }
  }
  uint32_t pk[4];
#pragma unroll
  for (int e = 0; e < 4; ++e)
    pk[e] = f32_to_bf16_bits(acc[2 * e]) | (f32_to_bf16_bits(acc[2 * e + 1]) << 16);
  *reinterpret_cast<uint4*>(out + (int64_t)t * H + o) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
}

__global__ void map_write_kernel(int32_t* row_map, int e_a, int v_a, int e_b, int v_b) {
  if (threadIdx.x == 0) {
    row_map[e_a] = v_a;
    row_map[e_b] = v_b;
  }
}

}  // namespace

hipError_t launch_finalize(const uint16_t* Y, const float* w, int T, int k, int H, uint16_t* out,
                           hipStream_t stream) {
  const int64_t threads = (int64_t)T * (H / 8);
  if (threads == 0) return hipSuccess;
  hipLaunchKernelGGL(finalize_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                     stream, Y, w, T, k, H, out);
  return hipGetLastError();
}

hipError_t launch_map_write(int32_t* row_map, int e_a, int v_a, int e_b, int v_b,
                            hipStream_t stream) {
  hipLaunchKernelGGL(map_write_kernel, dim3(1), dim3(64), 0, stream, row_map, e_a, v_a, e_b, v_b);
  return hipGetLastError();
}

}  // namespace moe
