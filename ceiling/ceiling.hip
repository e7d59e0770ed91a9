// Bandwidth ceilings for the roofline denominators and counter scaling.
//
// ceiling_stream_read: reads `bytes` once with 16-byte loads (grid-stride,
// four loads in flight per thread) and folds them into one word per block so
// nothing is optimized away. On device memory it gives the achievable HBM
// read rate; on pinned host memory, the zero-copy host-link read rate the
// cold bank sees.
// ceiling_stream_read_nt: the same with nontemporal loads (the best streaming
// read rate of the device).
// ceiling_copy: a plain 16-byte copy of known size; its FETCH_SIZE and
// WRITE_SIZE counter readings calibrate the HBM-traffic counters.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__global__ __launch_bounds__(256) void stream_read(const uint4* __restrict__ src, uint64_t n16,
                                                   uint64_t* __restrict__ sink) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  uint32_t acc = 0;
  uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^
           d.z ^ d.w;
  }
  for (; i < n16; i += stride) {
    const uint4 a = src[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  __shared__ uint32_t red[256];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) red[threadIdx.x] ^= red[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0];
}

// The same read with nontemporal (streaming) 16-byte loads: whole lines per
// instruction, so the streaming policy costs no second fetch.
__global__ __launch_bounds__(256) void stream_read_nt(const uint4* __restrict__ src, uint64_t n16,
                                                      uint64_t* __restrict__ sink) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4* s = reinterpret_cast<const u32x4*>(src);
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  uint32_t acc = 0;
  uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = __builtin_nontemporal_load(s + i), b = __builtin_nontemporal_load(s + i + stride),
                c = __builtin_nontemporal_load(s + i + 2 * stride),
                d = __builtin_nontemporal_load(s + i + 3 * stride);
    acc ^= a[0] ^ a[3] ^ b[1] ^ b[2] ^ c[0] ^ c[3] ^ d[1] ^ d[2];
  }
  for (; i < n16; i += stride) {
    const u32x4 a = __builtin_nontemporal_load(s + i);
    acc ^= a[0] ^ a[3];
  }
  __shared__ uint32_t red[256];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] ^= red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0];
}

__global__ __launch_bounds__(256) void copy16(uint4* __restrict__ dst, const uint4* __restrict__ src,
                                              uint64_t n16) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
    dst[i] = src[i];
}

}  // namespace

extern "C" {

// sink: device uint64 [blocks]. Returns 0 or a HIP error code.
int ceiling_stream_read(const void* src, uint64_t bytes, uint64_t* sink, int blocks,
                        hipStream_t stream) {
  if (!src || !sink || blocks <= 0 || (bytes & 15u) || ((uintptr_t)src & 15u)) return -1;
  hipLaunchKernelGGL(stream_read, dim3(blocks), dim3(256), 0, stream,
                     static_cast<const uint4*>(src), bytes / 16, sink);
  return (int)hipGetLastError();
}

int ceiling_stream_read_nt(const void* src, uint64_t bytes, uint64_t* sink, int blocks,
                           hipStream_t stream) {
  if (!src || !sink || blocks <= 0 || (bytes & 15u) || ((uintptr_t)src & 15u)) return -1;
  hipLaunchKernelGGL(stream_read_nt, dim3(blocks), dim3(256), 0, stream,
                     static_cast<const uint4*>(src), bytes / 16, sink);
  return (int)hipGetLastError();
}

int ceiling_copy(void* dst, const void* src, uint64_t bytes, int blocks, hipStream_t stream) {
  if (!src || !dst || blocks <= 0 || (bytes & 15u) || (((uintptr_t)src | (uintptr_t)dst) & 15u))
    return -1;
  hipLaunchKernelGGL(copy16, dim3(blocks), dim3(256), 0, stream, static_cast<uint4*>(dst),
                     static_cast<const uint4*>(src), bytes / 16);
  return (int)hipGetLastError();
}

}  // extern "C"
