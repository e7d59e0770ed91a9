// Seeded synthetic MXFP4 expert weights, device twin of synth.c.
//
// Input generator only (no MoE arithmetic). It produces, byte for byte, the
// streams that synth.c defines: counter-based SplitMix64 (Steele, Lea, Flood,
// OOPSLA 2014), word i of stream K = mix(K + (i + 1) * GAMMA), little-endian
// bytes, stream key derived from (seed, layer, expert, tensor) in four mixing
// rounds, scale bytes mapped to lo + ((b * cnt) >> 8). The test suite checks
// sampled rows of a device fill against the host fill.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kGamma = 0x9e3779b97f4a7c15ULL;

__host__ __device__ inline uint64_t mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
  return z ^ (z >> 31);
}

__device__ inline uint64_t stream_key(uint64_t seed, int64_t layer, int64_t expert, int64_t t) {
  uint64_t k = mix(seed + kGamma);
  k = mix(k ^ mix(static_cast<uint64_t>(layer) + 2 * kGamma));
  k = mix(k ^ mix(static_cast<uint64_t>(expert) + 3 * kGamma));
  k = mix(k ^ mix(static_cast<uint64_t>(t) + 4 * kGamma));
  return k;
}

// grid.y = bank row, grid.x * blockDim.x threads stride over the row's 8-byte words.
__global__ void fill_tensor(uint8_t* __restrict__ dst, uint64_t row_bytes,
                            const int32_t* __restrict__ owners, uint64_t seed, int64_t layer,
                            int tensor, int lo, int cnt) {
  const uint64_t row = blockIdx.y;
  const int e = owners[row];
  uint64_t* d = reinterpret_cast<uint64_t*>(dst + row * row_bytes);
  const uint64_t words = row_bytes / 8;
  const uint64_t key = e >= 0 ? stream_key(seed, layer, e, tensor) : 0;
  for (uint64_t i = blockIdx.x * (uint64_t)blockDim.x + threadIdx.x; i < words;
       i += (uint64_t)gridDim.x * blockDim.x) {
    uint64_t v = 0;
    if (e >= 0) {
      v = mix(key + (i + 1) * kGamma);
      if (cnt > 0) {
        uint64_t m = 0;
        for (int j = 0; j < 8; ++j) {
          uint64_t b = (v >> (8 * j)) & 0xffu;
          m |= (static_cast<uint64_t>(lo) + ((b * static_cast<uint64_t>(cnt)) >> 8)) << (8 * j);
        }
        v = m;
      }
    }
    d[i] = v;
  }
}

}  // namespace

extern "C" int synth_dev_fill_bank(void* w13, void* s13, void* w2, void* s2, int n_rows,
                                   const int32_t* owners_dev, uint64_t seed, int64_t layer, int H,
                                   int I, int scale_lo, int scale_cnt, hipStream_t stream) {
  if (n_rows <= 0) return 0;
  if (n_rows > 65535 || H % 32 || I % 32) return -1;
  void* dst[4] = {w13, s13, w2, s2};
  const uint64_t sz[4] = {2ull * I * (H / 2), 2ull * I * (H / 32), 1ull * H * (I / 2),
                          1ull * H * (I / 32)};
  for (int t = 0; t < 4; ++t) {
    const uint64_t words = sz[t] / 8;
    unsigned gx = static_cast<unsigned>((words + 255) / 256);
    if (gx > 1024) gx = 1024;
    if (gx == 0) gx = 1;
    const bool scale = (t == 1 || t == 3);
    hipLaunchKernelGGL(fill_tensor, dim3(gx, n_rows), dim3(256), 0, stream,
                       static_cast<uint8_t*>(dst[t]), sz[t], owners_dev, seed, layer, t, scale_lo,
                       scale ? scale_cnt : 0);
    if (hipGetLastError() != hipSuccess) return -2;
  }
  return 0;
}
