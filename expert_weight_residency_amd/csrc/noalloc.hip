// moe_expert_ffn_mxfp4_noalloc: the expert FFN with the library's own static
// scratch buffer in place of a caller-provided workspace, for callers that
// cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid hipMalloc).
//
// The scratch is one file-scope device array. Its host-side name is only a
// stand-in for the symbol: its device address is taken once per device with
// hipGetSymbolAddress (with that device current) and only that address is
// passed to kernels. Every call on a device shares that device's array, which
// keeps the last call's contents; the FFN writes every scratch byte it later
// reads (each slot's intermediate rows), so nothing needs clearing.
#include <mutex>

#include "internal.h"

namespace moe {
namespace {

static_assert(MOE_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");
__device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices];  // device address of `scratch` per device (null: not taken yet)

// The current device's address of the scratch array (taken on the first call
// on that device); MOE_OK or an error code with the message set.
int scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return set_error(MOE_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return set_error(MOE_ENOTSUP, "device %d: at most %d devices supported", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      return set_error(MOE_EHIP, "scratch address on device %d: %s", dev, hipGetErrorString(e));
    }
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return MOE_OK;
}

}  // namespace
}  // namespace moe

extern "C" {

int moe_expert_ffn_mxfp4_noalloc(const moe_bank* bank, moe_split split, const uint16_t* x, int T,
                                 int k, int H, int I, uint16_t* Y, void* stream) {
  // the size check runs before any HIP call
  if (T > 0 && k > 0 && H > 0 && I > 0) {
    const size_t need = moe_ffn_workspace_bytes(T, k, H, I);
    if (need > (size_t)MOE_NOALLOC_SCRATCH_BYTES)
      return moe::set_error(MOE_EINVAL,
                            "T=%d, k=%d, H=%d, I=%d needs %zu bytes of scratch; the static "
                            "buffer holds %d (use moe_expert_ffn_mxfp4 with a workspace)",
                            T, k, H, I, need, MOE_NOALLOC_SCRATCH_BYTES);
  }
  void* ws = nullptr;
  if (T > 0 && bank && bank->n_rows > 0) {
    const int rc = moe::scratch_ptr(&ws);
    if (rc != MOE_OK) return rc;
  }
  // T == 0 or an empty bank: the shared body returns before using ws
  return moe::expert_ffn(bank, split, x, T, k, H, I, ws ? ws : (void*)Y, Y, stream);
}

}  // extern "C"
