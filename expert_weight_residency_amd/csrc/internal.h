// Internal declarations shared by the library's translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe_residency.h"

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// fp32 -> bf16 bits, round to nearest even; NaN keeps its sign and is quieted.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Launchers (each returns hipSuccess or the launch error). Arguments are
// validated by the ABI layer before any of these runs.
hipError_t launch_route_split(const int32_t* ids, int T, int k, const int32_t* row_map, int E,
                              int n_hot, int n_cold, int32_t* counts, int count_on,
                              const moe_split& hot, const moe_split& cold, int32_t* n_invalid,
                              hipStream_t stream);

// cap: launch capacity in active rows (min(bank rows, T*k)); on_host: the
// bank is in host memory (caps the wavefronts that read it at once).
hipError_t launch_gate_up(const uint8_t* w13, const uint8_t* s13, int cap, int on_host,
                          const moe_split& split, const uint16_t* x, int T, int k, int H, int I,
                          uint16_t* h_ws, hipStream_t stream);

hipError_t launch_down(const uint8_t* w2, const uint8_t* s2, int cap, int on_host,
                       const moe_split& split, int T, int k, int H, int I, const uint16_t* h_ws,
                       uint16_t* Y, hipStream_t stream);

// Token-tiled kernels for steps with many picks per active row (ffn_tiled.hip);
// launch_gate_up / launch_down hand over to them when ffn_use_tiled says so.
// Both families give the same bits for every pick.
hipError_t launch_gate_up_tiled(const uint8_t* w13, const uint8_t* s13, int cap, int on_host,
                                const moe_split& split, const uint16_t* x, int T, int k, int H,
                                int I, uint16_t* h_ws, hipStream_t stream);
hipError_t launch_down_tiled(const uint8_t* w2, const uint8_t* s2, int cap, int on_host,
                             const moe_split& split, int T, int k, int H, int I,
                             const uint16_t* h_ws, uint16_t* Y, hipStream_t stream);

// CUs a host-resident bank's FFN launch occupies (each of its workgroups fills
// a CU). Persistent device-bank launches leave them free, so a cold-bank launch
// running beside them never holds a device-bank workgroup back.
constexpr int kHostBankCUs = 8;

// Gate/up with every token row resident in LDS (ffn_resident.hip): 1 <= T <=
// 16, H a multiple of 1024, an 8-byte aligned scale tensor, activations and
// tables within kResidentMaxLds bytes; either bank.
constexpr size_t kResidentMaxLds = 144 * 1024;
bool ffn_use_resident(int T, int k, int H, int cap, const void* s13);
hipError_t launch_gate_up_resident(const uint8_t* w13, const uint8_t* s13, int cap, int on_host,
                                   const moe_split& split, const uint16_t* x, int T, int k, int H,
                                   int I, uint16_t* h_ws, hipStream_t stream);

// Down GEMM as a persistent streaming kernel with the workgroup's h rows in
// LDS (ffn_down_resident.hip): I a multiple of 32 whose chunk count is a
// multiple of the ring length (of the unaligned or, for a device bank with a
// 128-byte aligned weight tensor, the line-aligned loads), 16-byte aligned
// weight and scale tensors; either bank.
bool ffn_use_down_resident(int T, int k, int H, int I, const void* w2, const void* s2,
                           int on_host);
hipError_t launch_down_resident(const uint8_t* w2, const uint8_t* s2, int cap, int on_host,
                                const moe_split& split, int T, int k, int H, int I,
                                const uint16_t* h_ws, uint16_t* Y, hipStream_t stream);

// Compute units of the current device (256 if the query fails).
int device_cus();
// LDS bytes one workgroup may allocate on the current device (64 KB if the
// query fails).
size_t device_lds_per_block();

// Average picks per launchable row from which the token-tiled kernels run
// (steps of 17..255 tokens; the resident kernels take T <= 16 first). Measured
// at H = 4096, I = 2880: the hot bank (295 rows) is faster on the decode
// kernels up to 96 tokens of top-6 (1.95 picks per row) and on the tiled ones
// at 112 (2.3); the staged cold bank (89 rows) is faster tiled from 48 tokens
// (3.2), equal at 32 (2.2), slower at 20 (1.35).
constexpr int kTiledMinPicksPerRow = 2;
// Wavefronts that read a host-resident bank at once in the token-tiled kernels.
constexpr int kTiledHostWaves = 64;
bool ffn_use_tiled(int T, int k, int cap);

// Host-bank kernels for decode-sized steps (ffn_host.hip): each work item's
// weights are copied from pinned host memory into LDS in the linear pattern
// the host link streams fastest, then multiplied from there. Steps of at most
// kHostMaxTokens tokens, a bank in host memory; same bits as the other bf16
// families.
constexpr int kHostMaxTokens = 16;
bool ffn_use_gate_up_host(int T, int k, int H, int I, const void* s13);
hipError_t launch_gate_up_host(const uint8_t* w13, const uint8_t* s13, const moe_split& split,
                               int T, int k, int H, int I, const uint16_t* x, uint16_t* h_ws,
                               hipStream_t stream);
bool ffn_use_down_host(int T, int k, int H, int I, const void* s2);
hipError_t launch_down_host(const uint8_t* w2, const uint8_t* s2, const moe_split& split, int T,
                            int k, int H, int I, const uint16_t* h_ws, uint16_t* Y,
                            hipStream_t stream);

// Steps of at least kFp4MinTokens tokens (prefill) run both GEMMs on the
// block-scaled FP4 matrix instruction (ffn_fp4.hip), for every bank: the choice
// depends on the step only, so split and unsplit steps take the same path.
// Its activations travel as two E4M3 terms per bf16 value, in the workspace
// (ffn_fp4_workspace_bytes).
constexpr int kFp4MinTokens = MOE_FP4_MIN_TOKENS;
bool ffn_use_fp4(int T);
// The FP4 kernels address each quantized activation region (x or h: T*k slot
// rows of ceil(K/256) chunks of 512 data bytes) with 32-bit byte offsets;
// false when a region would reach 4 GB (T*k >= 524,288 slots at H = 4096).
bool ffn_fp4_fits(int T, int k, int H, int I);
size_t ffn_fp4_workspace_bytes(int T, int k, int H, int I);
hipError_t launch_gate_up_fp4(const uint8_t* w13, const uint8_t* s13, int cap, int on_host,
                              const moe_split& split, const uint16_t* x, int T, int k, int H,
                              int I, void* ws, hipStream_t stream);
hipError_t launch_down_fp4(const uint8_t* w2, const uint8_t* s2, int cap, int on_host,
                           const moe_split& split, int T, int k, int H, int I, const void* ws,
                           uint16_t* Y, hipStream_t stream);

// Copy split.active_rows[a] of the four src tensors to row a of dst, and
// dst_rows[a] = a, for a < *split.n_active (stage_rows.hip).
hipError_t launch_stage_rows(const uint8_t* const src[4], uint8_t* const dst[4],
                             const uint64_t row_bytes[4], const moe_split& split,
                             int32_t* dst_rows, hipStream_t stream);

hipError_t launch_finalize(const uint16_t* Y, const float* w, int T, int k, int H, uint16_t* out,
                           hipStream_t stream);

hipError_t launch_map_write(int32_t* row_map, int e_a, int v_a, int e_b, int v_b,
                            hipStream_t stream);

// The body of moe_expert_ffn_mxfp4 (argument checks, then gate/up and down
// on `stream` with `workspace` as their scratch), shared with the entry point
// that takes no workspace; and the thread-local error message setter of the
// entry points (returns `code`).
int expert_ffn(const moe_bank* bank, const moe_split& split, const uint16_t* x, int T, int k,
               int H, int I, void* workspace, uint16_t* Y, void* stream);
int set_error(int code, const char* fmt, ...);

// Longest reduction axis (H or I) the expert FFN supports (one token row must
// fit its LDS activation tile).
int ffn_max_reduction();

// Largest pick count handled by the single-kernel split (its slot placement
// compares each pick with every earlier one; above this a second kernel
// places the slots with a stable counting scatter).
constexpr int kSplitSingleMaxPicks = 512;

}  // namespace moe
