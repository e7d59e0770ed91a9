// The C ABI: argument checks, then launches on the caller's stream.
// Every check runs before anything is enqueued, so an error return leaves the
// stream untouched. The library holds no state besides the thread-local error
// message.
#include <stdarg.h>
#include <stdio.h>

#include "internal.h"

namespace {

thread_local char g_err[512] = "";

int vfail(int code, const char* fmt, va_list ap) {
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  return code;
}

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vfail(code, fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return MOE_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_dims(int T, int k, int H, int I) {
  if (T < 0) return fail(MOE_EINVAL, "T=%d must be >= 0", T);
  if (k < 1 || k > MOE_MAX_TOPK) return fail(MOE_EINVAL, "k=%d outside [1, %d]", k, MOE_MAX_TOPK);
  if ((int64_t)T * k >= (int64_t)1 << 31) return fail(MOE_EINVAL, "T*k too large");
  if (H <= 0 || H % 64) return fail(MOE_EINVAL, "H=%d must be a positive multiple of 64", H);
  if (I <= 0 || I % 64) return fail(MOE_EINVAL, "I=%d must be a positive multiple of 64", I);
  if (H > moe::ffn_max_reduction() || I > moe::ffn_max_reduction())
    return fail(MOE_ENOTSUP, "H=%d, I=%d: at most %d supported", H, I, moe::ffn_max_reduction());
  if (moe::ffn_use_fp4(T) && !moe::ffn_fp4_fits(T, k, H, I))
    return fail(MOE_ENOTSUP,
                "T*k=%lld slots at H=%d, I=%d: the FP4 path addresses each activation region "
                "with 32-bit offsets; split the step into smaller chunks",
                (long long)T * k, H, I);
  return MOE_OK;
}

int check_split(const moe_split& s, const char* name) {
  if (!s.n_active || !s.active_rows || !s.row_off || !s.slots)
    return fail(MOE_EINVAL, "%s split has a NULL buffer", name);
  return MOE_OK;
}

// Device-visible addresses of a bank's tensors (pinned host memory is
// translated with hipHostGetDevicePointer).
int bank_device_ptrs(const moe_bank* b, const uint8_t* out[4]) {
  if (b->on_host != MOE_BANK_DEVICE && b->on_host != MOE_BANK_HOST &&
      b->on_host != MOE_BANK_HOST_WEIGHTS)
    return fail(MOE_EINVAL, "bank on_host=%d is not MOE_BANK_DEVICE, _HOST or _HOST_WEIGHTS",
                b->on_host);
  void* src[4] = {b->w13, b->s13, b->w2, b->s2};
  for (int i = 0; i < 4; ++i) {
    if (!src[i]) return fail(MOE_EINVAL, "bank tensor %d is NULL", i);
    // tensors 0 and 2 are the weights, 1 and 3 the scales
    const bool host = b->on_host == MOE_BANK_HOST || (b->on_host == MOE_BANK_HOST_WEIGHTS && !(i & 1));
    if (host) {
      void* d = nullptr;
      if (hipHostGetDevicePointer(&d, src[i], 0) != hipSuccess || !d) {
        (void)hipGetLastError();
        return fail(MOE_EINVAL, "bank tensor %d is not pinned host memory (on_host=%d)", i,
                    b->on_host);
      }
      out[i] = static_cast<const uint8_t*>(d);
    } else {
      out[i] = static_cast<const uint8_t*>(src[i]);
    }
  }
  if (!aligned16(out[0]) || !aligned16(out[2]))
    return fail(MOE_EINVAL, "bank weight tensors must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(out[1]) | reinterpret_cast<uintptr_t>(out[3])) & 1u)
    return fail(MOE_EINVAL, "bank scale tensors must be 2-byte aligned");
  return MOE_OK;
}

}  // namespace

namespace moe {

int set_error(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vfail(code, fmt, ap);
  va_end(ap);
  return code;
}

}  // namespace moe

extern "C" {

size_t moe_expert_bytes(int H, int I) {
  if (H <= 0 || I <= 0) return 0;
  return (size_t)2 * I * (H / 2) + (size_t)2 * I * (H / 32) + (size_t)H * (I / 2) +
         (size_t)H * (I / 32);
}

size_t moe_ffn_workspace_bytes(int T, int k, int H, int I) {
  if (T <= 0 || k <= 0 || H <= 0 || I <= 0) return 0;
  if (moe::ffn_use_fp4(T))
    return moe::ffn_fp4_fits(T, k, H, I) ? moe::ffn_fp4_workspace_bytes(T, k, H, I) : 0;
  return (size_t)T * k * I * sizeof(uint16_t);
}

const char* moe_last_error(void) { return g_err; }

int moe_route_split(const int32_t* topk_ids, int T, int k, const int32_t* row_map, int E,
                    int n_hot_rows, int n_cold_rows, int32_t* counts_layer, int count_tmax,
                    moe_split hot, moe_split cold, int32_t* n_invalid, void* stream) {
  if (T < 0) return fail(MOE_EINVAL, "T=%d must be >= 0", T);
  if (k < 1 || k > MOE_MAX_TOPK) return fail(MOE_EINVAL, "k=%d outside [1, %d]", k, MOE_MAX_TOPK);
  if ((int64_t)T * k >= (int64_t)1 << 31) return fail(MOE_EINVAL, "T*k too large");
  if (E < 1 || E > MOE_MAX_EXPERTS) return fail(MOE_EINVAL, "E=%d outside [1, %d]", E, MOE_MAX_EXPERTS);
  if (n_hot_rows < 0 || n_hot_rows > MOE_MAX_ROWS || n_cold_rows < 0 || n_cold_rows > MOE_MAX_ROWS)
    return fail(MOE_EINVAL, "bank rows (%d, %d) outside [0, %d]", n_hot_rows, n_cold_rows,
                MOE_MAX_ROWS);
  if (!row_map || !n_invalid || (T > 0 && !topk_ids))
    return fail(MOE_EINVAL, "topk_ids, row_map and n_invalid must not be NULL");
  int rc;
  if ((rc = check_split(hot, "hot")) || (rc = check_split(cold, "cold"))) return rc;
  const int count_on = counts_layer != nullptr && T <= count_tmax;
  hipError_t e = moe::launch_route_split(topk_ids, T, k, row_map, E, n_hot_rows, n_cold_rows,
                                         counts_layer, count_on, hot, cold, n_invalid,
                                         static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(MOE_EHIP, "route_split launch: %s", hipGetErrorString(e));
  return ok();
}

// Shared checks of the three FFN entry points. Returns MOE_OK with *skip set
// when there is nothing to launch.
static int ffn_prepare(const moe_bank* bank, const moe_split& split, const void* x, int T, int k,
                       int H, int I, const void* workspace, const void* Y, const uint8_t* p[4],
                       int* cap, bool* skip) {
  int rc;
  *skip = false;
  if ((rc = check_dims(T, k, H, I))) return rc;
  if (!bank) return fail(MOE_EINVAL, "bank is NULL");
  if (bank->n_rows < 0 || bank->n_rows > MOE_MAX_ROWS)
    return fail(MOE_EINVAL, "bank rows %d outside [0, %d]", bank->n_rows, MOE_MAX_ROWS);
  if (T == 0 || bank->n_rows == 0) {
    *skip = true;
    return MOE_OK;
  }
  if ((rc = check_split(split, "bank"))) return rc;
  if (!x || !workspace || !Y) return fail(MOE_EINVAL, "x, workspace and Y must not be NULL");
  if (!aligned16(x) || !aligned16(Y) || !aligned16(workspace))
    return fail(MOE_EINVAL, "x, workspace and Y must be 16-byte aligned");
  if ((rc = bank_device_ptrs(bank, p))) return rc;
  const int64_t picks = (int64_t)T * k;
  *cap = (int)(bank->n_rows < picks ? bank->n_rows : picks);
  return MOE_OK;
}

}  // extern "C"

namespace moe {

int expert_ffn(const moe_bank* bank, const moe_split& split, const uint16_t* x, int T, int k,
               int H, int I, void* workspace, uint16_t* Y, void* stream) {
  const uint8_t* p[4];
  int cap = 0, rc;
  bool skip;
  if ((rc = ffn_prepare(bank, split, x, T, k, H, I, workspace, Y, p, &cap, &skip))) return rc;
  if (skip) return ok();
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint16_t* h = static_cast<uint16_t*>(workspace);
  hipError_t e = launch_gate_up(p[0], p[1], cap, bank->on_host, split, x, T, k, H, I, h, s);
  if (e == hipSuccess) e = launch_down(p[2], p[3], cap, bank->on_host, split, T, k, H, I, h, Y, s);
  if (e != hipSuccess) return fail(MOE_EHIP, "expert FFN launch: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace moe

extern "C" {

int moe_expert_gate_up_mxfp4(const moe_bank* bank, moe_split split, const uint16_t* x, int T,
                             int k, int H, int I, void* workspace, void* stream) {
  const uint8_t* p[4];
  int cap = 0, rc;
  bool skip;
  // Y is not touched by this stage; pass x to satisfy the shared check
  if ((rc = ffn_prepare(bank, split, x, T, k, H, I, workspace, x, p, &cap, &skip))) return rc;
  if (skip) return ok();
  hipError_t e = moe::launch_gate_up(p[0], p[1], cap, bank->on_host, split, x, T, k, H, I,
                                     static_cast<uint16_t*>(workspace),
                                     static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(MOE_EHIP, "gate/up launch: %s", hipGetErrorString(e));
  return ok();
}

int moe_expert_down_mxfp4(const moe_bank* bank, moe_split split, int T, int k, int H, int I,
                          const void* workspace, uint16_t* Y, void* stream) {
  const uint8_t* p[4];
  int cap = 0, rc;
  bool skip;
  // x is not read by this stage; pass the workspace to satisfy the shared check
  if ((rc = ffn_prepare(bank, split, workspace, T, k, H, I, workspace, Y, p, &cap, &skip)))
    return rc;
  if (skip) return ok();
  hipError_t e = moe::launch_down(p[2], p[3], cap, bank->on_host, split, T, k, H, I,
                                  static_cast<const uint16_t*>(workspace), Y,
                                  static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(MOE_EHIP, "down launch: %s", hipGetErrorString(e));
  return ok();
}

int moe_expert_ffn_mxfp4(const moe_bank* bank, moe_split split, const uint16_t* x, int T, int k,
                         int H, int I, void* workspace, uint16_t* Y, void* stream) {
  return moe::expert_ffn(bank, split, x, T, k, H, I, workspace, Y, stream);
}

int moe_stage_rows(const moe_bank* src, moe_split split, int T, int k, const moe_bank* dst,
                   int32_t* dst_rows, int H, int I, int parts, void* stream) {
  int rc;
  if (parts < MOE_STAGE_GATE_UP || parts > MOE_STAGE_ALL)
    return fail(MOE_EINVAL, "parts=%d must be 1 (gate/up), 2 (down) or 3 (both)", parts);
  if (T < 0) return fail(MOE_EINVAL, "T=%d must be >= 0", T);
  if (k < 1 || k > MOE_MAX_TOPK) return fail(MOE_EINVAL, "k=%d outside [1, %d]", k, MOE_MAX_TOPK);
  if ((int64_t)T * k >= (int64_t)1 << 31) return fail(MOE_EINVAL, "T*k too large");
  if (H <= 0 || H % 64 || I <= 0 || I % 64) return fail(MOE_EINVAL, "H, I must be multiples of 64");
  if (!src || !dst) return fail(MOE_EINVAL, "src and dst must not be NULL");
  if (src->n_rows < 0 || src->n_rows > MOE_MAX_ROWS)
    return fail(MOE_EINVAL, "src rows %d outside [0, %d]", src->n_rows, MOE_MAX_ROWS);
  if (T == 0 || src->n_rows == 0) return ok();
  if ((rc = check_split(split, "src"))) return rc;
  if (!dst_rows) return fail(MOE_EINVAL, "dst_rows must not be NULL");
  if (dst->on_host) return fail(MOE_EINVAL, "dst must be a device bank (on_host = 0)");
  const int64_t picks = (int64_t)T * k;
  const int cap = (int)(src->n_rows < picks ? src->n_rows : picks);
  if (dst->n_rows < cap)
    return fail(MOE_EINVAL, "dst holds %d rows, the split can name %d", dst->n_rows, cap);
  const uint8_t* sp[4];
  const uint8_t* dq[4];
  if ((rc = bank_device_ptrs(src, sp)) || (rc = bank_device_ptrs(dst, dq))) return rc;
  // row bytes of each tensor; zero for a tensor this call does not copy
  const bool gu = parts & MOE_STAGE_GATE_UP, dn = parts & MOE_STAGE_DOWN;
  const uint64_t rb[4] = {gu ? (uint64_t)2 * I * (H / 2) : 0, gu ? (uint64_t)2 * I * (H / 32) : 0,
                          dn ? (uint64_t)H * (I / 2) : 0, dn ? (uint64_t)H * (I / 32) : 0};
  for (int t = 0; t < 4; ++t)
    if (rb[t] && ((reinterpret_cast<uintptr_t>(sp[t]) | reinterpret_cast<uintptr_t>(dq[t])) & 15u))
      return fail(MOE_EINVAL, "bank tensor %d must be 16-byte aligned for staging", t);
  uint8_t* dp[4] = {const_cast<uint8_t*>(dq[0]), const_cast<uint8_t*>(dq[1]),
                    const_cast<uint8_t*>(dq[2]), const_cast<uint8_t*>(dq[3])};
  hipError_t e = moe::launch_stage_rows(sp, dp, rb, split, dst_rows,
                                        static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(MOE_EHIP, "stage rows launch: %s", hipGetErrorString(e));
  return ok();
}

int moe_stage_rows_dma(const moe_bank* src, const int32_t* rows, int n, const moe_bank* dst,
                       int H, int I, int parts, void* stream) {
  int rc;
  if (parts < MOE_STAGE_GATE_UP || parts > MOE_STAGE_ALL)
    return fail(MOE_EINVAL, "parts=%d must be 1 (gate/up), 2 (down) or 3 (both)", parts);
  if (n < 0) return fail(MOE_EINVAL, "n=%d must be >= 0", n);
  if (H <= 0 || H % 64 || I <= 0 || I % 64) return fail(MOE_EINVAL, "H, I must be multiples of 64");
  if (!src || !dst) return fail(MOE_EINVAL, "src and dst must not be NULL");
  if (src->n_rows < 0 || src->n_rows > MOE_MAX_ROWS)
    return fail(MOE_EINVAL, "src rows %d outside [0, %d]", src->n_rows, MOE_MAX_ROWS);
  if (n == 0) return ok();
  if (!rows) return fail(MOE_EINVAL, "rows must not be NULL");
  if (dst->on_host) return fail(MOE_EINVAL, "dst must be a device bank (on_host = 0)");
  if (dst->n_rows < n) return fail(MOE_EINVAL, "dst holds %d rows, %d are named", dst->n_rows, n);
  for (int a = 0; a < n; ++a)
    if (rows[a] < 0 || rows[a] >= src->n_rows)
      return fail(MOE_EINVAL, "rows[%d]=%d outside [0, %d)", a, rows[a], src->n_rows);
  const uint8_t* sp[4];
  const uint8_t* dq[4];
  if ((rc = bank_device_ptrs(src, sp)) || (rc = bank_device_ptrs(dst, dq))) return rc;
  const uint8_t* const sh[4] = {static_cast<const uint8_t*>(src->w13),
                                static_cast<const uint8_t*>(src->s13),
                                static_cast<const uint8_t*>(src->w2),
                                static_cast<const uint8_t*>(src->s2)};
  const bool gu = parts & MOE_STAGE_GATE_UP, dn = parts & MOE_STAGE_DOWN;
  const uint64_t rb[4] = {gu ? (uint64_t)2 * I * (H / 2) : 0, gu ? (uint64_t)2 * I * (H / 32) : 0,
                          dn ? (uint64_t)H * (I / 2) : 0, dn ? (uint64_t)H * (I / 32) : 0};
  const hipMemcpyKind kind = hipMemcpyDefault;  // the tensors of a bank may sit on either side
  hipStream_t st = static_cast<hipStream_t>(stream);
  // one copy per run of consecutive source rows (they land on consecutive
  // destination rows), per tensor
  for (int a = 0; a < n;) {
    int b = a + 1;
    while (b < n && rows[b] == rows[b - 1] + 1) ++b;
    for (int t = 0; t < 4; ++t) {
      if (!rb[t]) continue;
      const hipError_t e =
          hipMemcpyAsync(const_cast<uint8_t*>(dq[t]) + (uint64_t)a * rb[t],
                         sh[t] + (uint64_t)rows[a] * rb[t], (uint64_t)(b - a) * rb[t], kind, st);
      if (e != hipSuccess) return fail(MOE_EHIP, "stage rows copy: %s", hipGetErrorString(e));
    }
    a = b;
  }
  return ok();
}

int moe_finalize(const uint16_t* Y, const float* topk_w, int T, int k, int H, uint16_t* out,
                 void* stream) {
  if (T < 0) return fail(MOE_EINVAL, "T=%d must be >= 0", T);
  if (k < 1 || k > MOE_MAX_TOPK) return fail(MOE_EINVAL, "k=%d outside [1, %d]", k, MOE_MAX_TOPK);
  if (H <= 0 || H % 8) return fail(MOE_EINVAL, "H=%d must be a positive multiple of 8", H);
  if (T == 0) return ok();
  if (!Y || !topk_w || !out) return fail(MOE_EINVAL, "Y, topk_w and out must not be NULL");
  if (!aligned16(Y) || !aligned16(out)) return fail(MOE_EINVAL, "Y and out must be 16-byte aligned");
  hipError_t e = moe::launch_finalize(Y, topk_w, T, k, H, out, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(MOE_EHIP, "finalize launch: %s", hipGetErrorString(e));
  return ok();
}

int moe_usage_counts(const int32_t* counts, int L, int E, int32_t* host_dst, void* stream) {
  if (L < 1 || E < 1 || E > MOE_MAX_EXPERTS) return fail(MOE_EINVAL, "bad table shape %d x %d", L, E);
  if (!counts || !host_dst) return fail(MOE_EINVAL, "counts and host_dst must not be NULL");
  hipError_t e = hipMemcpyAsync(host_dst, counts, (size_t)L * E * sizeof(int32_t),
                                hipMemcpyDeviceToHost, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(MOE_EHIP, "counter snapshot copy: %s", hipGetErrorString(e));
  return ok();
}

int moe_swap_rows(const moe_bank* hot, const moe_bank* cold, int hot_row, int cold_row,
                  int expect_hot_expert, int expect_cold_expert, int32_t* row_map, int E,
                  int32_t* hot_owner, int32_t* cold_owner, void* staging, size_t staging_bytes,
                  int H, int I, void* stream) {
  if (!hot || !cold || !row_map || !hot_owner || !cold_owner || !staging)
    return fail(MOE_EINVAL, "NULL argument");
  if (H <= 0 || H % 64 || I <= 0 || I % 64) return fail(MOE_EINVAL, "H, I must be multiples of 64");
  if (E < 1 || E > MOE_MAX_EXPERTS) return fail(MOE_EINVAL, "E=%d outside [1, %d]", E, MOE_MAX_EXPERTS);
  for (const moe_bank* b : {hot, cold})
    if (b->on_host != MOE_BANK_DEVICE && b->on_host != MOE_BANK_HOST &&
        b->on_host != MOE_BANK_HOST_WEIGHTS)
      return fail(MOE_EINVAL, "bank on_host=%d is not MOE_BANK_DEVICE, _HOST or _HOST_WEIGHTS",
                  b->on_host);
  if (hot_row < 0 || hot_row >= hot->n_rows || cold_row < 0 || cold_row >= cold->n_rows)
    return fail(MOE_EINVAL, "rows (%d, %d) outside banks (%d, %d)", hot_row, cold_row,
                hot->n_rows, cold->n_rows);
  if (expect_hot_expert < 0 || expect_hot_expert >= E || expect_cold_expert < 0 ||
      expect_cold_expert >= E || expect_hot_expert == expect_cold_expert)
    return fail(MOE_EINVAL, "expected experts (%d, %d) invalid for E=%d", expect_hot_expert,
                expect_cold_expert, E);
  const size_t sz[4] = {(size_t)2 * I * (H / 2), (size_t)2 * I * (H / 32), (size_t)H * (I / 2),
                        (size_t)H * (I / 32)};
  if (staging_bytes < sz[0] + sz[1] + sz[2] + sz[3])
    return fail(MOE_EINVAL, "staging holds %zu bytes, one expert needs %zu", staging_bytes,
                sz[0] + sz[1] + sz[2] + sz[3]);
  void* hp[4] = {hot->w13, hot->s13, hot->w2, hot->s2};
  void* cp[4] = {cold->w13, cold->s13, cold->w2, cold->s2};
  for (int t = 0; t < 4; ++t)
    if (!hp[t] || !cp[t]) return fail(MOE_EINVAL, "bank tensor %d is NULL", t);
  if (hot_owner[hot_row] != expect_hot_expert || cold_owner[cold_row] != expect_cold_expert)
    return fail(MOE_ESTALE,
                "stale swap: hot row %d holds %d (decided on %d), cold row %d holds %d (decided on %d)",
                hot_row, hot_owner[hot_row], expect_hot_expert, cold_row, cold_owner[cold_row],
                expect_cold_expert);
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* stage = static_cast<uint8_t*>(staging);
  for (int t = 0; t < 4; ++t) {
    uint8_t* h = static_cast<uint8_t*>(hp[t]) + (size_t)hot_row * sz[t];
    uint8_t* c = static_cast<uint8_t*>(cp[t]) + (size_t)cold_row * sz[t];
    hipError_t e;
    if ((e = hipMemcpyAsync(stage, h, sz[t], hipMemcpyDefault, s)) != hipSuccess ||
        (e = hipMemcpyAsync(h, c, sz[t], hipMemcpyDefault, s)) != hipSuccess ||
        (e = hipMemcpyAsync(c, stage, sz[t], hipMemcpyDefault, s)) != hipSuccess)
      return fail(MOE_EHIP, "swap copy (tensor %d): %s", t, hipGetErrorString(e));
    stage += sz[t];
  }
  hipError_t e = moe::launch_map_write(row_map, expect_hot_expert, -1 - cold_row,
                                       expect_cold_expert, hot_row, s);
  if (e != hipSuccess) return fail(MOE_EHIP, "map write launch: %s", hipGetErrorString(e));
  hot_owner[hot_row] = expect_cold_expert;
  cold_owner[cold_row] = expect_hot_expert;
  return ok();
}

}  // extern "C"
