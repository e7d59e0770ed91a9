/*
 * moe_residency.h -- C ABI of the hot/cold expert-residency MoE layer (gfx950).
 *
 * One routed mixture-of-experts layer whose experts live in two banks: a hot
 * bank in HBM and a cold bank in pinned host memory that the GPU reads in
 * place. A residency split resolves each token's top-k expert ids through a
 * per-layer row map, each bank runs the MXFP4 expert FFN on its own picks,
 * and an ordered fp32 FMA finalize combines the k unweighted rows per token,
 * so the split result is bit-identical to running every expert from one bank.
 * A usage counter fused into the split feeds a between-step row swap.
 *
 * Conventions for every entry point:
 *  - All pointers are caller-owned. "device" means device memory or any
 *    device-accessible memory; "host" means ordinary host memory. The library
 *    allocates nothing and keeps no state between calls.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream). All GPU
 *    work is enqueued on it in call order; nothing synchronizes the host, so
 *    device faults surface at the caller's next synchronization. The split,
 *    FFN and finalize calls issue only kernel launches and may be captured in
 *    a HIP graph.
 *  - Return value: MOE_OK (0) or a negative MOE_E* code. On error nothing has
 *    been enqueued and moe_last_error() holds a message (thread-local).
 *  - Sizes are element counts unless they say bytes.
 *
 * Data layout (the ABI layout; the kernels read it as is):
 *  - MXFP4 weights: E2M1 codes, two per byte, the LOW nibble holding the even
 *    element; one E8M0 scale byte per 32 consecutive elements along the
 *    reduction axis (OCP MX). The pages name the format and require that the
 *    scale tensors mirror the weight partition ("vLLM: Pin Hot Experts",
 *    sections "Where the experts live today" and "The one open door").
 *  - A bank of R rows holds four row-major tensors, row r = one expert:
 *      w13 u8 [R][2I][H/2]   rows [0,I) gate, rows [I,2I) up
 *      s13 u8 [R][2I][H/32]
 *      w2  u8 [R][H][I/2]
 *      s2  u8 [R][H][I/32]
 *    One expert at H=4096, I=2880 is 18,800,640 bytes.
 *  - Row map int32 [E] (device): m >= 0 means hot row m, m < 0 means cold row
 *    -1-m ("vLLM: Pin Hot Experts", section "The one open door": an int32[384]
 *    device tensor per layer resolving an id to which tensor and which row).
 *  - Slot s = t*k + j indexes pick j of token t. Y is bf16 [T*k][H], one
 *    unweighted expert row per slot.
 *
 * Shape limits: 1 <= E <= MOE_MAX_EXPERTS; bank rows <= MOE_MAX_ROWS; H and I
 * positive multiples of 64, at most 32768; 1 <= k <= MOE_MAX_TOPK; T >= 0 and
 * T*k < 2^31. Steps of MOE_FP4_MIN_TOKENS tokens or more also need
 * T*k * ceil(max(H, I)/256) * 512 < 2^32 (T*k < 524,288 at H = 4096); larger
 * ones are refused with MOE_ENOTSUP (split them into chunks).
 * Pointers to weights, activations and Y rows must be 16-byte aligned.
 */
#ifndef MOE_RESIDENCY_H
#define MOE_RESIDENCY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_OK 0
#define MOE_EINVAL (-1)  /* bad argument: shape, alignment, NULL, limit */
#define MOE_EHIP (-2)    /* a HIP launch or copy reported an error */
#define MOE_ESTALE (-3)  /* swap refused: owners changed since the decision */
#define MOE_ENOTSUP (-4) /* configuration the library does not implement */

#define MOE_MAX_EXPERTS 4096
#define MOE_MAX_ROWS 4096
#define MOE_MAX_TOPK 32
/* Steps of at least this many tokens (prefill) run the expert FFN on the
 * block-scaled FP4 matrix instruction; see moe_expert_ffn_mxfp4. */
#define MOE_FP4_MIN_TOKENS 256

/* One residency bank. The four pointers are device-accessible: device memory
 * for the hot bank; for the cold bank, pinned host memory (hipHostMalloc or
 * torch pin_memory) with on_host = MOE_BANK_HOST, which the kernels read in
 * place over the host link ("We Built the Counter", section 1: cold experts
 * sit in host memory and are read in place whenever the router picks one). A
 * cold bank may also live in device memory (MOE_BANK_DEVICE), or keep its
 * weight tensors w13, w2 in pinned host memory and its scale tensors s13, s2
 * (1/16 of the weight bytes) in device memory (MOE_BANK_HOST_WEIGHTS: only
 * the weights cross the link); results are identical in every case. Any other
 * on_host value is refused with MOE_EINVAL. */
#define MOE_BANK_DEVICE 0
#define MOE_BANK_HOST 1
#define MOE_BANK_HOST_WEIGHTS 2
typedef struct moe_bank {
    void *w13;
    void *s13;
    void *w2;
    void *s2;
    int32_t n_rows;
    int32_t on_host;
} moe_bank;

/* Split output for one bank, all device int32 buffers written by
 * moe_route_split and read by moe_expert_ffn_mxfp4. With cap = min(n_rows,
 * T*k): n_active [1]; active_rows [cap] (bank rows in ascending order);
 * row_off [cap+1] (CSR offsets into slots, row_off[0] = 0); slots [T*k]
 * (slot ids, ascending within each row). Entries past n_active (or past
 * row_off[n_active] in slots) are left unwritten. */
typedef struct moe_split {
    int32_t *n_active;
    int32_t *active_rows;
    int32_t *row_off;
    int32_t *slots;
} moe_split;

/* Bytes of one expert row (all four tensors) at hidden H, intermediate I. */
size_t moe_expert_bytes(int H, int I);

/* Bytes of the device workspace moe_expert_ffn_mxfp4 needs at step size T:
 * below MOE_FP4_MIN_TOKENS tokens, the bf16 SwiGLU output h [T*k][I]; from
 * MOE_FP4_MIN_TOKENS on, x and h per slot as the two E4M3 terms the FP4 path
 * reads ((T*k) * (ceil(H/256) + ceil(I/256)) * 528 bytes). Both bank calls of
 * one layer may share one workspace: each writes only its own slots. 0 when
 * any argument is <= 0, and for a step the FFN refuses with MOE_ENOTSUP (see
 * the shape limits above). */
size_t moe_ffn_workspace_bytes(int T, int k, int H, int I);

/*
 * moe_route_split -- residency split with deterministic compaction and the
 * fused usage counter.
 *
 * For every pick s = t*k + j with id = topk_ids[s] in [0, E): m = row_map[id];
 * m >= 0 routes the pick to hot row m, m < 0 to cold row -1-m. Picks whose id
 * is outside [0, E) or whose row is outside its bank are routed to neither
 * bank and counted in *n_invalid (the output of that token is then undefined:
 * a caller error). Each bank's output lists its active rows in ascending row
 * order and, per row, its slots in ascending s, so the result is unique.
 * ("vLLM: Pin Hot Experts", section "Results, September 17": split each token's
 * ids by residency; "We Built the Counter", section 2: the split kernel.)
 *
 * Counter: if counts_layer != NULL and T <= count_tmax, counts_layer[id] += 1
 * for every pick with id in [0, E), with relaxed device-scope atomics, inside
 * the same kernel ("We Built the Counter", section 2: one masked atomic add per
 * routed pick into a fixed layers x experts table, relaxed semantics, only
 * steps of at most 256 tokens). counts_layer is one layer's row [E] of a
 * caller-owned int32 [L][E] table; it is never reset here (int32 wraps;
 * readers diff snapshots modulo 2^32).
 *
 * topk_ids: device int32 [T][k]. row_map: device int32 [E]. n_hot_rows /
 * n_cold_rows: bank sizes (either may be 0; its split must then still be
 * valid buffers of capacity 0 plus n_active and row_off[1]). n_invalid:
 * device int32 [1]. Launches one kernel when T*k <= 512, two otherwise.
 */
int moe_route_split(const int32_t *topk_ids, int T, int k, const int32_t *row_map, int E,
                    int n_hot_rows, int n_cold_rows, int32_t *counts_layer, int count_tmax,
                    moe_split hot, moe_split cold, int32_t *n_invalid, void *stream);

/*
 * moe_expert_ffn_mxfp4 -- the expert FFN over one bank's picks.
 *
 * For each active row r of `split` and each slot s of that row, with token
 * t = s / k: g = Wgate[r] . x[t], u = Wup[r] . x[t] (E2M1 x E8M0 dequantized,
 * fp32 accumulation), h = silu(g) * u, y = Wdown[r] . h, and Y[s] = bf16(y)
 * rounded to nearest even. Rows are unweighted: the router weight is applied
 * only by moe_finalize ("vLLM: Pin Hot Experts", section "Results, September
 * 17": the routed MXFP4 MoE called once per bank with finalization deferred,
 * leaving six bf16 rows per token). Only this bank's slots of Y are written.
 *
 * The per-(row, slot) arithmetic, including its reduction order, does not
 * depend on the bank, the row index, the other slots or the grid, so a pick
 * gives the same bits from either bank. It depends on the step size only:
 * below MOE_FP4_MIN_TOKENS tokens the weights are dequantized to bf16 for bf16
 * matrix products (every E2M1 value times an E8M0 scale of byte 0 .. 252 is a
 * bf16 value, subnormals included, so the dequantization is exact there; those
 * bytes are tested against the CPU oracle); from MOE_FP4_MIN_TOKENS on
 * (prefill) the E2M1
 * weights and their scales go to the block-scaled FP4 matrix instruction as
 * stored, with each bf16 activation (x, and h after its bf16 rounding) carried
 * as two E4M3 terms with E8M0 per-32 scales, which hold it to within 2^-9 of
 * its magnitude ("vLLM: Pin Hot Experts": the MXFP4 expert GEMM; the FP4
 * instruction where the token count makes the GEMM a dense contraction).
 *
 * bank: see moe_bank. split: this bank's moe_route_split output (device).
 * x: device bf16 [T][H]. workspace: device, moe_ffn_workspace_bytes(T,k,H,I)
 * bytes. Y: device bf16 [T*k][H]. Below MOE_FP4_MIN_TOKENS tokens launches two
 * kernels (gate/up + SwiGLU, then down); from MOE_FP4_MIN_TOKENS on, three
 * (the activations' two-term split, gate/up + SwiGLU, down). Launches nothing
 * when T == 0 or the bank has no rows. MOE_ENOTSUP for a prefill step past the
 * FP4 path's offset limit (see the shape limits above).
 */
int moe_expert_ffn_mxfp4(const moe_bank *bank, moe_split split, const uint16_t *x, int T, int k,
                         int H, int I, void *workspace, uint16_t *Y, void *stream);

/* Bytes of the static device scratch buffer moe_expert_ffn_mxfp4_noalloc
 * uses in place of a workspace (32 MiB per device). */
#define MOE_NOALLOC_SCRATCH_BYTES (32 << 20)

/*
 * moe_expert_ffn_mxfp4_noalloc -- moe_expert_ffn_mxfp4 for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).
 *
 * The same operation, kernels and bits as moe_expert_ffn_mxfp4 with the same
 * arguments, but the intermediate rows live in one static device buffer of
 * MOE_NOALLOC_SCRATCH_BYTES per device, owned by the library and held until
 * the process ends, instead of a workspace argument. Steps whose
 * moe_ffn_workspace_bytes(T, k, H, I) exceeds that size are refused with
 * MOE_EINVAL before anything is enqueued (at H = 4096, I = 2880, top-6: every
 * step below MOE_FP4_MIN_TOKENS tokens, and prefill steps up to 378 tokens).
 * The buffer's device address is taken on the first call on each device
 * (hipGetSymbolAddress, no allocation). Every call on one device shares that
 * device's buffer: calls that overlap on one GPU race, except the two bank
 * calls of one step (the same T, k, H and I), which write disjoint slots of it.
 * Nothing in the buffer needs clearing between calls.
 */
int moe_expert_ffn_mxfp4_noalloc(const moe_bank *bank, moe_split split, const uint16_t *x, int T,
                                 int k, int H, int I, uint16_t *Y, void *stream);

/*
 * moe_expert_gate_up_mxfp4 / moe_expert_down_mxfp4 -- the two launches of
 * moe_expert_ffn_mxfp4, callable one at a time (for timing each kernel, or to
 * schedule them separately). gate_up writes h = silu(g) * u as bf16 into the
 * workspace for this bank's slots; down reads it and writes this bank's rows
 * of Y. moe_expert_ffn_mxfp4 is exactly gate_up followed by down, and the two
 * paths give identical bits. Arguments as for moe_expert_ffn_mxfp4.
 */
int moe_expert_gate_up_mxfp4(const moe_bank *bank, moe_split split, const uint16_t *x, int T,
                             int k, int H, int I, void *workspace, void *stream);
int moe_expert_down_mxfp4(const moe_bank *bank, moe_split split, int T, int k, int H, int I,
                          const void *workspace, uint16_t *Y, void *stream);

/* moe_stage_rows parts: the gate/up tensors (w13, s13), the down tensors (w2, s2). */
#define MOE_STAGE_GATE_UP 1
#define MOE_STAGE_DOWN 2
#define MOE_STAGE_ALL 3

/*
 * moe_stage_rows -- copy one bank's active rows into a compact device bank.
 *
 * For a = 0 .. n_active-1 (n_active = *split.n_active on the device): row
 * split.active_rows[a] of each tensor of `src` that `parts` names is copied to
 * row a of the same tensor of `dst`, and dst_rows[a] = a. The split {split.n_active, dst_rows,
 * split.row_off, split.slots} then drives moe_expert_ffn_mxfp4 on `dst` with
 * results identical to `split` on `src` (the FFN arithmetic does not depend on
 * the bank). For a cold bank in pinned host memory this replaces the FFN's
 * row-interleaved reads over the host link with one contiguous stream per
 * touched expert, copied into HBM before use ("Should a GB300 Prefetch Its
 * Cold Experts?": bring a cold expert into HBM instead of reading it in place;
 * "We Built the Counter", section 6: cold reads in place as the baseline).
 *
 * src: the bank the split was made for (host or device). split: its
 * moe_route_split output for a step of T tokens, k picks each. dst: a device
 * bank (on_host = 0) with n_rows >= min(src->n_rows, T*k); rows past n_active
 * are left unwritten. dst_rows: device int32 [min(src->n_rows, T*k)]. parts:
 * MOE_STAGE_GATE_UP, MOE_STAGE_DOWN or both (MOE_STAGE_ALL); the tensors it
 * names 16-byte aligned. Staging the two parts in two calls lets the gate/up
 * GEMM on dst start while the down tensors are still being copied. Launches
 * one kernel; nothing when T == 0 or src has no rows. MOE_EINVAL for a parts
 * value outside 1..3, before any work is enqueued.
 */
int moe_stage_rows(const moe_bank *src, moe_split split, int T, int k, const moe_bank *dst,
                   int32_t *dst_rows, int H, int I, int parts, void *stream);

/*
 * moe_stage_rows_dma -- the copy of moe_stage_rows by the DMA engines, for a
 * row list the host holds ("Should a GB300 Prefetch Its Cold Experts?": copy
 * a cold expert into HBM on a miss instead of reading it in place).
 *
 * For a = 0 .. n-1: row rows[a] of each tensor of `src` that `parts` names is
 * copied to row a of the same tensor of `dst` with hipMemcpyAsync on `stream`
 * (one copy per run of consecutive rows per tensor); no compute unit takes
 * part. With rows = the split's active rows (read back to the host after
 * moe_route_split) and a device row list 0 .. n-1 in place of
 * split.active_rows, moe_expert_ffn_mxfp4 on `dst` gives the same results as
 * on `src`.
 *
 * src: host or device bank. rows: host int32 [n], each in [0, src->n_rows).
 * dst: a device bank with n_rows >= n. parts as for moe_stage_rows. Every
 * argument is checked before any copy is enqueued (MOE_EINVAL); MOE_EHIP if
 * the runtime refuses a copy (copies enqueued before it stay enqueued).
 * Nothing is enqueued when n == 0.
 */
int moe_stage_rows_dma(const moe_bank *src, const int32_t *rows, int n, const moe_bank *dst,
                       int H, int I, int parts, void *stream);

/*
 * moe_finalize -- ordered fp32 FMA combine of the k rows of each token.
 *
 * out[t][o] = bf16_rne(acc) with acc = +0.0f and, for j = 0 .. k-1 in the
 * order topk gives, acc = fmaf(topk_w[t][j], float(Y[t*k+j][o]), acc) ("vLLM:
 * Pin Hot Experts", sections "Results, September 17" and "Update, September 17
 * afternoon": accumulate the six bf16 rows in fp32 with fma in the original k
 * order and cast once; bit-identical to the unsplit call by construction).
 *
 * Y: device bf16 [T*k][H]. topk_w: device fp32 [T][k]. out: device bf16 [T][H].
 */
int moe_finalize(const uint16_t *Y, const float *topk_w, int T, int k, int H, uint16_t *out,
                 void *stream);

/*
 * moe_usage_counts -- snapshot of the usage-counter table for a host reader.
 *
 * Enqueues an asynchronous copy of counts (device int32 [L][E]) into host_dst
 * (pinned host int32 [L][E], L*E*4 bytes; 61,440 bytes for 40 x 384). The
 * table is not reset. The snapshot is complete once the stream reaches this
 * point ("We Built the Counter", section 2: a side thread reads the table
 * every 64 steps; the counts are read approximately, so no ordering against
 * in-flight atomics is needed).
 */
int moe_usage_counts(const int32_t *counts, int L, int E, int32_t *host_dst, void *stream);

/*
 * moe_swap_rows -- true row swap between the banks, applied between steps.
 *
 * Stale check on the host mirrors first: hot_owner[hot_row] must equal
 * expect_hot_expert and cold_owner[cold_row] must equal expect_cold_expert;
 * otherwise MOE_ESTALE and nothing is enqueued ("We Built the Counter",
 * section 2: swaps are decided against a host copy of each layer's hot/cold
 * lists and refused if the rows moved since). Then, on `stream`, for each of
 * w13, s13, w2, s2: staging <- hot[hot_row]; hot[hot_row] <- cold[cold_row];
 * cold[cold_row] <- staging; then the two-element map write
 * row_map[expect_hot_expert] = -1 - cold_row and
 * row_map[expect_cold_expert] = hot_row, ordered after the copies ("vLLM: Pin
 * Hot Experts", section "Closed, September 17 evening", E4/E4b: hot row to a
 * staging row, cold row into the hot slot, staging into the cold slot, then a
 * two-element write to the device row map). Finally the host mirrors are
 * updated: hot_owner[hot_row] = expect_cold_expert, cold_owner[cold_row] =
 * expect_hot_expert.
 *
 * Call only between steps, on the stream the layer runs on. staging: device,
 * >= moe_expert_bytes(H, I) bytes. row_map: device int32 [E]. hot_owner /
 * cold_owner: host int32 [n_rows] of each bank, owned by the caller.
 */
int moe_swap_rows(const moe_bank *hot, const moe_bank *cold, int hot_row, int cold_row,
                  int expect_hot_expert, int expect_cold_expert, int32_t *row_map, int E,
                  int32_t *hot_owner, int32_t *cold_owner, void *staging, size_t staging_bytes,
                  int H, int I, void *stream);

/* Message for the last error returned on this thread ("" if none). */
const char *moe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_RESIDENCY_H */
