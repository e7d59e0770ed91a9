/*
 * CPU oracle for the routed MXFP4 MoE layer with hot/cold expert residency.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the plain, slow, obviously correct
 * definition that the GPU path is checked against. Only the test suite, the
 * smoke check and the benchmark's CPU-baseline leg may load it. The product
 * library never links, loads or calls it, and it includes nothing from the
 * product sources (no shared headers, tables or helpers).
 *
 * What it computes, and the passage each step follows:
 *
 *  - MXFP4 element decode (E2M1) and block-scale decode (E8M0): the pages only
 *    name the format ("packed weights plus ue8m0 block scales", "vLLM: Pin Hot
 *    Experts", section "Where the experts live today"); the values follow the
 *    OCP Microscaling (MX) v1.0 definitions, written out from the bit fields.
 *  - Expert FFN per (token, pick): gate/up GEMM, SwiGLU, down GEMM, producing one
 *    unweighted bf16 row per pick (the "six bf16 rows" that the split calls
 *    leave unfinalized, "vLLM: Pin Hot Experts", section "Results, September
 *    17"). Accumulation in fp64, rounded to fp32 at g, u, h and y; the row is
 *    then rounded once to bf16 (round to nearest even).
 *  - Finalize: per token, acc = +0.0f and acc = fmaf(w[j], Y[j], acc) for
 *    j = 0..k-1 in the router's order, then one cast to bf16 ("vLLM: Pin Hot
 *    Experts", sections "Results, September 17" and "Update, September 17
 *    afternoon": accumulate in fp32 with fma in the original k order, cast
 *    once).
 *  - Layer: each pick's expert id is resolved through the row map to (bank,
 *    row); the expert's weights are read from that bank row ("vLLM: Pin Hot
 *    Experts", section "The one open door": int32[384] row map per layer).
 *
 * Compiled with -O2 -ffp-contract=off and no fast-math, so every multiply and
 * add above is a separately rounded IEEE operation, and fmaf is the only fused
 * operation.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- MX element formats (OCP MX v1.0) ---------------------------------- */

/* E2M1: 1 sign bit (bit 3), 2 exponent bits (bits 2..1, bias 1), 1 mantissa
 * bit (bit 0). Exponent field 0 encodes subnormals: 2^(1-bias) * (m/2).
 * Otherwise 2^(e-bias) * (1 + m/2). No infinities or NaNs. */
double oracle_e2m1(int code)
{
    int sign = (code >> 3) & 1;
    int e = (code >> 1) & 3;
    int m = code & 1;
    double mag;
    if (e == 0)
        mag = ldexp((double)m / 2.0, 1 - 1);
    else
        mag = ldexp(1.0 + (double)m / 2.0, e - 1);
    return sign ? -mag : mag;
}

/* E8M0: an unsigned biased exponent, value 2^(b-127); 0xFF is NaN. */
double oracle_e8m0(int b)
{
    if (b == 255)
        return NAN;
    return ldexp(1.0, b - 127);
}

/* ---- bf16 <-> fp32 ------------------------------------------------------ */

float oracle_bf16_to_f32(uint16_t v)
{
    uint32_t u = (uint32_t)v << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Round to nearest, ties to even, on the 16 dropped mantissa bits. NaN stays
 * NaN (sign kept, quiet bit forced). */
uint16_t oracle_f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t keep = u >> 16;
    uint32_t rest = u & 0xffffu;
    if (rest > 0x8000u || (rest == 0x8000u && (keep & 1u)))
        keep += 1u;
    return (uint16_t)keep;
}

/* ---- dequantization ----------------------------------------------------- */

/* Element c of a packed row: byte c/2, low nibble for even c, high for odd c.
 * Its scale is byte c/32 of the row's scale vector. */
static double deq(const uint8_t *wrow, const uint8_t *srow, int c)
{
    int byte = wrow[c >> 1];
    int code = (c & 1) ? (byte >> 4) : (byte & 15);
    return oracle_e2m1(code) * oracle_e8m0(srow[c >> 5]);
}

/* Dequantize `rows` rows of K elements into fp32. An E2M1 value times a power
 * of two is exact in fp32 for every E8M0 byte up to 252; from 253 on the
 * largest magnitudes overflow to +-inf (the FFN below dequantizes in fp64 and
 * never overflows). */
void oracle_dequant(const uint8_t *w, const uint8_t *s, int64_t rows, int K, float *out)
{
    for (int64_t r = 0; r < rows; ++r)
        for (int c = 0; c < K; ++c)
            out[r * K + c] = (float)deq(w + r * (K / 2), s + r * (K / 32), c);
}

/* ---- SwiGLU ------------------------------------------------------------- */

/* silu(z) = z / (1 + e^-z), in fp64, written in the form that does not
 * overflow for large |z|. */
double oracle_silu(double z)
{
    if (z >= 0.0)
        return z / (1.0 + exp(-z));
    double ez = exp(z);
    return z * ez / (1.0 + ez);
}

/* ---- one expert FFN on one token --------------------------------------- */

/*
 * w13: [2I][H/2] bytes, rows [0,I) gate, [I,2I) up; s13: [2I][H/32].
 * w2:  [H][I/2] bytes;  s2: [H][I/32].
 * x: [H] bf16. Outputs (any may be NULL): g, u, h as fp32 [I]; y as fp32 [H];
 * y_bf16 as bf16 [H].
 */
void oracle_expert_ffn(const uint8_t *w13, const uint8_t *s13, const uint8_t *w2,
                       const uint8_t *s2, int H, int I, const uint16_t *x, float *g_out,
                       float *u_out, float *h_out, float *y_out, uint16_t *y_bf16)
{
    double *xd = (double *)malloc(sizeof(double) * (size_t)H);
    float *h = (float *)malloc(sizeof(float) * (size_t)I);
    for (int c = 0; c < H; ++c)
        xd[c] = (double)oracle_bf16_to_f32(x[c]);

    for (int i = 0; i < I; ++i) {
        const uint8_t *gw = w13 + (size_t)i * (H / 2);
        const uint8_t *gs = s13 + (size_t)i * (H / 32);
        const uint8_t *uw = w13 + (size_t)(I + i) * (H / 2);
        const uint8_t *us = s13 + (size_t)(I + i) * (H / 32);
        double g = 0.0, u = 0.0;
        for (int c = 0; c < H; ++c) {
            g += deq(gw, gs, c) * xd[c];
            u += deq(uw, us, c) * xd[c];
        }
        float gf = (float)g, uf = (float)u;
        float hf = (float)(oracle_silu((double)gf) * (double)uf);
        h[i] = hf;
        if (g_out) g_out[i] = gf;
        if (u_out) u_out[i] = uf;
        if (h_out) h_out[i] = hf;
    }
    for (int o = 0; o < H; ++o) {
        const uint8_t *dw = w2 + (size_t)o * (I / 2);
        const uint8_t *ds = s2 + (size_t)o * (I / 32);
        double y = 0.0;
        for (int i = 0; i < I; ++i)
            y += deq(dw, ds, i) * (double)h[i];
        float yf = (float)y;
        if (y_out) y_out[o] = yf;
        if (y_bf16) y_bf16[o] = oracle_f32_to_bf16(yf);
    }
    free(h);
    free(xd);
}

/* ---- finalize ----------------------------------------------------------- */

/* out[t][o] = bf16( fma chain over j = 0..k-1 of w[t][j] * float(Y[t][j][o]) ),
 * starting from +0.0f. */
void oracle_finalize(const uint16_t *Y, const float *w, int T, int k, int H, uint16_t *out)
{
    for (int t = 0; t < T; ++t)
        for (int o = 0; o < H; ++o) {
            float acc = 0.0f;
            for (int j = 0; j < k; ++j)
                acc = fmaf(w[t * k + j],
                           oracle_bf16_to_f32(Y[((size_t)t * k + j) * H + o]), acc);
            out[(size_t)t * H + o] = oracle_f32_to_bf16(acc);
        }
}

/* ---- whole layer -------------------------------------------------------- */

typedef struct {
    const uint8_t *w13, *s13, *w2, *s2;
    int32_t n_rows;
} oracle_bank;

/*
 * Resolve pick s = t*k + j: id = topk_ids[s], m = row_map[id]; m >= 0 is hot
 * row m, m < 0 is cold row -1-m. Compute the expert FFN on x[t] and write the
 * bf16 row Y[s]. Returns the number of picks whose id or row is out of range
 * (their Y rows are zero-filled and they make the layer output meaningless).
 * Then finalize into out[T][H]. nthreads <= 0 keeps the OpenMP default.
 */
int oracle_moe_layer(const uint8_t *hw13, const uint8_t *hs13, const uint8_t *hw2,
                     const uint8_t *hs2, int n_hot, const uint8_t *cw13, const uint8_t *cs13,
                     const uint8_t *cw2, const uint8_t *cs2, int n_cold,
                     const int32_t *row_map, int E, const int32_t *topk_ids,
                     const float *topk_w, int T, int k, int H, int I, const uint16_t *x,
                     uint16_t *Y, uint16_t *out, int nthreads)
{
    oracle_bank hot = {hw13, hs13, hw2, hs2, n_hot};
    oracle_bank cold = {cw13, cs13, cw2, cs2, n_cold};
    const size_t b13 = (size_t)2 * I * (H / 2), bs13 = (size_t)2 * I * (H / 32);
    const size_t b2 = (size_t)H * (I / 2), bs2 = (size_t)H * (I / 32);
    int bad = 0;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel for schedule(dynamic, 1) reduction(+ : bad)
    for (int s = 0; s < T * k; ++s) {
        int id = topk_ids[s];
        uint16_t *yrow = Y + (size_t)s * H;
        const oracle_bank *b = NULL;
        int row = -1;
        if (id >= 0 && id < E) {
            int m = row_map[id];
            if (m >= 0 && m < hot.n_rows) {
                b = &hot;
                row = m;
            } else if (m < 0 && -1 - m < cold.n_rows) {
                b = &cold;
                row = -1 - m;
            }
        }
        if (!b) {
            memset(yrow, 0, sizeof(uint16_t) * (size_t)H);
            bad += 1;
            continue;
        }
        oracle_expert_ffn(b->w13 + (size_t)row * b13, b->s13 + (size_t)row * bs13,
                          b->w2 + (size_t)row * b2, b->s2 + (size_t)row * bs2, H, I,
                          x + (size_t)(s / k) * H, NULL, NULL, NULL, NULL, yrow);
    }
    oracle_finalize(Y, topk_w, T, k, H, out);
    return bad;
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
