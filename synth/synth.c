/*
 * Seeded synthetic MXFP4 expert weights (host side).
 *
 * This is an input generator only: it holds none of the MoE layer's arithmetic.
 * It serves both the CPU oracle (through the tests) and the GPU path (through
 * the benchmark), and has a device twin in synth_dev.hip that must produce the
 * same bytes.
 *
 * Generator: counter-based SplitMix64. The mixing function is the finalizer of
 * SplitMix64 as published by Steele, Lea and Flood ("Fast splittable
 * pseudorandom number generators", OOPSLA 2014; constants as in Vigna's
 * public-domain splitmix64.c). Word i of a stream with key K is
 * mix(K + (i + 1) * GAMMA); byte n of the stream is byte (n mod 8), little
 * endian, of word n / 8.
 *
 * Stream key for (seed, layer, expert, tensor), tensor 0..3 = w13, s13, w2, s2:
 *   k0 = mix(seed + GAMMA)
 *   k1 = mix(k0 ^ mix(layer  + 2*GAMMA))
 *   k2 = mix(k1 ^ mix(expert + 3*GAMMA))
 *   k3 = mix(k2 ^ mix(tensor + 4*GAMMA))
 *
 * Weight bytes are the raw stream bytes (two uniform E2M1 codes per byte).
 * Scale bytes map a stream byte b to lo + ((b * cnt) >> 8), i.e. E8M0 values
 * spread near-uniformly over lo .. lo+cnt-1.
 */
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define GAMMA 0x9e3779b97f4a7c15ULL

static inline uint64_t mix(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
    return z ^ (z >> 31);
}

uint64_t synth_key(uint64_t seed, int64_t layer, int64_t expert, int64_t tensor)
{
    uint64_t k = mix(seed + GAMMA);
    k = mix(k ^ mix((uint64_t)layer + 2 * GAMMA));
    k = mix(k ^ mix((uint64_t)expert + 3 * GAMMA));
    k = mix(k ^ mix((uint64_t)tensor + 4 * GAMMA));
    return k;
}

static inline uint64_t word(uint64_t key, uint64_t i) { return mix(key + (i + 1) * GAMMA); }

/* Fill n bytes (n a multiple of 8) of stream `key`, starting at word w0. If
 * cnt > 0 the bytes are mapped to lo + ((b * cnt) >> 8). */
static void fill_words(uint8_t *dst, uint64_t n, uint64_t key, uint64_t w0, int lo, int cnt)
{
    for (uint64_t i = 0; i < n / 8; ++i) {
        uint64_t v = word(key, w0 + i);
        uint8_t b[8];
        memcpy(b, &v, 8);
        if (cnt > 0)
            for (int j = 0; j < 8; ++j)
                b[j] = (uint8_t)(lo + ((b[j] * cnt) >> 8));
        memcpy(dst + 8 * i, b, 8);
    }
}

/* Byte sizes of one expert's tensors. */
static void sizes(int H, int I, uint64_t sz[4])
{
    sz[0] = (uint64_t)2 * I * (H / 2);
    sz[1] = (uint64_t)2 * I * (H / 32);
    sz[2] = (uint64_t)H * (I / 2);
    sz[3] = (uint64_t)H * (I / 32);
}

/*
 * Fill a bank: row r holds expert owners[r] (rows with owner < 0 are zeroed).
 * Tensors are [n_rows][bytes-per-expert] each. Parallel over (tensor, row,
 * 1 MiB piece).
 */
void synth_fill_bank(uint8_t *w13, uint8_t *s13, uint8_t *w2, uint8_t *s2, int n_rows,
                     const int32_t *owners, uint64_t seed, int64_t layer, int H, int I,
                     int scale_lo, int scale_cnt, int nthreads)
{
    uint8_t *dst[4] = {w13, s13, w2, s2};
    uint64_t sz[4];
    sizes(H, I, sz);
    const uint64_t piece = 1u << 20;
    uint64_t npieces[4], total = 0, start[5];
    for (int t = 0; t < 4; ++t) {
        npieces[t] = (sz[t] + piece - 1) / piece;
        start[t] = total;
        total += npieces[t] * (uint64_t)n_rows;
    }
    start[4] = total;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t job = 0; job < (int64_t)total; ++job) {
        int t = 0;
        while ((uint64_t)job >= start[t + 1])
            ++t;
        uint64_t rel = (uint64_t)job - start[t];
        uint64_t r = rel / npieces[t], p = rel % npieces[t];
        uint64_t off = p * piece;
        uint64_t n = sz[t] - off < piece ? sz[t] - off : piece;
        uint8_t *d = dst[t] + r * sz[t] + off;
        int e = owners[r];
        if (e < 0) {
            memset(d, 0, n);
            continue;
        }
        uint64_t key = synth_key(seed, layer, e, t);
        int scale = (t == 1 || t == 3);
        fill_words(d, n, key, off / 8, scale_lo, scale ? scale_cnt : 0);
    }
}
