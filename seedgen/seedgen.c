/*
 * seedgen.c -- seeded synthetic inputs for the MoE expert stack (host side).
 *
 * This module produces input bytes only: random expert blobs in the canonical
 * byte layout, normally distributed router weights and activations.  It holds
 * none of the MoE block's arithmetic (no dequantisation, no products, no
 * routing).  Both the oracle tests and the GPU path consume what it writes;
 * the GPU twin of the blob generator lives in seedgen_dev.hip and must write
 * the same bytes (checked by the GPU tests).
 *
 * Generator: SplitMix64 (Steele, Lea, Flood, "Fast splittable pseudorandom
 * number generators", OOPSLA 2014) used counter-style: output i of a stream
 * with key k is mix64(k + (i + 1) * 0x9E3779B97F4A7C15), where mix64 is the
 * SplitMix64 finaliser.  Every value is a pure function of
 * (seed, layer, expert, stream, index), so any sub-range can be regenerated
 * independently and in parallel.
 *
 * Build: gcc -O2 -fPIC -shared -ffp-contract=off -fopenmp seedgen.c -lm
 * (-ffp-contract=off keeps the uniform -> [lo,hi) mapping a separate multiply
 * and add, which the device twin reproduces with explicitly rounded ops).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#define SG_GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t sg_mix64(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

/* Stream key for (seed, layer, expert, stream). */
uint64_t sg_key(uint64_t seed, uint64_t layer, uint64_t expert, uint64_t stream)
{
    uint64_t k = sg_mix64(seed + SG_GOLDEN);
    k = sg_mix64(k ^ (layer + 1) * 0xD1B54A32D192ED03ULL);
    k = sg_mix64(k ^ (expert + 1) * 0xABC98388FB8FAC03ULL);
    k = sg_mix64(k ^ (stream + 1) * 0x8CB92BA72F3D8DD7ULL);
    return k;
}

uint64_t sg_at(uint64_t key, uint64_t i) { return sg_mix64(key + (i + 1) * SG_GOLDEN); }

/* Round an fp32 value to bf16, round-to-nearest-even on the bit pattern. */
uint16_t sg_bf16_rne(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* Uniform fp32 in [lo, hi) from 24 random bits: lo + (u24 * 2^-24) * (hi - lo),
 * each operation rounded to fp32 separately. */
static inline float sg_unif24(uint32_t u24, float lo, float width)
{
    volatile float t = (float)u24 * (1.0f / 16777216.0f);
    volatile float p = t * width;
    return lo + p;
}

/* n_words uniform 32-bit words: word 2p and 2p+1 are the low and high halves
 * of output p.  Fills dst[w] for w in [w0, w0 + n). */
void sg_fill_words(uint64_t key, uint32_t *dst, uint64_t w0, uint64_t n)
{
#pragma omp parallel for schedule(static) if (n > (1u << 20))
    for (int64_t t = 0; t < (int64_t)n; ++t) {
        uint64_t w = w0 + (uint64_t)t;
        uint64_t z = sg_at(key, w >> 1);
        dst[t] = (w & 1) ? (uint32_t)(z >> 32) : (uint32_t)z;
    }
}

/* Group words {bf16 scale (low half), bf16 bias (high half)} for groups
 * [n0, n0 + n): scale from bits 40..63, bias from bits 8..31 of output n. */
void sg_fill_sb(uint64_t key, uint32_t *dst, uint64_t n0, uint64_t n,
                float s_lo, float s_hi, float b_lo, float b_hi)
{
    volatile float sw = s_hi - s_lo, bw = b_hi - b_lo;
    float s_w = sw, b_w = bw;
#pragma omp parallel for schedule(static) if (n > (1u << 18))
    for (int64_t t = 0; t < (int64_t)n; ++t) {
        uint64_t z = sg_at(key, n0 + (uint64_t)t);
        float s = sg_unif24((uint32_t)(z >> 40), s_lo, s_w);
        float b = sg_unif24((uint32_t)(z >> 8) & 0xFFFFFFu, b_lo, b_w);
        dst[t] = (uint32_t)sg_bf16_rne(s) | ((uint32_t)sg_bf16_rne(b) << 16);
    }
}

/* Byte size of one canonical expert blob: three packed matrices of D*I
 * elements at `bits` each, then one 32-bit {scale, bias} word per group of
 * `group` consecutive elements along each row. */
uint64_t sg_blob_bytes(int D, int I, int bits, int group)
{
    uint64_t n = 3ull * (uint64_t)D * (uint64_t)I;
    return n * (uint64_t)bits / 8 + n / (uint64_t)group * 4;
}

/* One expert blob: q region from stream 0, group words from stream 1. */
void sg_blob(uint64_t seed, int layer, int expert, int D, int I, int bits, int group,
             float s_lo, float s_hi, float b_lo, float b_hi, uint8_t *dst)
{
    uint64_t n = 3ull * (uint64_t)D * (uint64_t)I;
    uint64_t q_words = n * (uint64_t)bits / 32;
    uint64_t n_groups = n / (uint64_t)group;
    sg_fill_words(sg_key(seed, (uint64_t)layer, (uint64_t)(uint32_t)expert, 0), (uint32_t *)dst, 0, q_words);
    sg_fill_sb(sg_key(seed, (uint64_t)layer, (uint64_t)(uint32_t)expert, 1),
               (uint32_t *)(dst + q_words * 4), 0, n_groups, s_lo, s_hi, b_lo, b_hi);
}

/* n normal deviates N(0, sigma^2) as fp32, Box-Muller in fp64: pair p uses
 * outputs 2p and 2p+1 of the stream; element 2p = r cos(theta),
 * element 2p+1 = r sin(theta). */
void sg_normal(uint64_t key, float *dst, uint64_t n, double sigma)
{
    const double two_pi = 6.283185307179586476925286766559;
    int64_t pairs = (int64_t)((n + 1) / 2);
#pragma omp parallel for schedule(static) if (n > (1u << 18))
    for (int64_t p = 0; p < pairs; ++p) {
        uint64_t a = sg_at(key, 2 * (uint64_t)p), b = sg_at(key, 2 * (uint64_t)p + 1);
        double u1 = ((double)(a >> 11) + 1.0) * (1.0 / 9007199254740992.0); /* (0, 1] */
        double u2 = (double)(b >> 11) * (1.0 / 9007199254740992.0);         /* [0, 1) */
        double r = sqrt(-2.0 * log(u1)) * sigma;
        double th = two_pi * u2;
        dst[2 * p] = (float)(r * cos(th));
        if ((uint64_t)(2 * p + 1) < n) dst[2 * p + 1] = (float)(r * sin(th));
    }
}
