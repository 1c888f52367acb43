// moe_device.h -- device building blocks shared by libmoe's kernels.
//
// Dequantised matrix-vector products.  The weight is w = q*scale + bias with
// one bf16 scale/bias pair per group of 64 inputs (toolarium.ru,
// "Оптимизации, которые сработали": nibble*scale + bias, and its FMA rewrite
// fma(nibble, scale*x, bias*x)).  The rewrite is taken one step further and
// applied per group: sum_j (q_j*s + b) x_j = s * sum_j q_j x_j + b * sum_j x_j,
// so the bias costs one FMA per group and the inner loop is a pure
// code-times-activation sum.
//
// That inner sum runs on the integer dot unit.  An activation vector is
// turned into fixed point once (x_int = round(x * 2^k), |x_int| < 2^22, k
// from the vector's largest magnitude) and split into three signed 8-bit
// digit planes, x_int = d0 + 256 d1 + 65536 d2.  A 32-bit word of codes,
// masked so that each byte holds one code, then meets the matching digit
// words in three v_dot4_i32_i8 (four code*digit products each, exact in
// int32).  In the one-vector kernels the activations take six base-16
// digit planes instead and the codes meet them eight at a time in
// v_dot8 (4-bit codes: unsigned digits of x_int + 2^22, the offset removed
// exactly with the codes' sum; 2-bit codes: signed digits, x_int =
// sum_p d_p 16^p, after one mask or one shift and mask of a code word).
// Per 16-byte chunk the plane sums are combined exactly in int32, rounded
// once to fp32 and scaled by 2^-k * scale.  Apart from the fixed-point rounding of x
// (half a unit of 2^-k, about 1e-7 of the vector's largest element) the sum
// is exact.  Cost in the one-vector kernels: under one vector operation per
// weight, against about 3 for a float conversion and an FMA per weight.
#pragma once
#include "moe_internal.h"

namespace moe {
namespace dev {

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Sum / max over groups of W consecutive lanes (W a power of two <= 64),
// the result in every lane of the group.  Inside a row of 16 lanes the
// steps are DPP moves (two quad permutations, the half-row and the row
// mirror: each pairs a lane with one of the other half of its group), 32
// lanes swap halves through ds_swizzle, and the full wave reads the four
// row results (lanes 0, 16, 32, 48) as scalars, with no LDS round trip.
// Every lane of a group adds the same operands, so the result is
// bit-identical across the group.  All 64 lanes must be active.
template <int CTRL>
__device__ __forceinline__ float fdpp(float v, float identity)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(identity), __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int W>
__device__ __forceinline__ float group_sum(float v)
{
    static_assert(W >= 1 && W <= 64 && (W & (W - 1)) == 0, "W: power of two <= 64");
    if constexpr (W >= 2) v += fdpp<0xB1>(v, 0.f);   // quad_perm [1,0,3,2]
    if constexpr (W >= 4) v += fdpp<0x4E>(v, 0.f);   // quad_perm [2,3,0,1]
    if constexpr (W >= 8) v += fdpp<0x141>(v, 0.f);  // row_half_mirror
    if constexpr (W >= 16) v += fdpp<0x140>(v, 0.f); // row_mirror
    if constexpr (W == 32) v += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F));  // lane ^ 16
    if constexpr (W == 64)
        v = (__int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0)) +
             __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16))) +
            (__int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32)) +
             __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48)));
    return v;
}
template <int W>
__device__ __forceinline__ float group_max(float v)
{
    static_assert(W >= 1 && W <= 64 && (W & (W - 1)) == 0, "W: power of two <= 64");
    if constexpr (W >= 2) v = fmaxf(v, fdpp<0xB1>(v, -INFINITY));
    if constexpr (W >= 4) v = fmaxf(v, fdpp<0x4E>(v, -INFINITY));
    if constexpr (W >= 8) v = fmaxf(v, fdpp<0x141>(v, -INFINITY));
    if constexpr (W >= 16) v = fmaxf(v, fdpp<0x140>(v, -INFINITY));
    if constexpr (W == 32) v = fmaxf(v, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F)));
    if constexpr (W == 64)
        v = fmaxf(fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0)),
                        __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16))),
                  fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32)),
                        __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48))));
    return v;
}

// Code layout of one 16-byte chunk (four little-endian 32-bit words).
// A word holds 32/BITS codes; SUBS masked copies of it put one code per
// byte: sub s keeps codes s, s+SUBS, s+2*SUBS, s+3*SUBS of the word, so byte
// j of sub s of word k is the chunk's code k*(32/BITS) + s + SUBS*j.
template <int BITS>
struct Codes {
    static constexpr int CODES = 128 / BITS;       // codes per chunk
    static constexpr int PER_WORD = 32 / BITS;     // codes per word
    static constexpr int SUBS = 8 / BITS;          // masked copies per word
    static constexpr uint32_t MASK = BITS == 4 ? 0x0F0F0F0Fu : 0x03030303u;
    static constexpr int PW = 4 * SUBS;            // base-256 digit words per plane and chunk
    static constexpr int DW = 3 * PW;              // digit words per chunk (both digit formats)
};

// Fixed-point exponent for a vector whose largest magnitude is amax:
// mul = 2^k with amax * 2^k < 2^22 (k = 0 for a zero vector).
__device__ __forceinline__ void fixed_scale(float amax, float &mul, float &inv)
{
    int e = 0;
    if (amax > 0.f && amax < INFINITY) (void)frexpf(amax, &e);  // amax < 2^e
    const int k = amax > 0.f ? 22 - e : 0;
    mul = ldexpf(1.f, k);
    inv = ldexpf(1.f, -k);
}

// The matrix-core (batched) path's digits: the three signed base-256
// digits of xi = round(v * mul) (|xi| < 2^22):
// xi = d0 + 256 d1 + 65536 d2 with d0, d1 in [-128, 127] (sign-extended low
// bytes) and |d2| <= 64.  Four values at once, as three packed digit words
// (byte j of word p: digit p of value j).  d0 is the low byte of xi;
// y = xi - d0 holds d1 in its byte 1; z = y - 256 d1 holds d2 in its byte 2;
// the bytes are gathered with byte permutes.
__device__ __forceinline__ void digit_words(float a, float b, float c, float d, float mul, int &w0, int &w1, int &w2)
{
    const int xa = __float2int_rn(a * mul), xb = __float2int_rn(b * mul);
    const int xc = __float2int_rn(c * mul), xd = __float2int_rn(d * mul);
    const int ya = xa - __builtin_amdgcn_sbfe(xa, 0, 8), yb = xb - __builtin_amdgcn_sbfe(xb, 0, 8);
    const int yc = xc - __builtin_amdgcn_sbfe(xc, 0, 8), yd = xd - __builtin_amdgcn_sbfe(xd, 0, 8);
    const int za = ya - (__builtin_amdgcn_sbfe(ya, 8, 8) << 8), zb = yb - (__builtin_amdgcn_sbfe(yb, 8, 8) << 8);
    const int zc = yc - (__builtin_amdgcn_sbfe(yc, 8, 8) << 8), zd = yd - (__builtin_amdgcn_sbfe(yd, 8, 8) << 8);
    // v_perm_b32(hi, lo, sel): selector bytes 0-3 pick lo's bytes, 4-7 hi's
    w0 = (int)__builtin_amdgcn_perm(__builtin_amdgcn_perm(xd, xc, 0x0c0c0400u), __builtin_amdgcn_perm(xb, xa, 0x0c0c0400u),
                                    0x05040100u);
    w1 = (int)__builtin_amdgcn_perm(__builtin_amdgcn_perm(yd, yc, 0x0c0c0501u), __builtin_amdgcn_perm(yb, ya, 0x0c0c0501u),
                                    0x05040100u);
    w2 = (int)__builtin_amdgcn_perm(__builtin_amdgcn_perm(zd, zc, 0x0c0c0602u), __builtin_amdgcn_perm(zb, za, 0x0c0c0602u),
                                    0x05040100u);
}

// 2-bit chunks: six signed base-16 digits of xi = round(v * mul),
// xi = sum_p d_p 16^p with d_p in [-8, 7] (|xi| < 2^22 leaves |d_5| <= 4).
// Word (2 k + s) * 6 + p of a chunk holds, in nibble j, digit p of value
// 16 k + s + 2 j: the values of codes s, s + 2, ..., s + 14 of code word k,
// which the mask 0x33333333 of the word (s = 0) or of the word shifted
// right by 2 (s = 1) leaves as nibbles.  48 words per chunk (Codes<2>::DW).
constexpr int kNibPlanes = 6;

// The digits come out of one add and one XOR: y = xi + 0x888888 lies in
// [0, 2^24) and equals sum_p (d_p + 8) 16^p, so nibble p of y is d_p + 8
// in [0, 15], and flipping its top bit leaves d_p as a signed 4-bit number.
__device__ __forceinline__ uint32_t nib_digits(float v, float mul)
{
    return (uint32_t)(__float2int_rn(v * mul) + 0x888888) ^ 0x888888u;
}

// the six digit words of the eight values v[0], v[2], ..., v[14]
__device__ __forceinline__ void nib_words(const float *v, float mul, int *o)
{
    uint32_t w[kNibPlanes] = {0u, 0u, 0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint32_t z = nib_digits(v[2 * j], mul);
#pragma unroll
        for (int p = 0; p < kNibPlanes; ++p) w[p] |= ((z >> (4 * p)) & 15u) << (4 * j);
    }
#pragma unroll
    for (int p = 0; p < kNibPlanes; ++p) o[p] = (int)w[p];
}

// 4-bit chunks: six unsigned base-16 digits of u = xi + 2^22, which lies in
// [0, 2^23): word k * 6 + p of a chunk holds, in nibble j, digit p of
// value 8 k + j, the value of code j of code word k, so a code word meets
// its six digit words unmasked in v_dot8_u32_u4.  sum code * u minus
// 2^22 * sum code is sum code * xi exactly (modulo 2^32, and that sum is
// below 2^31 in magnitude).  24 words per chunk (Codes<4>::DW).
__device__ __forceinline__ uint32_t unib_digits(float v, float mul)
{
    return (uint32_t)(__float2int_rn(v * mul) + 0x400000);
}

// the six digit words of the eight values v[0..8)
__device__ __forceinline__ void unib_words(const float *v, float mul, int *o)
{
    uint32_t w[kNibPlanes] = {0u, 0u, 0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint32_t z = unib_digits(v[j], mul);
#pragma unroll
        for (int p = 0; p < kNibPlanes; ++p) w[p] |= ((z >> (4 * p)) & 15u) << (4 * j);
    }
#pragma unroll
    for (int p = 0; p < kNibPlanes; ++p) o[p] = (int)w[p];
}

// Digit words of one chunk from the chunk's activations v[0..CODES) in the
// nibble planes above (2-bit signed, 4-bit unsigned), by one thread.
template <int BITS>
__device__ __forceinline__ void chunk_digits(const float *v, float mul, int *dg)
{
    if constexpr (BITS == 2) {
#pragma unroll
        for (int k = 0; k < 4; ++k)
#pragma unroll
            for (int sh = 0; sh < 2; ++sh) nib_words(v + 16 * k + sh, mul, dg + (2 * k + sh) * kNibPlanes);
    } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) unib_words(v + 8 * k, mul, dg + k * kNibPlanes);
    }
}

// sum over one chunk of code * x_int, from the chunk's digit words; exact
// in int32, rounded to fp32 once.
template <int BITS>
__device__ __forceinline__ float qdot(const uint4 q, const int *dg)
{
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
    if constexpr (BITS == 2) {
        // nibble planes: |a_p| <= 64 * 3 * 8, and the Horner sums are partial
        // sums of sum code * (xi >> 4m), below 8.1e8: exact in int32
        int a[kNibPlanes] = {0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int ev = (int)(w[k] & 0x33333333u), od = (int)((w[k] >> 2) & 0x33333333u);
#pragma unroll
            for (int p = 0; p < kNibPlanes; ++p) {
                a[p] = __builtin_amdgcn_sdot8(ev, dg[(2 * k) * kNibPlanes + p], a[p], false);
                a[p] = __builtin_amdgcn_sdot8(od, dg[(2 * k + 1) * kNibPlanes + p], a[p], false);
            }
        }
        int h = a[kNibPlanes - 1];
#pragma unroll
        for (int p = kNibPlanes - 2; p >= 0; --p) h = h * 16 + a[p];
        return (float)h;
    } else {
        // unsigned nibble planes: sum code * (xi + 2^22) by Horner over the
        // planes (modulo 2^32), less 2^22 times the codes' sum
        uint32_t a[kNibPlanes] = {0u, 0u, 0u, 0u, 0u, 0u};
        uint32_t qs = 0u;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
#pragma unroll
            for (int p = 0; p < kNibPlanes; ++p)
                a[p] = __builtin_amdgcn_udot8(w[k], (uint32_t)dg[k * kNibPlanes + p], a[p], false);
            qs = __builtin_amdgcn_udot8(w[k], 0x11111111u, qs, false);
        }
        uint32_t h = a[kNibPlanes - 1];
#pragma unroll
        for (int p = kNibPlanes - 2; p >= 0; --p) h = h * 16u + a[p];
        return (float)(int)(h - (qs << 22));
    }
}

// Digit table of one chunk built in registers, with a fixed-point step of
// its own.  A chunk's CODES values are held as float4 by G = CODES/4
// consecutive lanes (lane f of the chunk holds values 4f..4f+3, float4 q
// of the vector).  4-bit: the word of plane p for code word k, sub s holds
// values k*PER_WORD + s + SUBS*j, which lie in the two lanes of word k, so
// those lanes trade components through DPP and lane f writes word f of
// every plane.  2-bit: the nibble planes, written bytewise.  The chunk's largest magnitude (step inv = 2^-k with
// max * 2^k < 2^22) and its fp32 sum come from DPP reductions over the G
// lanes; lane 0 of the chunk writes csum[c] and cinv[c].  All 64 lanes
// call it; lanes past the end (whole chunks) pass valid = false and write
// nothing.
template <int BITS>
__device__ __forceinline__ void chunk_digits_lane(float4 v, int q, bool valid, int *dig, float *csum, float *cinv)
{
    using C = Codes<BITS>;
    constexpr int G = C::CODES / 4;
    static_assert(C::SUBS == C::PER_WORD / 4, "one sub per lane of a code word");
    if (!valid) v = make_float4(0.f, 0.f, 0.f, 0.f);
    const float m = group_max<G>(fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
    const float sum = group_sum<G>((v.x + v.y) + (v.z + v.w));
    float mul, inv;
    fixed_scale(m, mul, inv);
    if constexpr (BITS == 2) {
        // nibble planes: lane f (values 4f..4f+3, code word f / 4) supplies
        // byte f % 4 of its code word's twelve words, nibble pairs of its
        // values (s, s + 2) for half s
        if (!valid) return;  // after the reductions, which need every lane
        const int ch = q / G, f = q - ch * G;
        const uint32_t z[4] = {nib_digits(v.x, mul), nib_digits(v.y, mul), nib_digits(v.z, mul), nib_digits(v.w, mul)};
        uint8_t *base = reinterpret_cast<uint8_t *>(dig + ch * C::DW) + (f & 3);
#pragma unroll
        for (int sh = 0; sh < 2; ++sh) {
            // byte m: planes 2m (ev) and 2m + 1 (od) of values sh and sh + 2
            const uint32_t ev = (z[sh] & 0x0F0F0Fu) | ((z[sh + 2] & 0x0F0F0Fu) << 4);
            const uint32_t od = ((z[sh] >> 4) & 0x0F0F0Fu) | (z[sh + 2] & 0xF0F0F0u);
            uint8_t *wb = base + ((f >> 2) * 2 + sh) * kNibPlanes * 4;
#pragma unroll
            for (int m2 = 0; m2 < 3; ++m2) {
                wb[(2 * m2) * 4] = (uint8_t)(ev >> (8 * m2));
                wb[(2 * m2 + 1) * 4] = (uint8_t)(od >> (8 * m2));
            }
        }
        if (f == 0) {
            csum[ch] = sum;
            cinv[ch] = inv;
        }
    } else {
        // unsigned nibble planes: lane f (values 4f..4f+3, code word f / 2)
        // supplies bytes 2 (f % 2) and 2 (f % 2) + 1 of its code word's six
        // words, as one 16-bit store per word
        if (!valid) return;  // after the reductions, which need every lane
        const int ch = q / G, f = q - ch * G;
        const uint32_t z0 = unib_digits(v.x, mul), z1 = unib_digits(v.y, mul);
        const uint32_t z2 = unib_digits(v.z, mul), z3 = unib_digits(v.w, mul);
        // byte m: digits 2m (ev) and 2m + 1 (od) of a value pair
        const uint32_t ev01 = (z0 & 0x0F0F0Fu) | ((z1 & 0x0F0F0Fu) << 4), od01 = ((z0 >> 4) & 0x0F0F0Fu) | (z1 & 0xF0F0F0u);
        const uint32_t ev23 = (z2 & 0x0F0F0Fu) | ((z3 & 0x0F0F0Fu) << 4), od23 = ((z2 >> 4) & 0x0F0F0Fu) | (z3 & 0xF0F0F0u);
        uint16_t *wh = reinterpret_cast<uint16_t *>(dig + ch * C::DW + (f >> 1) * kNibPlanes) + (f & 1);
#pragma unroll
        for (int m2 = 0; m2 < 3; ++m2) {
            // v_perm_b32(hi, lo, sel): byte m2 of lo, then byte m2 of hi
            const uint32_t sel = 0x0c0c0000u | (uint32_t)m2 | ((uint32_t)(4 + m2) << 8);
            wh[(2 * m2) * 2] = (uint16_t)__builtin_amdgcn_perm(ev23, ev01, sel);
            wh[(2 * m2 + 1) * 2] = (uint16_t)__builtin_amdgcn_perm(od23, od01, sel);
        }
        if (f == 0) {
            csum[ch] = sum;
            cinv[ch] = inv;
        }
    }
}

// Block barrier for LDS traffic only: unlike __syncthreads it does not wait
// for the wave's outstanding global loads (prefetches may stay in flight).
__device__ __forceinline__ void lds_barrier()
{
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Block barrier: LDS-only (LDS_SYNC) or a full __syncthreads.
template <bool LDS_SYNC>
__device__ __forceinline__ void bsync()
{
    if constexpr (LDS_SYNC) lds_barrier();
    else __syncthreads();
}

// csum[c] = sum of the fp32 values of chunk c of x, for c < nc: four lanes
// per chunk, each summing a quarter in order, then the four quarters.
// Called by whole waves of the block (blockDim a multiple of 64).
template <int BITS>
__device__ __forceinline__ void chunk_sums(const float *x, int nc, float *csum)
{
    using C = Codes<BITS>;
    constexpr int Q = C::CODES / 4;
    const int nt = blockDim.x;
    for (int t0 = 0; t0 < 4 * nc; t0 += nt) {
        const int t = t0 + (int)threadIdx.x, c = t >> 2;
        float sum = 0.f;
        if (c < nc) {
            const float4 *v = reinterpret_cast<const float4 *>(x + c * C::CODES + (t & 3) * Q);
#pragma unroll
            for (int j = 0; j < Q / 4; ++j) {
                const float4 f = v[j];
                sum += f.x;
                sum += f.y;
                sum += f.z;
                sum += f.w;
            }
        }
        sum = group_sum<4>(sum);
        if (c < nc && (t & 3) == 0) csum[c] = sum;
    }
}

// Block-cooperative fixed-point digit table of an activation vector x[0..n)
// (n a multiple of the chunk width): dig[c*DW + ...] as chunk_digits lays
// out chunk c, csum[c] = sum of the chunk's fp32 values; returns 2^-k.
// `red` is LDS scratch of 16 floats.  Ends with __syncthreads.
template <int BITS, bool LDS_SYNC = false>
__device__ __forceinline__ float block_digit_table(const float *x, int n, int *dig, float *csum, float *red)
{
    using C = Codes<BITS>;
    const int tid = threadIdx.x, nt = blockDim.x;
    float m = 0.f;
    for (int i0 = tid; i0 < n; i0 += 4 * nt) {
        float v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = i0 + u * nt < n ? fabsf(x[i0 + u * nt]) : 0.f;
#pragma unroll
        for (int u = 0; u < 4; ++u) m = fmaxf(m, v[u]);
    }
    m = group_max<64>(m);
    if ((tid & 63) == 0) red[tid >> 6] = m;
    bsync<LDS_SYNC>();
    float amax = 0.f;
    for (int w = 0; w < (nt >> 6); ++w) amax = fmaxf(amax, red[w]);
    float mul, inv;
    fixed_scale(amax, mul, inv);
    if constexpr (BITS == 2) {
        // one thread per (chunk, code word, half): eight activations -> six
        // nibble words
        const int nw = n / C::CODES * 8;
        for (int t = tid; t < nw; t += nt) {
            const int c = t >> 3, k = (t >> 1) & 3, sh = t & 1;
            nib_words(x + c * C::CODES + 16 * k + sh, mul, dig + c * C::DW + (2 * k + sh) * kNibPlanes);
        }
    } else {
        // one thread per (chunk, code word): eight activations -> six
        // unsigned nibble words
        const int nw = n / C::CODES * 4;
        for (int t = tid; t < nw; t += nt) {
            const int c = t >> 2, k = t & 3;
            unib_words(x + c * C::CODES + 8 * k, mul, dig + c * C::DW + k * kNibPlanes);
        }
    }
    chunk_sums<BITS>(x, n / C::CODES, csum);
    bsync<LDS_SYNC>();
    return inv;
}

// Blob of slot k holding expert e (k < top_k) or the shared expert
// (k == top_k); nullptr, with the range bit raised, for an id outside
// [0, n_experts).  Streamed layers read slot k of the slab.
__device__ __forceinline__ const uint8_t *blob_of(const BlobSrc &s, int k, int32_t e, uint32_t *flags)
{
    if (s.slab) return s.slab + (uint64_t)k * s.blob_bytes;
    if (k >= s.top_k) return s.shared;
    if (e < 0 || e >= s.n_experts) {
        atomicOr(flags, MOE_DEVERR_EXPERT_RANGE);
        return nullptr;
    }
    return s.experts + (uint64_t)e * s.blob_bytes;
}

// Data handed between blocks inside one launch (logits, h, partial sums)
// goes through agent-scope coherent stores and loads (write-through and
// miss-on-stale at the device's coherence point), so no cache-wide
// write-back or invalidate is needed around the grid barriers.
__device__ __forceinline__ void xstore(float *p, float v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float xload(const float *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// 16 coherent bytes at float index i (a multiple of 4) of `base`.
__device__ __forceinline__ float4 xload4(const float *base, int i)
{
    __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(base), (short)0, 0x7FFFFFFF,
                                                                 0x00020000);
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, i * 4, 0, 16 /* sc1: agent scope */);
    return make_float4(__uint_as_float(v[0]), __uint_as_float(v[1]), __uint_as_float(v[2]), __uint_as_float(v[3]));
}

// Values handed between the blocks of one persistent launch travel with the
// epoch that produced them, as one 64-bit word (value low, epoch high),
// stored single-copy atomically at agent scope.  A reader polls the words it
// needs until every epoch is the expected one, so no grid barrier and no wait
// for store acknowledgements separate producer and consumer.
__device__ __forceinline__ void tag_store(uint64_t *p, float v, uint32_t tag)
{
    __hip_atomic_store(p, ((uint64_t)tag << 32) | __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Pairs i and i+1 (16 coherent bytes): x = value i, y = epoch i, z = value
// i+1, w = epoch i+1.  Each 8-byte half is one stored word.
__device__ __forceinline__ uint4 tag_load2(const uint64_t *base, int i)
{
    __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint64_t *>(base), (short)0, 0x7FFFFFFF,
                                                                 0x00020000);
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, i * 8, 0, 16 /* sc1: agent scope */);
    return make_uint4(v[0], v[1], v[2], v[3]);
}

// Byte offset past the num_records (0x7FFFFFFF) of the tag buffers' resource
// for every dword of a load issued there: such a buffer load is out of
// range, returns zeros and makes no memory access.
constexpr uint32_t kNoAccess = 0x80000000u;

// tag_load2 for a lane that still needs the words; a lane that has them
// already issues an out-of-range buffer load (no memory access, zeros).
__device__ __forceinline__ uint4 tag_load2_if(const uint64_t *base, int i, bool need)
{
    __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint64_t *>(base), (short)0, 0x7FFFFFFF,
                                                                 0x00020000);
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, need ? (uint32_t)i * 8u : kNoAccess, 0, 16 /* sc1: agent scope */);
    return make_uint4(v[0], v[1], v[2], v[3]);
}

// One wave: dot of router row `row` (D fp32) with x; x may live in LDS.
// Returns the full sum in every lane.  Rows of up to 4096 are fetched with
// every load in flight before the first FMA.
__device__ __forceinline__ float wave_router_row(const float *row, const float *x, int D, int lane)
{
    const float4 *W = reinterpret_cast<const float4 *>(row);
    const float4 *X = reinterpret_cast<const float4 *>(x);
    const int nc = D / 4;
    float acc0 = 0.f, acc1 = 0.f;
    for (int c0 = 0; c0 < nc; c0 += 16 * 64) {
        float4 w[16];
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            const int c = c0 + lane + 64 * m;
            w[m] = c < nc ? W[c] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            const int c = c0 + lane + 64 * m;
            const float4 xv = c < nc ? X[c] : make_float4(0.f, 0.f, 0.f, 0.f);
            acc0 = fmaf(w[m].x, xv.x, acc0);
            acc1 = fmaf(w[m].y, xv.y, acc1);
            acc0 = fmaf(w[m].z, xv.z, acc0);
            acc1 = fmaf(w[m].w, xv.w, acc1);
        }
    }
    return group_sum<64>(acc0 + acc1);
}

// Weight loads go through buffer instructions: the blob base sits in a
// scalar resource, the row offset in a scalar register and the lane's
// offset in one vector register (its constant part in the instruction), so
// a wave's many loads in flight cost data registers only.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t blob_rsrc(const void *base)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, 0x7FFFFFFF, 0x00020000);
}
__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
{
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
    return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ uint32_t bload4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
{
    return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}

// Gate/up rows, split into the loads and the arithmetic so that a caller can
// issue a unit's loads long before its activation is ready.  One wave owns R
// consecutive intermediate rows i0.. of one expert's gate and up matrices;
// lane l holds 16-byte chunks l, l+64, ... of every row and the scale/bias
// word of each chunk's group.  A NULL blob or a row/chunk outside the
// matrix loads zeros.
template <int BITS, int CPL, int R>
struct GuRegs {
    uint4 q[CPL][R][2];
    uint32_t sb[CPL][R][2];
};

template <int BITS, int CPL, int R>
__device__ __forceinline__ void gu_load(GuRegs<BITS, CPL, R> &g, const uint8_t *blob, int D, int I, int i0, int lane)
{
    using C = Codes<BITS>;
    const int nchunks = D * BITS / 128;
    const uint32_t mat_q = (uint32_t)I * D * BITS / 8;
    const uint32_t row_q = (uint32_t)D * BITS / 8;
    const uint32_t sb0 = 3 * mat_q;
    const uint32_t mat_sb = (uint32_t)I * (D / kGroup) * 4;
    const uint32_t row_sb = (uint32_t)(D / kGroup) * 4;
#pragma unroll
    for (int m = 0; m < CPL; ++m)
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int mat = 0; mat < 2; ++mat) {
                g.q[m][r][mat] = make_uint4(0, 0, 0, 0);
                g.sb[m][r][mat] = 0u;
            }
    if (!blob) return;
    const __amdgpu_buffer_rsrc_t rs = blob_rsrc(blob);
#pragma unroll
    for (int m = 0; m < CPL; ++m) {
        const int c = lane + 64 * m;
        if (c >= nchunks) continue;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int i = i0 + r;
            if (i >= I) continue;
#pragma unroll
            for (int mat = 0; mat < 2; ++mat) {
                g.q[m][r][mat] = bload16(rs, (uint32_t)c * 16, mat * mat_q + (uint32_t)i * row_q);
                g.sb[m][r][mat] = bload4(rs, (uint32_t)(c * C::CODES / kGroup) * 4, sb0 + mat * mat_sb + (uint32_t)i * row_sb);
            }
        }
    }
}

// The arithmetic: the activation arrives as a digit table (block_digit_table,
// in LDS) with its per-chunk sums and fixed-point step inv.  Writes
// h[i] = silu(g_i) * u_i, silu(z) = z / (1 + exp(-z)), agent-coherently.
template <int BITS, int CPL, int R>
__device__ __forceinline__ void gu_finish(const GuRegs<BITS, CPL, R> &g, const int *dig, const float *csum, float inv,
                                          int D, int I, int i0, int lane, float *h)
{
    using C = Codes<BITS>;
    const int nchunks = D * BITS / 128;
    float acc[R][2];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r][0] = acc[r][1] = 0.f;
#pragma unroll
    for (int m = 0; m < CPL; ++m) {
        const int c = lane + 64 * m;
        int dg[C::DW];
        float cs = 0.f;
        if (c < nchunks) {
            const int4 *src = reinterpret_cast<const int4 *>(dig + c * C::DW);
#pragma unroll
            for (int t = 0; t < C::DW / 4; ++t) {
                const int4 v = src[t];
                dg[4 * t] = v.x;
                dg[4 * t + 1] = v.y;
                dg[4 * t + 2] = v.z;
                dg[4 * t + 3] = v.w;
            }
            cs = csum[c];
        } else {
#pragma unroll
            for (int t = 0; t < C::DW; ++t) dg[t] = 0;
        }
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int mat = 0; mat < 2; ++mat) {
                const float qx = qdot<BITS>(g.q[m][r][mat], dg);
                acc[r][mat] = fmaf(bf16_lo(g.sb[m][r][mat]) * inv, qx, acc[r][mat]);
                acc[r][mat] = fmaf(bf16_hi(g.sb[m][r][mat]), cs, acc[r][mat]);
            }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const float gg = group_sum<64>(acc[r][0]);
        const float u = group_sum<64>(acc[r][1]);
        const int i = i0 + r;
        if (lane == 0 && i < I) xstore(h + i, gg / (1.f + expf(-gg)) * u);
    }
}

template <int BITS, int CPL, int R>
__device__ __forceinline__ void wave_gate_up(const uint8_t *blob, const int *dig, const float *csum, float inv, int D,
                                             int I, int i0, int lane, float *h)
{
    GuRegs<BITS, CPL, R> g;
    gu_load<BITS, CPL, R>(g, blob, D, I, i0, lane);
    gu_finish<BITS, CPL, R>(g, dig, csum, inv, D, I, i0, lane, h);
}

// As gu_finish against a digit table with one fixed-point step per chunk
// (cinv[c], chunk_digits_lane), returning h of the unit's rows in every
// lane instead of storing it.
template <int BITS, int CPL, int R>
__device__ __forceinline__ void gu_finish_c(const GuRegs<BITS, CPL, R> &g, const int *dig, const float *csum,
                                            const float *cinv, int D, int lane, float (&h)[R])
{
    using C = Codes<BITS>;
    const int nchunks = D * BITS / 128;
    float acc[R][2];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r][0] = acc[r][1] = 0.f;
#pragma unroll
    for (int m = 0; m < CPL; ++m) {
        // a chunk past the row's end has zero codes (gu_load) and zero
        // weights here; it reads the last chunk's digits, so that no branch
        // or zeroing of the digit registers is needed
        const int c = lane + 64 * m;
        const bool okc = c < nchunks;
        const int cc = okc ? c : nchunks - 1;
        int dg[C::DW];
        const int4 *src = reinterpret_cast<const int4 *>(dig + cc * C::DW);
#pragma unroll
        for (int t = 0; t < C::DW / 4; ++t) {
            const int4 v = src[t];
            dg[4 * t] = v.x;
            dg[4 * t + 1] = v.y;
            dg[4 * t + 2] = v.z;
            dg[4 * t + 3] = v.w;
        }
        const float cs = okc ? csum[cc] : 0.f, ci = okc ? cinv[cc] : 0.f;
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int mat = 0; mat < 2; ++mat) {
                const float qx = qdot<BITS>(g.q[m][r][mat], dg);
                acc[r][mat] = fmaf(bf16_lo(g.sb[m][r][mat]) * ci, qx, acc[r][mat]);
                acc[r][mat] = fmaf(bf16_hi(g.sb[m][r][mat]), cs, acc[r][mat]);
            }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const float gg = group_sum<64>(acc[r][0]);
        const float u = group_sum<64>(acc[r][1]);
        h[r] = gg / (1.f + expf(-gg)) * u;
    }
}

// Down rows, split the same way: one wave owns 64/LPR consecutive output
// rows o0.. of one expert's down matrix, LPR lanes per row, lane chunk
// lc + LPR*m of its row (lc = lane % LPR).
template <int BITS, int CPL>
struct DnRegs {
    uint4 q[CPL];
    uint32_t sb[CPL];
};

template <int BITS, int LPR, int CPL>
__device__ __forceinline__ void dn_load(DnRegs<BITS, CPL> &d, const uint8_t *blob, int D, int I, int o0, int lane)
{
    using C = Codes<BITS>;
    const int nchunks = I * BITS / 128;
    const int o = o0 + lane / LPR, lc = lane % LPR;
    const uint32_t mat_q = (uint32_t)I * D * BITS / 8;
    const uint32_t row_q = (uint32_t)I * BITS / 8;
    const uint32_t sbd = 3 * mat_q + 2 * ((uint32_t)D * (I / kGroup) * 4);
    const uint32_t row_sb = (uint32_t)(I / kGroup) * 4;
#pragma unroll
    for (int m = 0; m < CPL; ++m) {
        d.q[m] = make_uint4(0, 0, 0, 0);
        d.sb[m] = 0u;
    }
    if (!blob) return;
    const __amdgpu_buffer_rsrc_t rs = blob_rsrc(blob);
    // the wave's rows are o0 .. o0 + 64/LPR - 1: one scalar base, the lane's
    // row and chunk in the vector offset
#pragma unroll
    for (int m = 0; m < CPL; ++m) {
        const int c = lc + LPR * m;
        if (o < D && c < nchunks) {
            d.q[m] = bload16(rs, (uint32_t)(lane / LPR) * row_q + (uint32_t)c * 16, 2 * mat_q + (uint32_t)o0 * row_q);
            d.sb[m] = bload4(rs, (uint32_t)(lane / LPR) * row_sb + (uint32_t)(c * C::CODES / kGroup) * 4,
                             sbd + (uint32_t)o0 * row_sb);
        }
    }
}

// A lane's share of the row sums of a dn_load unit against a digit table
// of h (LDS: hdig/hcsum/hcinv of this expert's slot, one fixed-point step
// per chunk); the row's sum is the sum over its LPR lanes.
template <int BITS, int LPR, int CPL>
__device__ __forceinline__ float dn_part_c(const DnRegs<BITS, CPL> &d, const int *hdig, const float *hcsum,
                                           const float *hcinv, int I, int lane)
{
    using C = Codes<BITS>;
    const int nchunks = I * BITS / 128;
    const int lc = lane % LPR;
    float t = 0.f;
#pragma unroll
    for (int m = 0; m < CPL; ++m) {
        const int c = lc + LPR * m;
        if (c < nchunks) {
            int dg[C::DW];
            const int4 *src = reinterpret_cast<const int4 *>(hdig + c * C::DW);
#pragma unroll
            for (int t4 = 0; t4 < C::DW / 4; ++t4) {
                const int4 v = src[t4];
                dg[4 * t4] = v.x;
                dg[4 * t4 + 1] = v.y;
                dg[4 * t4 + 2] = v.z;
                dg[4 * t4 + 3] = v.w;
            }
            const float qh = qdot<BITS>(d.q[m], dg);
            t = fmaf(bf16_lo(d.sb[m]) * hcinv[c], qh, t);
            t = fmaf(bf16_hi(d.sb[m]), hcsum[c], t);
        }
    }
    return t;
}

// Router row slice: float4 columns [c_lo, c_hi) of a row, lane l holding
// columns c_lo + l + 64 m.
template <int N>
struct RtRegs {
    float4 w[N];
};

template <int N>
__device__ __forceinline__ void rt_load(RtRegs<N> &r, const float *row, int c_lo, int c_hi, int lane)
{
#pragma unroll
    for (int m = 0; m < N; ++m) r.w[m] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (!row) return;
    const __amdgpu_buffer_rsrc_t rs = blob_rsrc(row);
#pragma unroll
    for (int m = 0; m < N; ++m) {
        const int c = c_lo + lane + 64 * m;
        if (c < c_hi) {
            const uint4 v = bload16(rs, (uint32_t)(lane + 64 * m) * 16, (uint32_t)c_lo * 16);
            r.w[m] = make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w));
        }
    }
}

// Per-lane partial dot of a loaded slice with x (LDS).
template <int N>
__device__ __forceinline__ float rt_finish(const RtRegs<N> &r, const float *x, int c_lo, int c_hi, int lane)
{
    const float4 *X = reinterpret_cast<const float4 *>(x);
    float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
    for (int m = 0; m < N; ++m) {
        const int c = c_lo + lane + 64 * m;
        const float4 xv = c < c_hi ? X[c] : make_float4(0.f, 0.f, 0.f, 0.f);
        acc0 = fmaf(r.w[m].x, xv.x, acc0);
        acc1 = fmaf(r.w[m].y, xv.y, acc1);
        acc0 = fmaf(r.w[m].z, xv.z, acc0);
        acc1 = fmaf(r.w[m].w, xv.w, acc1);
    }
    return acc0 + acc1;
}

// One wave's slice sw (of kRouterSlices) of a router row: the dot of row
// (fp32 [D]) with x over float4 columns [sw*Q, min(D/4, sw*Q + Q)), Q =
// ceil(D/4 / kRouterSlices), in rounds of 64*RN float4, reduced over the
// wave; the full slice sum in every lane.  `loaded`: the first round's
// weights are already in r (loaded ahead with the same bounds).  The row's
// logit is the kRouterSlices slice sums added in slice order; every router
// GEMV of one token (the fused stack kernel's and k_route's) runs through
// this function, so they agree bit for bit.
template <int RN>
__device__ __forceinline__ float router_slice(RtRegs<RN> &r, bool loaded, const float *row, const float *x, int D,
                                              int sw, int lane)
{
    const int nc4 = D / 4, Q = (nc4 + kRouterSlices - 1) / kRouterSlices;
    const int c_hi = min(nc4, sw * Q + Q);
    float acc = 0.f;
    for (int c0 = 0; c0 < Q; c0 += 64 * RN) {
        const int c_lo = sw * Q + c0;
        if (!loaded || c0 > 0) rt_load<RN>(r, row, c_lo, c_hi, lane);
        acc += rt_finish<RN>(r, x, c_lo, c_hi, lane);
    }
    return group_sum<64>(acc);
}
// The first round of router_slice's loads, issued ahead.
template <int RN>
__device__ __forceinline__ void router_slice_load(RtRegs<RN> &r, const float *row, int D, int sw, int lane)
{
    const int nc4 = D / 4, Q = (nc4 + kRouterSlices - 1) / kRouterSlices;
    rt_load<RN>(r, row, sw * Q, min(nc4, sw * Q + Q), lane);
}

// One wave: STEPS x (64/LPR) consecutive rows o0.. of one expert's down
// matrix times h; LPR lanes per row.  A lane turns its slice of h into
// digits once (fixed-point step shared by the LPR lanes of a row, so that
// it is the same for every row) and uses them for every row it visits
// (COH: h was written by other blocks of the same launch).  out[s] (valid
// in lanes with lane % LPR == 0) is row o0 + s*(64/LPR) + lane/LPR.
template <int BITS, int LPR, int CPL, int STEPS, bool COH>
__device__ __forceinline__ void wave_down(const uint8_t *blob, const float *h, int D, int I, int o0, int lane, float *out)
{
    using C = Codes<BITS>;
    constexpr int RPS = 64 / LPR;
    const int nchunks = I * BITS / 128;
    const int sub = lane / LPR, lc = lane % LPR;
    const uint64_t mat_q = (uint64_t)I * D * BITS / 8;
    const uint64_t row_q = (uint64_t)I * BITS / 8;
    const uint64_t sbd = 3 * mat_q + 2 * ((uint64_t)D * (I / kGroup) * 4);
    const int gpr = I / kGroup;

    uint4 q[CPL][STEPS];
    uint32_t sb[CPL][STEPS];
#pragma unroll
    for (int m = 0; m < CPL; ++m)
#pragma unroll
        for (int s = 0; s < STEPS; ++s) {
            const int o = o0 + s * RPS + sub, c = lc + LPR * m;
            const bool ok = blob && o < D && c < nchunks;
            q[m][s] = ok ? *reinterpret_cast<const uint4 *>(blob + 2 * mat_q + (uint64_t)o * row_q + (uint64_t)c * 16)
                         : make_uint4(0, 0, 0, 0);
            sb[m][s] = ok ? *reinterpret_cast<const uint32_t *>(blob + sbd + ((uint64_t)o * gpr + (uint64_t)c * C::CODES / kGroup) * 4)
                          : 0u;
        }

    float t[STEPS];
#pragma unroll
    for (int s = 0; s < STEPS; ++s) t[s] = 0.f;
#pragma unroll
    for (int m = 0; m < CPL; ++m) {
        const int c = lc + LPR * m;
        const bool ok = blob && c < nchunks;
        float hv[C::CODES];
        float hs = 0.f, amax = 0.f;
#pragma unroll
        for (int j = 0; j < C::CODES; j += 4) {
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            if (ok) v = COH ? xload4(h, c * C::CODES + j) : *reinterpret_cast<const float4 *>(h + c * C::CODES + j);
            hv[j] = v.x;
            hv[j + 1] = v.y;
            hv[j + 2] = v.z;
            hv[j + 3] = v.w;
            hs += (v.x + v.y) + (v.z + v.w);
            amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
        }
        float mul, inv;
        fixed_scale(group_max<LPR>(amax), mul, inv);
        int dg[C::DW];
        chunk_digits<BITS>(hv, mul, dg);
#pragma unroll
        for (int s = 0; s < STEPS; ++s) {
            const float qh = qdot<BITS>(q[m][s], dg);
            t[s] = fmaf(bf16_lo(sb[m][s]) * inv, qh, t[s]);
            t[s] = fmaf(bf16_hi(sb[m][s]), hs, t[s]);
        }
    }
#pragma unroll
    for (int s = 0; s < STEPS; ++s) out[s] = group_sum<LPR>(t[s]);
}

constexpr uint32_t kSpinLimit = 1u << 22;

// One wave: the K largest of lg[0..E) (LDS), descending, the lower index
// first on an exact tie; idx/vals identical in every lane.  Loops run over
// the compile-time bound so the arrays stay in registers.
__device__ __forceinline__ void wave_topk(const float *lg, int E, int K, int lane, int (&idx)[kMaxTopK], float (&vals)[kMaxTopK])
{
    uint64_t taken = 0;  // bit j: element lane + 64 j already selected
#pragma unroll
    for (int k = 0; k < kMaxTopK; ++k) {
        idx[k] = -1;
        vals[k] = -INFINITY;
        if (k >= K) continue;
        float bv = -INFINITY;
        int bi = -1;
        for (int j = 0, e = lane; e < E; ++j, e += 64) {
            if ((taken >> j) & 1ull) continue;
            const float v = lg[e];
            if (bi < 0 || v > bv) {
                bv = v;
                bi = e;
            }
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            const float ov = __shfl_xor(bv, o, 64);
            const int oi = __shfl_xor(bi, o, 64);
            if (oi >= 0 && (bi < 0 || ov > bv || (ov == bv && oi < bi))) {
                bv = ov;
                bi = oi;
            }
        }
        if ((bi & 63) == lane) taken |= 1ull << (bi >> 6);
        vals[k] = bv;
        idx[k] = bi;
    }
}

// Routing weights: softmax over the selected logits (the softmax over all E
// renormalised over the selection).
__device__ __forceinline__ void topk_weights(const float (&vals)[kMaxTopK], int K, float (&w)[kMaxTopK])
{
    float z = 0.f;
#pragma unroll
    for (int k = 0; k < kMaxTopK; ++k)
        if (k < K) z += expf(vals[k] - vals[0]);
#pragma unroll
    for (int k = 0; k < kMaxTopK; ++k) w[k] = k < K ? expf(vals[k] - vals[0]) / z : 0.f;
}

// The order of fp32 logits as unsigned keys: a larger key is a larger
// value; -0 and +0 map to the same key (they tie, and the lower index wins,
// as for any other equal values).  0 is below every real key.
__device__ __forceinline__ uint32_t order_key(uint32_t u)
{
    u = u == 0x80000000u ? 0u : u;
    const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return o ? o : 1u;
}
__device__ __forceinline__ float order_value(uint32_t o)
{
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

// Routing candidates as 64-bit keys: order_key of the logit (high word), the
// complement of the expert index (low word).  A larger key is a larger
// logit, then the lower index.
__device__ __forceinline__ uint64_t route_key(float v, int e)
{
    return ((uint64_t)order_key(__float_as_uint(v)) << 32) | (uint32_t)~(uint32_t)e;
}
__device__ __forceinline__ float key_value(uint64_t k) { return order_value((uint32_t)(k >> 32)); }
__device__ __forceinline__ int key_index(uint64_t k) { return (int)~(uint32_t)k; }

template <int CTRL, int ROWS>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v)
{
    const uint32_t lo = __builtin_amdgcn_update_dpp(0u, (uint32_t)v, CTRL, ROWS, 0xF, false);
    const uint32_t hi = __builtin_amdgcn_update_dpp(0u, (uint32_t)(v >> 32), CTRL, ROWS, 0xF, false);
    return ((uint64_t)hi << 32) | lo;
}

// Largest key of a full wave, returned in every lane: DPP inside rows of
// 16, then the row broadcasts (row 15 -> rows 1 and 3, row 31 -> rows 2 and
// 3) leave the maximum in lane 63.
__device__ __forceinline__ uint64_t wave_max_key(uint64_t k)
{
    uint64_t o;
    o = dpp_u64<0xB1, 0xF>(k);   // quad_perm [1,0,3,2]
    k = o > k ? o : k;
    o = dpp_u64<0x4E, 0xF>(k);   // quad_perm [2,3,0,1]
    k = o > k ? o : k;
    o = dpp_u64<0x141, 0xF>(k);  // row_half_mirror
    k = o > k ? o : k;
    o = dpp_u64<0x140, 0xF>(k);  // row_mirror
    k = o > k ? o : k;
    o = dpp_u64<0x142, 0xA>(k);  // row_bcast:15 into rows 1, 3
    k = o > k ? o : k;
    o = dpp_u64<0x143, 0xC>(k);  // row_bcast:31 into rows 2, 3
    k = o > k ? o : k;
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)k, 63);
    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(k >> 32), 63);
    return ((uint64_t)hi << 32) | lo;
}

// Wave-wide maximum / minimum of an unsigned value (DPP inside rows of 16,
// then the four row results as scalars), returned in every lane.
__device__ __forceinline__ uint32_t udpp_max(uint32_t v)
{
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));
    return max(max((uint32_t)__builtin_amdgcn_readlane((int)v, 0), (uint32_t)__builtin_amdgcn_readlane((int)v, 16)),
               max((uint32_t)__builtin_amdgcn_readlane((int)v, 32), (uint32_t)__builtin_amdgcn_readlane((int)v, 48)));
}
__device__ __forceinline__ uint32_t udpp_min(uint32_t v)
{
    v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0xB1, 0xF, 0xF, false));
    v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0x4E, 0xF, 0xF, false));
    v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0x141, 0xF, 0xF, false));
    v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0x140, 0xF, 0xF, false));
    return min(min((uint32_t)__builtin_amdgcn_readlane((int)v, 0), (uint32_t)__builtin_amdgcn_readlane((int)v, 16)),
               min((uint32_t)__builtin_amdgcn_readlane((int)v, 32), (uint32_t)__builtin_amdgcn_readlane((int)v, 48)));
}

// Wait until wave_topk_global has published index k of the selection
// (rdy[k] == tag, LDS); bounded like the grid barrier.
__device__ __forceinline__ void wait_selected(const int *rdy, int k, int tag, uint32_t *flags)
{
    uint32_t spins = 0;
    while (__hip_atomic_load(rdy + k, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) != tag) {
        __builtin_amdgcn_s_sleep(1);
        if (++spins == kSpinLimit) {
            atomicOr(flags, MOE_DEVERR_BARRIER_TIMEOUT);
            break;
        }
    }
}

// Top K of E logits (E <= 64 * KPL) by one wave, from order keys: lane l
// holds ord[j] = order_key of element l + 64 j (0: no element).  Order: the
// larger key, then the lower index.  Each lane keeps its best element (the
// lowest j on equal keys); a round takes the wave's largest key, the lowest
// index among the lanes holding it, and that lane moves to its next best.
// sel/selw (LDS) receive the indices in rank order and the routing weights
// (lanes k < K write).  Each index is published as soon as its round ends:
// sel[k] is written, then rdy[k] = tag (LDS), so that other waves can start
// on slot k before the later rounds finish.
template <int KPL>
__device__ __forceinline__ void topk_select(uint32_t (&ord)[KPL], int K, int *sel, float *selw, int *rdy, int tag,
                                            int lane)
{
    uint32_t bo = 0u;
    int bj = 0;
#pragma unroll
    for (int j = 0; j < KPL; ++j)
        if (ord[j] > bo) {
            bo = ord[j];
            bj = j;
        }
    int idx[kMaxTopK];
    float vals[kMaxTopK];
#pragma unroll
    for (int k = 0; k < kMaxTopK; ++k) {
        idx[k] = 0;
        vals[k] = -INFINITY;
        if (k >= K) continue;
        const uint32_t m = udpp_max(bo);
        const uint64_t cand = __ballot(bo == m);
        int e;
        if (__popcll(cand) == 1) {
            const int wl = __builtin_ctzll(cand);
            e = __builtin_amdgcn_readlane(bj, wl) * 64 + wl;
        } else {
            e = (int)udpp_min(bo == m ? (uint32_t)(bj * 64 + lane) : 0xFFFFFFFFu);
        }
        idx[k] = e;
        vals[k] = order_value(m);
        if (lane == 0) {
            __hip_atomic_store(sel + k, e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            __hip_atomic_store(rdy + k, tag, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
        if (lane == (e & 63)) {
            const int jw = e >> 6;
#pragma unroll
            for (int j = 0; j < KPL; ++j)
                if (j == jw) ord[j] = 0u;
            bo = 0u;
            bj = 0;
#pragma unroll
            for (int j = 0; j < KPL; ++j)
                if (ord[j] > bo) {
                    bo = ord[j];
                    bj = j;
                }
        }
    }
    // routing weights: softmax over the selected logits, lane k < K taking
    // selection k (one exp per lane), the sum in rank order
    float mv = vals[0];
#pragma unroll
    for (int k = 0; k < kMaxTopK; ++k)
        if (lane == k) mv = vals[k];
    const float ex = lane < K ? expf(mv - vals[0]) : 0.f;
    float z = 0.f;
#pragma unroll
    for (int k = 0; k < kMaxTopK; ++k)
        if (k < K) z += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ex), k));
    if (lane < K) selw[lane] = ex / z;
}

// topk_select over the tagged logits of a persistent launch (agent-coherent
// loads, lane l holding elements l + 64 j; the wave polls until every logit
// carries epoch `ltag`).
template <int KPL>
__device__ __forceinline__ void wave_topk_global(const uint64_t *tlog, uint32_t ltag, int E, int K, int *sel,
                                                 float *selw, int *rdy, int tag, int lane, uint32_t *flags)
{
    // every load in flight before the first use (clamped indices, masked
    // afterwards)
    uint32_t ord[KPL];
    for (uint32_t spins = 0;;) {
        bool ok = true;
#pragma unroll
        for (int j = 0; j < KPL; ++j) {
            const uint64_t w = __hip_atomic_load(tlog + min(lane + 64 * j, E - 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            ord[j] = (uint32_t)w;
            ok &= (uint32_t)(w >> 32) == ltag;
        }
        if (__all(ok)) break;
        __builtin_amdgcn_s_sleep(1);
        if (++spins == (1u << 16)) {
            atomicOr(flags, MOE_DEVERR_BARRIER_TIMEOUT);
            break;
        }
    }
#pragma unroll
    for (int j = 0; j < KPL; ++j) ord[j] = lane + 64 * j < E ? order_key(ord[j]) : 0u;
    topk_select<KPL>(ord, K, sel, selw, rdy, tag, lane);
}

}  // namespace dev
}  // namespace moe
