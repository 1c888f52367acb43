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
// int32).  Per 16-byte chunk the three plane sums are combined once in fp32
// and scaled by 2^-k * scale.  Apart from the fixed-point rounding of x
// (half a unit of 2^-k, about 1e-7 of the vector's largest element) the sum
// is exact.  Cost: 4-bit about 1.4 VALU operations per weight, 2-bit about
// 1.3, against about 3 for a float conversion and an FMA per weight.
#pragma once
#include "moe_internal.h"

namespace moe {
namespace dev {

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Sum / max over groups of W consecutive lanes (W a power of two <= 64).
template <int W>
__device__ __forceinline__ float group_sum(float v)
{
#pragma unroll
    for (int o = W / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}
template <int W>
__device__ __forceinline__ float group_max(float v)
{
#pragma unroll
    for (int o = W / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
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
    static constexpr int DW = 4 * SUBS * 3;        // digit words per chunk
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

// The three signed base-256 digits of round(v * mul), each in [-128, 127].
__device__ __forceinline__ void digits3(float v, float mul, int &d0, int &d1, int &d2)
{
    const int xi = __float2int_rn(v * mul);
    d0 = ((xi + 128) & 255) - 128;
    const int x1 = (xi - d0) >> 8;
    d1 = ((x1 + 128) & 255) - 128;
    d2 = (x1 - d1) >> 8;
}

__device__ __forceinline__ int pack4(int a, int b, int c, int d)
{
    return (a & 255) | ((b & 255) << 8) | ((c & 255) << 16) | (int)((uint32_t)d << 24);
}

// Digit words of word k, sub s of one chunk from the chunk's activations
// v[0..CODES): plane p of (k, s) holds, byte j, the digit of v[k*PER_WORD +
// s + SUBS*j].  dg index: (k*SUBS + s)*3 + p.
template <int BITS>
__device__ __forceinline__ void chunk_digits(const float *v, float mul, int *dg)
{
    using C = Codes<BITS>;
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int s = 0; s < C::SUBS; ++s) {
            int d[4][3];
#pragma unroll
            for (int j = 0; j < 4; ++j) digits3(v[k * C::PER_WORD + s + C::SUBS * j], mul, d[j][0], d[j][1], d[j][2]);
#pragma unroll
            for (int p = 0; p < 3; ++p) dg[(k * C::SUBS + s) * 3 + p] = pack4(d[0][p], d[1][p], d[2][p], d[3][p]);
        }
}

// sum over one chunk of code * x_int, from the chunk's digit words; exact
// in int32 per plane, combined in fp32.
template <int BITS>
__device__ __forceinline__ float qdot(const uint4 q, const int *dg)
{
    using C = Codes<BITS>;
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
    int a0 = 0, a1 = 0, a2 = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int s = 0; s < C::SUBS; ++s) {
            const int m = (int)((w[k] >> (BITS * s)) & C::MASK);
            const int *d = dg + (k * C::SUBS + s) * 3;
            a0 = __builtin_amdgcn_sdot4(m, d[0], a0, false);
            a1 = __builtin_amdgcn_sdot4(m, d[1], a1, false);
            a2 = __builtin_amdgcn_sdot4(m, d[2], a2, false);
        }
    return fmaf((float)a2, 65536.f, fmaf((float)a1, 256.f, (float)a0));
}

// Block-cooperative fixed-point digit table of an activation vector x[0..n)
// (n a multiple of the chunk width): dig[c*DW + ...] as chunk_digits lays
// out chunk c, csum[c] = sum of the chunk's fp32 values; returns 2^-k.
// `red` is LDS scratch of 16 floats.  Ends with __syncthreads.
template <int BITS>
__device__ __forceinline__ float block_digit_table(const float *x, int n, int *dig, float *csum, float *red)
{
    using C = Codes<BITS>;
    const int tid = threadIdx.x, nt = blockDim.x;
    float m = 0.f;
    for (int i = tid; i < n; i += nt) m = fmaxf(m, fabsf(x[i]));
    m = group_max<64>(m);
    if ((tid & 63) == 0) red[tid >> 6] = m;
    __syncthreads();
    float amax = 0.f;
    for (int w = 0; w < (nt >> 6); ++w) amax = fmaxf(amax, red[w]);
    float mul, inv;
    fixed_scale(amax, mul, inv);
    // one thread per (chunk, word, sub): four activations -> three words
    const int nwords = n / C::CODES * 4 * C::SUBS;
    for (int t = tid; t < nwords; t += nt) {
        const int c = t / (4 * C::SUBS), r = t - c * 4 * C::SUBS;
        const int k = r / C::SUBS, s = r - k * C::SUBS;
        const float *v = x + c * C::CODES + k * C::PER_WORD + s;
        int d[4][3];
#pragma unroll
        for (int j = 0; j < 4; ++j) digits3(v[C::SUBS * j], mul, d[j][0], d[j][1], d[j][2]);
        int *o = dig + c * C::DW + (k * C::SUBS + s) * 3;
#pragma unroll
        for (int p = 0; p < 3; ++p) o[p] = pack4(d[0][p], d[1][p], d[2][p], d[3][p]);
    }
    for (int c = tid; c < n / C::CODES; c += nt) {
        float sum = 0.f;
        for (int j = 0; j < C::CODES; ++j) sum += x[c * C::CODES + j];
        csum[c] = sum;
    }
    __syncthreads();
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

// One wave: R consecutive intermediate rows i0.. of one expert's gate and up
// matrices; lane l owns 16-byte chunks l, l+64, ... of every row.  The
// activation arrives as a digit table (block_digit_table, in LDS) with its
// per-chunk sums and fixed-point step inv.  All weight loads are issued
// first.  Writes h[i] = silu(g_i) * u_i, silu(z) = z / (1 + exp(-z)).
template <int BITS, int CPL, int R>
__device__ __forceinline__ void wave_gate_up(const uint8_t *blob, const int *dig, const float *csum, float inv, int D,
                                             int I, int i0, int lane, float *h)
{
    using C = Codes<BITS>;
    const int nchunks = D * BITS / 128;
    const uint64_t mat_q = (uint64_t)I * D * BITS / 8;
    const uint64_t row_q = (uint64_t)D * BITS / 8;
    const uint64_t sb0 = 3 * mat_q;
    const uint64_t mat_sb = (uint64_t)I * (D / kGroup) * 4;
    const int gpr = D / kGroup;

    uint4 q[CPL][R][2];
    uint32_t sb[CPL][R][2];
#pragma unroll
    for (int m = 0; m < CPL; ++m)
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int mat = 0; mat < 2; ++mat) {
                const int i = i0 + r, c = lane + 64 * m;
                const bool ok = i < I && c < nchunks;
                q[m][r][mat] = ok ? *reinterpret_cast<const uint4 *>(blob + mat * mat_q + (uint64_t)i * row_q + (uint64_t)c * 16)
                                  : make_uint4(0, 0, 0, 0);
                sb[m][r][mat] = ok ? *reinterpret_cast<const uint32_t *>(
                                         blob + sb0 + mat * mat_sb + ((uint64_t)i * gpr + (uint64_t)c * C::CODES / kGroup) * 4)
                                   : 0u;
            }

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
                const float qx = qdot<BITS>(q[m][r][mat], dg);
                acc[r][mat] = fmaf(bf16_lo(sb[m][r][mat]) * inv, qx, acc[r][mat]);
                acc[r][mat] = fmaf(bf16_hi(sb[m][r][mat]), cs, acc[r][mat]);
            }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const float g = group_sum<64>(acc[r][0]);
        const float u = group_sum<64>(acc[r][1]);
        const int i = i0 + r;
        if (lane == 0 && i < I) xstore(h + i, g / (1.f + expf(-g)) * u);
    }
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

}  // namespace dev
}  // namespace moe
