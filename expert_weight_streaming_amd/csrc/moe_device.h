// moe_device.h -- device building blocks shared by libmoe's kernels.
//
// Dequantisation follows the affine form w = q*scale + bias with one bf16
// scale/bias pair per group of 64 inputs (toolarium.ru, "Оптимизации,
// которые сработали").  The FMA rewrite fma(q, scale*x, bias*x) is applied
// per group instead of per weight: sum_j (q_j*s + b) x_j = s*sum_j q_j x_j +
// b*sum_j x_j, so each weight costs one code->float conversion and one FMA
// and the bias term is paid once per group from a per-lane sum of x.
#pragma once
#include "moe_internal.h"

namespace moe {
namespace dev {

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Sum over groups of W consecutive lanes (W a power of two <= 64).
template <int W>
__device__ __forceinline__ float group_sum(float v)
{
#pragma unroll
    for (int o = W / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// sum over one 16-byte chunk of 4-bit codes (32 codes) of code * x[code].
// Word k holds codes 8k..8k+7, code n at bits 4n..4n+3.  Masking with
// 0x0F0F0F0F leaves the even codes in the four bytes, the shifted copy the
// odd ones, so every code converts with one byte->float conversion.
__device__ __forceinline__ float qdot4(const uint4 q, const float *x)
{
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t lo = w[k] & 0x0F0F0F0Fu, hi = (w[k] >> 4) & 0x0F0F0F0Fu;
        const float *xx = x + 8 * k;
        a0 = fmaf((float)(lo & 0xFFu), xx[0], a0);
        a1 = fmaf((float)(hi & 0xFFu), xx[1], a1);
        a0 = fmaf((float)((lo >> 8) & 0xFFu), xx[2], a0);
        a1 = fmaf((float)((hi >> 8) & 0xFFu), xx[3], a1);
        a0 = fmaf((float)((lo >> 16) & 0xFFu), xx[4], a0);
        a1 = fmaf((float)((hi >> 16) & 0xFFu), xx[5], a1);
        a0 = fmaf((float)(lo >> 24), xx[6], a0);
        a1 = fmaf((float)(hi >> 24), xx[7], a1);
    }
    return a0 + a1;
}

// Same for 2-bit codes (64 codes per chunk): word k holds codes
// 16k..16k+15, code n at bits 2n; byte j of (w >> 2p) & 0x03030303 is
// code 4j + p.
__device__ __forceinline__ float qdot2(const uint4 q, const float *x)
{
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const float *xx = x + 16 * k;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const uint32_t m = (w[k] >> (2 * p)) & 0x03030303u;
            a0 = fmaf((float)(m & 0xFFu), xx[p], a0);
            a1 = fmaf((float)((m >> 8) & 0xFFu), xx[4 + p], a1);
            a0 = fmaf((float)((m >> 16) & 0xFFu), xx[8 + p], a0);
            a1 = fmaf((float)(m >> 24), xx[12 + p], a1);
        }
    }
    return a0 + a1;
}

template <int BITS>
__device__ __forceinline__ float qdot(const uint4 q, const float *x)
{
    if constexpr (BITS == 4) return qdot4(q, x);
    else return qdot2(q, x);
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

// One wave: dot of router row `row` (D fp32) with x; x may live in LDS.
// Returns the full sum in every lane.
__device__ __forceinline__ float wave_router_row(const float *row, const float *x, int D, int lane)
{
    const float4 *W = reinterpret_cast<const float4 *>(row);
    const float4 *X = reinterpret_cast<const float4 *>(x);
    const int nc = D / 4;
    float acc0 = 0.f, acc1 = 0.f;
    int c = lane;
    for (; c + 192 < nc; c += 256) {
        const float4 w0 = W[c], w1 = W[c + 64], w2 = W[c + 128], w3 = W[c + 192];
        const float4 x0 = X[c], x1 = X[c + 64], x2 = X[c + 128], x3 = X[c + 192];
        acc0 = fmaf(w0.x, x0.x, acc0); acc1 = fmaf(w0.y, x0.y, acc1);
        acc0 = fmaf(w0.z, x0.z, acc0); acc1 = fmaf(w0.w, x0.w, acc1);
        acc0 = fmaf(w1.x, x1.x, acc0); acc1 = fmaf(w1.y, x1.y, acc1);
        acc0 = fmaf(w1.z, x1.z, acc0); acc1 = fmaf(w1.w, x1.w, acc1);
        acc0 = fmaf(w2.x, x2.x, acc0); acc1 = fmaf(w2.y, x2.y, acc1);
        acc0 = fmaf(w2.z, x2.z, acc0); acc1 = fmaf(w2.w, x2.w, acc1);
        acc0 = fmaf(w3.x, x3.x, acc0); acc1 = fmaf(w3.y, x3.y, acc1);
        acc0 = fmaf(w3.z, x3.z, acc0); acc1 = fmaf(w3.w, x3.w, acc1);
    }
    for (; c < nc; c += 64) {
        const float4 w0 = W[c], x0 = X[c];
        acc0 = fmaf(w0.x, x0.x, acc0); acc1 = fmaf(w0.y, x0.y, acc1);
        acc0 = fmaf(w0.z, x0.z, acc0); acc1 = fmaf(w0.w, x0.w, acc1);
    }
    return group_sum<64>(acc0 + acc1);
}

// One wave: R consecutive intermediate rows i0.. of one expert's gate and up
// matrices; lane l owns 16-byte chunks l, l+64, ... of every row, so each
// slice of x (and the slice's sum) serves all R rows.  All weight loads are
// issued first; the x slices are then walked one chunk at a time.  Writes
// h[i] = silu(g_i) * u_i, silu(z) = z / (1 + exp(-z)).
template <int BITS, int CPL, int R>
__device__ __forceinline__ void wave_gate_up(const uint8_t *blob, const float *x, int D, int I, int i0, int lane, float *h)
{
    constexpr int CODES = 128 / BITS;
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
                                         blob + sb0 + mat * mat_sb + ((uint64_t)i * gpr + (uint64_t)c * CODES / kGroup) * 4)
                                   : 0u;
            }

    float acc[R][2];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r][0] = acc[r][1] = 0.f;
#pragma unroll
    for (int m = 0; m < CPL; ++m) {
        const int c = lane + 64 * m;
        float xv[CODES];
        float xs = 0.f;
#pragma unroll
        for (int j = 0; j < CODES; j += 4) {
            float4 v = c < nchunks ? *reinterpret_cast<const float4 *>(x + c * CODES + j) : make_float4(0.f, 0.f, 0.f, 0.f);
            xv[j] = v.x;
            xv[j + 1] = v.y;
            xv[j + 2] = v.z;
            xv[j + 3] = v.w;
            xs += (v.x + v.y) + (v.z + v.w);
        }
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int mat = 0; mat < 2; ++mat) {
                const float qx = qdot<BITS>(q[m][r][mat], xv);
                acc[r][mat] = fmaf(bf16_lo(sb[m][r][mat]), qx, acc[r][mat]);
                acc[r][mat] = fmaf(bf16_hi(sb[m][r][mat]), xs, acc[r][mat]);
            }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const float g = group_sum<64>(acc[r][0]);
        const float u = group_sum<64>(acc[r][1]);
        const int i = i0 + r;
        if (lane == 0 && i < I) h[i] = g / (1.f + expf(-g)) * u;
    }
}

// One wave: STEPS x (64/LPR) consecutive rows o0.. of one expert's down
// matrix times h; LPR lanes per row, a lane's slice of h serving every row
// it visits.  out[s] (valid in lanes with lane % LPR == 0) is row
// o0 + s*(64/LPR) + lane/LPR.
template <int BITS, int LPR, int CPL, int STEPS>
__device__ __forceinline__ void wave_down(const uint8_t *blob, const float *h, int D, int I, int o0, int lane, float *out)
{
    constexpr int CODES = 128 / BITS;
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
            sb[m][s] = ok ? *reinterpret_cast<const uint32_t *>(blob + sbd + ((uint64_t)o * gpr + (uint64_t)c * CODES / kGroup) * 4)
                          : 0u;
        }

    float t[STEPS];
#pragma unroll
    for (int s = 0; s < STEPS; ++s) t[s] = 0.f;
#pragma unroll
    for (int m = 0; m < CPL; ++m) {
        const int c = lc + LPR * m;
        const bool ok = blob && c < nchunks;
        float hv[CODES];
        float hs = 0.f;
#pragma unroll
        for (int j = 0; j < CODES; j += 4) {
            float4 v = ok ? *reinterpret_cast<const float4 *>(h + c * CODES + j) : make_float4(0.f, 0.f, 0.f, 0.f);
            hv[j] = v.x;
            hv[j + 1] = v.y;
            hv[j + 2] = v.z;
            hv[j + 3] = v.w;
            hs += (v.x + v.y) + (v.z + v.w);
        }
#pragma unroll
        for (int s = 0; s < STEPS; ++s) {
            const float qh = qdot<BITS>(q[m][s], hv);
            t[s] = fmaf(bf16_lo(sb[m][s]), qh, t[s]);
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
