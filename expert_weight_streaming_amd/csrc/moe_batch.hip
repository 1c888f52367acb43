// moe_batch.hip -- the MoE block for a batch of T > 1 tokens.
//
// Batching must not change the arithmetic of a token (the pages run one
// token at a time, hakusoku.com "パイプライン概要"); what it changes is how
// often an expert's weights are read.  Tokens are grouped by expert so that
// every selected expert's rows are fetched once per step and applied to all
// of that expert's tokens:
//
//   k_route_b      logits[t][e] for all tokens (each router row read once)
//   k_topk_group   per-token top-K and softmax weights, then the grouping:
//                  count[e], offset[e] (exclusive prefix sum), the pair
//                  permutation perm[pos] = t*K + k sorted by (expert, pair
//                  index), its inverse, and the list of active experts
//   k_digits       fixed-point digit tables of the tokens' activations
//   k_gate_up_b    per active expert (and the shared expert, all tokens):
//                  gate/up rows x that expert's tokens, SwiGLU -> h[pos]
//   k_digits       digit tables of h
//   k_down_b       per active expert: down rows x its tokens' h -> y[pos]
//   k_combine_b    per token, in slot order: sum_k w_k y[pos(t,k)] + the
//                  shared expert's y, then (layer mode) residual + RMSNorm
//
// Every step is deterministic (no float atomics, fixed summation orders).
#include "moe_device.h"

namespace moe {
namespace {

using namespace dev;

// ---------------------------------------------------------------------------
// Router for T tokens: one row per wave, 4 rows per block; the tokens'
// activations pass through LDS in 256-column slices.
template <int TT>
__global__ void __launch_bounds__(256) k_route_b(BatchArgs a)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int row = blockIdx.x * 4 + wave;
    constexpr int CH = 256;
    __shared__ __align__(16) float xs[TT][CH];
    float acc[TT];
#pragma unroll
    for (int t = 0; t < TT; ++t) acc[t] = 0.f;
    for (int t0 = 0; t0 < a.T; t0 += TT) {
#pragma unroll
        for (int t = 0; t < TT; ++t) acc[t] = 0.f;
        for (int c0 = 0; c0 < a.D; c0 += CH) {
            __syncthreads();
            for (int i = tid; i < TT * CH; i += 256) {
                const int t = i / CH, c = i - t * CH;
                xs[t][c] = (t0 + t < a.T && c0 + c < a.D) ? a.x[(size_t)(t0 + t) * a.D + c0 + c] : 0.f;
            }
            __syncthreads();
            if (row < a.E && c0 + 4 * lane < a.D) {
                const float4 w = *reinterpret_cast<const float4 *>(a.router + (size_t)row * a.D + c0 + 4 * lane);
#pragma unroll
                for (int t = 0; t < TT; ++t) {
                    const float4 v = *reinterpret_cast<const float4 *>(&xs[t][4 * lane]);
                    acc[t] = fmaf(w.x, v.x, fmaf(w.y, v.y, fmaf(w.z, v.z, fmaf(w.w, v.w, acc[t]))));
                }
            }
        }
#pragma unroll
        for (int t = 0; t < TT; ++t) {
            const float v = group_sum<64>(acc[t]);
            if (lane == 0 && row < a.E && t0 + t < a.T) a.logits[(size_t)(t0 + t) * a.E + row] = v;
        }
    }
}

// ---------------------------------------------------------------------------
// One block of 1024 threads: top-K of every token (unless the routing is
// given), then the token -> expert grouping.
__global__ void __launch_bounds__(1024) k_topk_group(BatchArgs a, int do_topk)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int T = a.T, K = a.K, E = a.E, P = T * K;
    __shared__ float lg[16][512];
    __shared__ int s_idx[64 * kMaxTopK];
    __shared__ int s_count[4096];
    __shared__ int s_off[4097];

    if (do_topk) {
        for (int t = wave; t < T; t += 16) {
            // logits of token t, 512 at a time into this wave's LDS row
            int idx[kMaxTopK];
            float vals[kMaxTopK];
            // top-K over E in slices: keep the running best K (merge by repeated selection)
            float bestv[kMaxTopK];
            int besti[kMaxTopK];
#pragma unroll
            for (int k = 0; k < kMaxTopK; ++k) {
                bestv[k] = -INFINITY;
                besti[k] = -1;
            }
            for (int e0 = 0; e0 < E; e0 += 512) {
                const int n = E - e0 < 512 ? E - e0 : 512;
                for (int e = lane; e < n; e += 64) lg[wave][e] = a.logits[(size_t)t * E + e0 + e];
                __builtin_amdgcn_s_waitcnt(0);
                __builtin_amdgcn_wave_barrier();
                wave_topk(lg[wave], n, K, lane, idx, vals);
                // merge this slice's K with the running K: both sorted descending
                float mv[kMaxTopK];
                int mi[kMaxTopK];
                int p = 0, q = 0;
#pragma unroll
                for (int k = 0; k < kMaxTopK; ++k) {
                    if (k >= K) {
                        mv[k] = -INFINITY;
                        mi[k] = -1;
                        continue;
                    }
                    const int gi = idx[q] < 0 ? -1 : idx[q] + e0;
                    // running entries have lower indices than this slice's: ties keep them first
                    const bool take_run = besti[p] >= 0 && (gi < 0 || bestv[p] >= vals[q]);
                    mv[k] = take_run ? bestv[p] : vals[q];
                    mi[k] = take_run ? besti[p] : gi;
                    if (take_run) ++p;
                    else ++q;
                }
#pragma unroll
                for (int k = 0; k < kMaxTopK; ++k) {
                    bestv[k] = mv[k];
                    besti[k] = mi[k];
                }
                __builtin_amdgcn_wave_barrier();
            }
            float w[kMaxTopK];
            topk_weights(bestv, K, w);
            if (lane == 0) {
#pragma unroll
                for (int k = 0; k < kMaxTopK; ++k) {
                    if (k >= K) continue;
                    a.topk_idx[(size_t)t * K + k] = besti[k];
                    a.topk_w[(size_t)t * K + k] = w[k];
                }
            }
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }
    for (int p = tid; p < P; p += 1024) s_idx[p] = a.topk_idx[p];
    for (int e = tid; e < E; e += 1024) s_count[e] = 0;
    __syncthreads();
    for (int p = tid; p < P; p += 1024) {
        const int e = s_idx[p];
        if (e >= 0 && e < E) atomicAdd(&s_count[e], 1);
        else atomicOr(a.flags, MOE_DEVERR_EXPERT_RANGE);
    }
    __syncthreads();
    if (tid == 0) {
        int run = 0, nact = 0;
        for (int e = 0; e < E; ++e) {
            s_off[e] = run;
            a.offset[e] = run;
            a.count[e] = s_count[e];
            if (s_count[e]) a.act[nact++] = e;
            run += s_count[e];
        }
        s_off[E] = run;
        a.offset[E] = run;
        *a.n_act = nact;
    }
    __syncthreads();
    for (int p = tid; p < P; p += 1024) {
        const int e = s_idx[p];
        if (e < 0 || e >= E) {
            a.pos_of_pair[p] = -1;
            continue;
        }
        int rank = 0;
        for (int q = 0; q < p; ++q) rank += s_idx[q] == e;
        const int pos = s_off[e] + rank;
        a.perm[pos] = p;
        a.pos_of_pair[p] = pos;
    }
}

// ---------------------------------------------------------------------------
// Digit tables of n vectors of length len (one block per vector).
template <int BITS>
__global__ void __launch_bounds__(256) k_digits(const float *v, int len, int *dig, float *csum, float *inv, int dig_stride,
                                                 int csum_stride)
{
    __shared__ float red[16];
    const int b = blockIdx.x;
    const float r = block_digit_table<BITS>(v + (size_t)b * len, len, dig + (size_t)b * dig_stride,
                                            csum + (size_t)b * csum_stride, red);
    if (threadIdx.x == 0) inv[b] = r;
}

// Experts with at least this many tokens in a step take the matrix-core
// kernels (k_gate_up_m, k_down_m), the others the dot-product kernels.
constexpr int kMfmaMin = 8;

// Tokens of active item a: routed expert act[a] (positions offset..+count),
// or, for a == n_act, the shared expert (positions T*K .. T*K+T-1, token j).
struct Item {
    const uint8_t *blob;
    int pos0, n;
    int slot;  // 0: routed, 1: shared
};

__device__ __forceinline__ Item item_of(const BatchArgs &a, int it, int nact)
{
    Item r;
    if (it < nact) {
        const int e = a.act[it];
        r.blob = a.src.experts + (uint64_t)e * a.src.blob_bytes;
        r.pos0 = a.offset[e];
        r.n = a.count[e];
        r.slot = 0;
    } else {
        r.blob = a.src.shared;
        r.pos0 = a.T * a.K;
        r.n = a.T;
        r.slot = 1;
    }
    return r;
}

__device__ __forceinline__ int token_of(const BatchArgs &a, const Item &it, int j)
{
    return it.slot ? j : a.perm[it.pos0 + j] / a.K;
}

// ---------------------------------------------------------------------------
// Grouped gate/up: wave units of R intermediate rows of one item, applied to
// every token of the item.
template <int BITS, int CPL, int R>
__global__ void __launch_bounds__(256) k_gate_up_b(BatchArgs a)
{
    using C = Codes<BITS>;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int D = a.D, I = a.I;
    const int nact = *a.n_act;
    const int items = nact + (a.src.n_slots > a.src.top_k ? 1 : 0);
    const int upi = (I + R - 1) / R;
    const int nchunks = D * BITS / 128;
    const int xdw = nchunks * C::DW, xcs = nchunks;
    const uint64_t mat_q = (uint64_t)I * D * BITS / 8;
    const uint64_t row_q = (uint64_t)D * BITS / 8;
    const uint64_t sb0 = 3 * mat_q;
    const uint64_t mat_sb = (uint64_t)I * (D / kGroup) * 4;
    const int gpr = D / kGroup;
    for (int u = blockIdx.x * 4 + wave; u < items * upi; u += gridDim.x * 4) {
        const int ii = u / upi, i0 = (u - ii * upi) * R;
        const Item it = item_of(a, ii, nact);
        if (it.n >= kMfmaMin) continue;  // taken by the matrix-core kernel
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
                    q[m][r][mat] = ok ? *reinterpret_cast<const uint4 *>(it.blob + mat * mat_q + (uint64_t)i * row_q +
                                                                         (uint64_t)c * 16)
                                      : make_uint4(0, 0, 0, 0);
                    sb[m][r][mat] = ok ? *reinterpret_cast<const uint32_t *>(it.blob + sb0 + mat * mat_sb +
                                                                             ((uint64_t)i * gpr + (uint64_t)c * C::CODES / kGroup) * 4)
                                       : 0u;
                }
        for (int j = 0; j < it.n; ++j) {
            const int t = token_of(a, it, j);
            const float inv = a.xinv[t];
            float acc[R][2];
#pragma unroll
            for (int r = 0; r < R; ++r) acc[r][0] = acc[r][1] = 0.f;
#pragma unroll
            for (int m = 0; m < CPL; ++m) {
                const int c = lane + 64 * m;
                int dg[C::DW];
                float cs = 0.f;
                if (c < nchunks) {
                    const int4 *src = reinterpret_cast<const int4 *>(a.xdig + (size_t)t * xdw + c * C::DW);
#pragma unroll
                    for (int v = 0; v < C::DW / 4; ++v) {
                        const int4 w = src[v];
                        dg[4 * v] = w.x;
                        dg[4 * v + 1] = w.y;
                        dg[4 * v + 2] = w.z;
                        dg[4 * v + 3] = w.w;
                    }
                    cs = a.xcsum[(size_t)t * xcs + c];
                } else {
#pragma unroll
                    for (int v = 0; v < C::DW; ++v) dg[v] = 0;
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
                const float uu = group_sum<64>(acc[r][1]);
                const int i = i0 + r;
                if (lane == 0 && i < I) a.h[(size_t)(it.pos0 + j) * I + i] = g / (1.f + expf(-g)) * uu;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Grouped down: wave units of STEPS x (64/LPR) output rows of one item,
// applied to every token of the item (digits of that token's h).
template <int BITS, int LPR, int CPL, int STEPS>
__global__ void __launch_bounds__(256) k_down_b(BatchArgs a)
{
    using C = Codes<BITS>;
    constexpr int RPS = 64 / LPR;
    constexpr int RW = RPS * STEPS;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int D = a.D, I = a.I;
    const int nact = *a.n_act;
    const int items = nact + (a.src.n_slots > a.src.top_k ? 1 : 0);
    const int upi = (D + RW - 1) / RW;
    const int nchunks = I * BITS / 128;
    const int hdw = nchunks * C::DW;
    const int sub = lane / LPR, lc = lane % LPR;
    const uint64_t mat_q = (uint64_t)I * D * BITS / 8;
    const uint64_t row_q = (uint64_t)I * BITS / 8;
    const uint64_t sbd = 3 * mat_q + 2 * ((uint64_t)D * (I / kGroup) * 4);
    const int gpr = I / kGroup;
    for (int u = blockIdx.x * 4 + wave; u < items * upi; u += gridDim.x * 4) {
        const int ii = u / upi, o0 = (u - ii * upi) * RW;
        const Item it = item_of(a, ii, nact);
        if (it.n >= kMfmaMin) continue;  // taken by the matrix-core kernel
        uint4 q[CPL][STEPS];
        uint32_t sb[CPL][STEPS];
#pragma unroll
        for (int m = 0; m < CPL; ++m)
#pragma unroll
            for (int s = 0; s < STEPS; ++s) {
                const int o = o0 + s * RPS + sub, c = lc + LPR * m;
                const bool ok = o < D && c < nchunks;
                q[m][s] = ok ? *reinterpret_cast<const uint4 *>(it.blob + 2 * mat_q + (uint64_t)o * row_q + (uint64_t)c * 16)
                             : make_uint4(0, 0, 0, 0);
                sb[m][s] = ok ? *reinterpret_cast<const uint32_t *>(it.blob + sbd +
                                                                    ((uint64_t)o * gpr + (uint64_t)c * C::CODES / kGroup) * 4)
                              : 0u;
            }
        for (int j = 0; j < it.n; ++j) {
            const int pos = it.pos0 + j;
            const float inv = a.hinv[pos];
            float t[STEPS];
#pragma unroll
            for (int s = 0; s < STEPS; ++s) t[s] = 0.f;
#pragma unroll
            for (int m = 0; m < CPL; ++m) {
                const int c = lc + LPR * m;
                int dg[C::DW];
                float cs = 0.f;
                if (c < nchunks) {
                    const int4 *src = reinterpret_cast<const int4 *>(a.hdig + (size_t)pos * hdw + c * C::DW);
#pragma unroll
                    for (int v = 0; v < C::DW / 4; ++v) {
                        const int4 w = src[v];
                        dg[4 * v] = w.x;
                        dg[4 * v + 1] = w.y;
                        dg[4 * v + 2] = w.z;
                        dg[4 * v + 3] = w.w;
                    }
                    cs = a.hcsum[(size_t)pos * nchunks + c];
                } else {
#pragma unroll
                    for (int v = 0; v < C::DW; ++v) dg[v] = 0;
                }
#pragma unroll
                for (int s = 0; s < STEPS; ++s) {
                    const float qh = qdot<BITS>(q[m][s], dg);
                    t[s] = fmaf(bf16_lo(sb[m][s]) * inv, qh, t[s]);
                    t[s] = fmaf(bf16_hi(sb[m][s]), cs, t[s]);
                }
            }
#pragma unroll
            for (int s = 0; s < STEPS; ++s) {
                const float v = group_sum<LPR>(t[s]);
                const int o = o0 + s * RPS + sub;
                if (lc == 0 && o < D) a.y[(size_t)pos * D + o] = v;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Per token: combine in slot order (routed k = 0..K-1, then shared), then
// (mode 1) residual + RMSNorm; one block per token.
__global__ void __launch_bounds__(256) k_combine_b(BatchArgs a)
{
    const int t = blockIdx.x, tid = threadIdx.x;
    const int D = a.D, K = a.K;
    __shared__ float red[16];
    __shared__ int pos[kMaxSlots];
    __shared__ float wts[kMaxSlots];
    if (tid < K) {
        pos[tid] = a.pos_of_pair[t * K + tid];
        wts[tid] = a.topk_w[t * K + tid];
    }
    __syncthreads();
    const bool has_shared = a.src.n_slots > K;
    constexpr int PER = 32;
    float rv[PER];
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int o = tid + 256 * j;
        rv[j] = 0.f;
        if (o >= D) continue;
        float c = 0.f;
        for (int k = 0; k < K; ++k)
            if (pos[k] >= 0) c += wts[k] * a.y[(size_t)pos[k] * D + o];
        if (has_shared) c += a.y[(size_t)(a.T * K + t) * D + o];
        if (a.mode == 0) {
            a.yout[(size_t)t * D + o] = c;
        } else {
            const float r = a.resid[(size_t)t * D + o] + c;
            a.resid[(size_t)t * D + o] = r;
            rv[j] = r;
            ss += r * r;
        }
    }
    if (a.mode == 0) return;
    ss = group_sum<64>(ss);
    if ((tid & 63) == 0) red[tid >> 6] = ss;
    __syncthreads();
    const float tot = (red[0] + red[1]) + (red[2] + red[3]);
    const float inv = 1.f / sqrtf(tot / (float)D + a.eps);
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int o = tid + 256 * j;
        if (o < D) a.xout[(size_t)t * D + o] = rv[j] * inv * a.gamma[o];
    }
}

// ---------------------------------------------------------------------------
// Matrix-core variants for experts with at least kMfmaMin tokens: the
// expert's weights meet its tokens as a dense contraction.  One
// v_mfma_i32_16x16x64_i8 multiplies a 16-row x 64-code tile of masked codes
// (A, one code per byte) by the tokens' 64 x 16 digits of one plane (B):
// exact int32 sums over one scale group, so the bf16 scale and bias of the
// group apply to its three plane sums exactly as in the dot-product path.
// Lane l supplies row (A) / token (B) l % 16 and the 16 codes of K-slice
// l / 16; A and B list a slice's codes in the same order (the masked-word
// order of the digit table), and the C tile arrives as rows 4 (l / 16) + r,
// token l % 16.
typedef int v4i __attribute__((ext_vector_type(4)));

// Masked codes of row `q` (the row's packed codes), scale group g, slice h.
template <int BITS>
__device__ __forceinline__ v4i mfma_a(const uint8_t *q, int g, int h)
{
    using C = Codes<BITS>;
    v4i r;
    if constexpr (BITS == 4) {
        const uint2 w = *reinterpret_cast<const uint2 *>(q + 32 * g + 8 * h);
        r[0] = (int)(w.x & C::MASK);
        r[1] = (int)((w.x >> 4) & C::MASK);
        r[2] = (int)(w.y & C::MASK);
        r[3] = (int)((w.y >> 4) & C::MASK);
    } else {
        const uint32_t w = *reinterpret_cast<const uint32_t *>(q + 16 * g + 4 * h);
        r[0] = (int)(w & C::MASK);
        r[1] = (int)((w >> 2) & C::MASK);
        r[2] = (int)((w >> 4) & C::MASK);
        r[3] = (int)((w >> 6) & C::MASK);
    }
    return r;
}

// Digit words of plane p matching mfma_a's slice h of group g, from a
// vector's digit table.
template <int BITS>
__device__ __forceinline__ v4i mfma_b(const int *dig, int g, int h, int p)
{
    using C = Codes<BITS>;
    const int4 *src;
    if constexpr (BITS == 4)
        src = reinterpret_cast<const int4 *>(dig + (2 * g + (h >> 1)) * C::DW + p * C::PW + 4 * (h & 1));
    else
        src = reinterpret_cast<const int4 *>(dig + g * C::DW + p * C::PW + 4 * h);
    const int4 v = *src;
    v4i r;
    r[0] = v.x;
    r[1] = v.y;
    r[2] = v.z;
    r[3] = v.w;
    return r;
}

__device__ __forceinline__ float plane_sum(const v4i &c0, const v4i &c1, const v4i &c2, int r)
{
    return fmaf((float)c2[r], 65536.f, fmaf((float)c1[r], 256.f, (float)c0[r]));
}

// Gate/up: a wave unit is RT tiles of 16 intermediate rows of one item x
// all its tokens (16 at a time); the tokens' digit loads serve all RT tiles.
template <int BITS, int RT>
__global__ void __launch_bounds__(256) k_gate_up_m(BatchArgs a)
{
    using C = Codes<BITS>;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r16 = lane & 15, h = lane >> 4;
    const int D = a.D, I = a.I;
    const int nact = *a.n_act;
    const int items = nact + (a.src.n_slots > a.src.top_k ? 1 : 0);
    const int upi = I / (16 * RT);  // I is a multiple of 64
    const int ng = D / kGroup, nchunks = D * BITS / 128;
    const int xdw = nchunks * C::DW;
    const uint64_t mat_q = (uint64_t)I * D * BITS / 8, row_q = (uint64_t)D * BITS / 8;
    const uint64_t sb0 = 3 * mat_q, mat_sb = (uint64_t)I * ng * 4;
    for (int u = blockIdx.x * 4 + wave; u < items * upi; u += gridDim.x * 4) {
        const int ii = u / upi, i0 = (u - ii * upi) * 16 * RT;
        const Item it = item_of(a, ii, nact);
        if (it.n < kMfmaMin) continue;
        for (int j0 = 0; j0 < it.n; j0 += 16) {
            const int jt = j0 + r16;
            const bool tok_ok = jt < it.n;
            const int tok = token_of(a, it, tok_ok ? jt : j0);
            const int *xd = a.xdig + (size_t)tok * xdw;
            const float *xc = a.xcsum + (size_t)tok * nchunks;
            const float inv = a.xinv[tok];
            float acc[RT][2][4];
#pragma unroll
            for (int t = 0; t < RT; ++t)
#pragma unroll
                for (int m = 0; m < 2; ++m)
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[t][m][r] = 0.f;
            for (int g = 0; g < ng; ++g) {
                const v4i b0 = mfma_b<BITS>(xd, g, h, 0), b1 = mfma_b<BITS>(xd, g, h, 1), b2 = mfma_b<BITS>(xd, g, h, 2);
                const float gs = BITS == 4 ? xc[2 * g] + xc[2 * g + 1] : xc[g];
#pragma unroll
                for (int t = 0; t < RT; ++t)
#pragma unroll
                    for (int m = 0; m < 2; ++m) {
                        const v4i av = mfma_a<BITS>(it.blob + m * mat_q + (uint64_t)(i0 + 16 * t + r16) * row_q, g, h);
                        const v4i z = {0, 0, 0, 0};
                        const v4i c0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, b0, z, 0, 0, 0);
                        const v4i c1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, b1, z, 0, 0, 0);
                        const v4i c2 = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, b2, z, 0, 0, 0);
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int row = i0 + 16 * t + 4 * h + r;
                            const uint32_t sb = *reinterpret_cast<const uint32_t *>(
                                it.blob + sb0 + m * mat_sb + ((uint64_t)row * ng + g) * 4);
                            acc[t][m][r] = fmaf(bf16_lo(sb) * inv, plane_sum(c0, c1, c2, r), acc[t][m][r]);
                            acc[t][m][r] = fmaf(bf16_hi(sb), gs, acc[t][m][r]);
                        }
                    }
            }
            if (tok_ok) {
#pragma unroll
                for (int t = 0; t < RT; ++t)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float gg = acc[t][0][r], uu = acc[t][1][r];
                        a.h[(size_t)(it.pos0 + jt) * I + i0 + 16 * t + 4 * h + r] = gg / (1.f + expf(-gg)) * uu;
                    }
            }
        }
    }
}

// Down: a wave unit is RT tiles of 16 output rows of one item x all its
// positions (16 at a time), against the positions' digit tables of h.
template <int BITS, int RT>
__global__ void __launch_bounds__(256) k_down_m(BatchArgs a)
{
    using C = Codes<BITS>;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r16 = lane & 15, h = lane >> 4;
    const int D = a.D, I = a.I;
    const int nact = *a.n_act;
    const int items = nact + (a.src.n_slots > a.src.top_k ? 1 : 0);
    const int upi = D / (16 * RT);  // D is a multiple of 64
    const int ng = I / kGroup, nchunks = I * BITS / 128;
    const int hdw = nchunks * C::DW;
    const uint64_t mat_q = (uint64_t)I * D * BITS / 8, row_q = (uint64_t)I * BITS / 8;
    const uint64_t sbd = 3 * mat_q + 2 * ((uint64_t)D * ng * 4);
    for (int u = blockIdx.x * 4 + wave; u < items * upi; u += gridDim.x * 4) {
        const int ii = u / upi, o0 = (u - ii * upi) * 16 * RT;
        const Item it = item_of(a, ii, nact);
        if (it.n < kMfmaMin) continue;
        for (int j0 = 0; j0 < it.n; j0 += 16) {
            const int jt = j0 + r16;
            const bool ok = jt < it.n;
            const int pos = it.pos0 + (ok ? jt : j0);
            const int *hd = a.hdig + (size_t)pos * hdw;
            const float *hc = a.hcsum + (size_t)pos * nchunks;
            const float inv = a.hinv[pos];
            float acc[RT][4];
#pragma unroll
            for (int t = 0; t < RT; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[t][r] = 0.f;
            for (int g = 0; g < ng; ++g) {
                const v4i b0 = mfma_b<BITS>(hd, g, h, 0), b1 = mfma_b<BITS>(hd, g, h, 1), b2 = mfma_b<BITS>(hd, g, h, 2);
                const float gs = BITS == 4 ? hc[2 * g] + hc[2 * g + 1] : hc[g];
#pragma unroll
                for (int t = 0; t < RT; ++t) {
                    const v4i av = mfma_a<BITS>(it.blob + 2 * mat_q + (uint64_t)(o0 + 16 * t + r16) * row_q, g, h);
                    const v4i z = {0, 0, 0, 0};
                    const v4i c0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, b0, z, 0, 0, 0);
                    const v4i c1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, b1, z, 0, 0, 0);
                    const v4i c2 = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, b2, z, 0, 0, 0);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int row = o0 + 16 * t + 4 * h + r;
                        const uint32_t sb = *reinterpret_cast<const uint32_t *>(it.blob + sbd + ((uint64_t)row * ng + g) * 4);
                        acc[t][r] = fmaf(bf16_lo(sb) * inv, plane_sum(c0, c1, c2, r), acc[t][r]);
                        acc[t][r] = fmaf(bf16_hi(sb), gs, acc[t][r]);
                    }
                }
            }
            if (ok) {
#pragma unroll
                for (int t = 0; t < RT; ++t)
#pragma unroll
                    for (int r = 0; r < 4; ++r) a.y[(size_t)(it.pos0 + jt) * D + o0 + 16 * t + 4 * h + r] = acc[t][r];
            }
        }
    }
}

// ---------------------------------------------------------------------------
template <int BITS>
hipError_t batch_bits(const BatchArgs &a, int stage, hipStream_t s)
{
    using C = Codes<BITS>;
    const int nchunks_d = a.D * BITS / 128, nchunks_i = a.I * BITS / 128;
    const int cpl = (nchunks_d + 63) / 64;
    const DownShape d = down_shape(a.I, BITS);
    switch (stage) {
    case 0:  // x digits
        hipLaunchKernelGGL(k_digits<BITS>, dim3(a.T), dim3(256), 0, s, a.x, a.D, a.xdig, a.xcsum, a.xinv,
                           nchunks_d * C::DW, nchunks_d);
        break;
    case 1: {  // gate/up
        constexpr int R = BITS == 4 ? 4 : 8;
        if (cpl <= 1) hipLaunchKernelGGL((k_gate_up_b<BITS, 1, R>), dim3(1024), dim3(256), 0, s, a);
        else if constexpr (BITS == 4) {
            if (cpl <= 2) hipLaunchKernelGGL((k_gate_up_b<BITS, 2, 2>), dim3(1024), dim3(256), 0, s, a);
            else hipLaunchKernelGGL((k_gate_up_b<BITS, 4, 1>), dim3(1024), dim3(256), 0, s, a);
        } else {
            hipLaunchKernelGGL((k_gate_up_b<BITS, 2, 4>), dim3(1024), dim3(256), 0, s, a);
        }
        if (a.T >= kMfmaMin) hipLaunchKernelGGL((k_gate_up_m<BITS, 2>), dim3(1024), dim3(256), 0, s, a);
        break;
    }
    case 2:  // h digits (all positions)
        hipLaunchKernelGGL(k_digits<BITS>, dim3(a.T * a.src.n_slots), dim3(256), 0, s, a.h, a.I, a.hdig, a.hcsum,
                           a.hinv, nchunks_i * C::DW, nchunks_i);
        break;
    case 3: {  // down
#define MOE_DB(LPR_)                                                                                         \
    case LPR_:                                                                                               \
        if (d.cpl <= 1)                                                                                      \
            hipLaunchKernelGGL((k_down_b<BITS, LPR_, 1, ((4 * LPR_ / 64) < 1 ? 1 : 4 * LPR_ / 64)>), dim3(1024), \
                               dim3(256), 0, s, a);                                                          \
        else                                                                                                 \
            hipLaunchKernelGGL((k_down_b<BITS, LPR_, 2, ((4 * LPR_ / 64) < 1 ? 1 : 4 * LPR_ / 64)>), dim3(1024), \
                               dim3(256), 0, s, a);                                                          \
        break;
        switch (d.lpr) {
            MOE_DB(1)
            MOE_DB(2)
            MOE_DB(4)
            MOE_DB(8)
            MOE_DB(16)
            MOE_DB(32)
            MOE_DB(64)
        }
#undef MOE_DB
        if (a.T >= kMfmaMin) hipLaunchKernelGGL((k_down_m<BITS, 2>), dim3(1024), dim3(256), 0, s, a);
        break;
    }
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_batch_route(const BatchArgs &a, int do_topk, hipStream_t s)
{
    if (do_topk) {
        if (a.T <= 8) hipLaunchKernelGGL(k_route_b<8>, dim3((a.E + 3) / 4), dim3(256), 0, s, a);
        else hipLaunchKernelGGL(k_route_b<32>, dim3((a.E + 3) / 4), dim3(256), 0, s, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k_topk_group, dim3(1), dim3(1024), 0, s, a, do_topk);
    return hipGetLastError();
}

hipError_t launch_batch_experts(const BatchArgs &a, int bits, hipStream_t s)
{
    for (int stage = 0; stage < 4; ++stage) {
        hipError_t e = bits == 4 ? batch_bits<4>(a, stage, s) : batch_bits<2>(a, stage, s);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k_combine_b, dim3(a.T), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace moe
