// moe_batch.hip -- the MoE block for a batch of T > 1 tokens.
//
// Batching must not change the arithmetic of a token (the pages run one
// token at a time, hakusoku.com "パイプライン概要"); what it changes is how
// often an expert's weights are read.  Tokens are grouped by expert so that
// every selected expert's rows are fetched once per step and applied to all
// of that expert's tokens:
//
//   k_route_m      partial logits of every token over kRouteSplit slices of
//                  the hidden dimension (fp32 matrix cores)
//   k_topk_b       the logits (slices added in order), per-token top-K and
//                  softmax weights (one wave per token)
//   k_group        the grouping: count[e], offset[e] (exclusive prefix
//                  sum), the pair permutation perm[pos] = t*K + k sorted by
//                  (expert, pair index), its inverse, and the list of active
//                  experts
//   k_digits       fixed-point digit tables of the tokens' activations
//   k_gate_up_b    per active expert (and the shared expert, all tokens):
//                  gate/up rows x that expert's tokens, SwiGLU -> h[pos]
//                  (k_gate_up_m on the matrix cores for experts with 8+
//                  tokens)
//   k_digits       digit tables of h
//   k_down_b       per active expert: down rows x its tokens' h -> y[pos]
//                  (k_down_m for experts with 8+ tokens)
//   k_combine_b    per token, in slot order: sum_k w_k y[pos(t,k)] + the
//                  shared expert's y, then (layer mode) residual + RMSNorm
//
// Every step is deterministic (no float atomics, fixed summation orders).
#include "moe_device.h"

namespace moe {
namespace {

using namespace dev;

// ---------------------------------------------------------------------------
// Router for T tokens on the matrix cores (fp32): a block owns a tile of 16
// router rows x 16 tokens over one slice of the hidden dimension (slices
// spread the router's bytes over enough CUs); its four waves take every
// fourth 64-column block of the slice, and their partial logits are added
// in order in LDS.  lpart[s][t][e] receives slice s's partial logit.
// v_mfma_f32_16x16x4f32: lane l supplies row (A) / token (B) l % 16 at
// k = l / 16; each lane loads 4 consecutive columns, so 4 instructions
// cover 16 columns (A and B use the same column-to-instruction map).
typedef float v4f __attribute__((ext_vector_type(4)));
__global__ void __launch_bounds__(256) k_route_m(BatchArgs a, int splits)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r16 = lane & 15, h = lane >> 4;
    const int D = a.D, E = a.E, T = a.T;
    const int ttiles = (T + 15) / 16, rtiles = (E + 15) / 16;
    const int sl = blockIdx.x / (rtiles * ttiles), rem = blockIdx.x - sl * rtiles * ttiles;
    const int e0 = (rem / ttiles) * 16, t0 = (rem % ttiles) * 16;
    const int row = min(e0 + r16, E - 1), tok = min(t0 + r16, T - 1);
    const float *w = a.router + (size_t)row * D;
    const float *x = a.x + (size_t)tok * D;
    const int lo = sl * (D / splits), hi = lo + D / splits;  // D / splits is a multiple of 64
    v4f c = {0.f, 0.f, 0.f, 0.f};
    for (int k0 = lo + 64 * wave; k0 < hi; k0 += 256) {
        float4 wv[4], xv[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int k = k0 + 16 * u + 4 * h;
            wv[u] = *reinterpret_cast<const float4 *>(w + k);
            xv[u] = *reinterpret_cast<const float4 *>(x + k);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            c = __builtin_amdgcn_mfma_f32_16x16x4f32(wv[u].x, xv[u].x, c, 0, 0, 0);
            c = __builtin_amdgcn_mfma_f32_16x16x4f32(wv[u].y, xv[u].y, c, 0, 0, 0);
            c = __builtin_amdgcn_mfma_f32_16x16x4f32(wv[u].z, xv[u].z, c, 0, 0, 0);
            c = __builtin_amdgcn_mfma_f32_16x16x4f32(wv[u].w, xv[u].w, c, 0, 0, 0);
        }
    }
    __shared__ float part[4][64][4];
#pragma unroll
    for (int r = 0; r < 4; ++r) part[wave][lane][r] = c[r];
    __syncthreads();
    if (wave == 0) {
        const int t = t0 + r16;
        float *out = a.lpart + (size_t)sl * T * E;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int e = e0 + 4 * h + r;
            const float v = ((part[0][lane][r] + part[1][lane][r]) + part[2][lane][r]) + part[3][lane][r];
            if (e < E && t < T) out[(size_t)t * E + e] = v;
        }
    }
}

// Hidden-dimension slices of the batched router: kRouteSplit when the
// slices stay multiples of 64 columns.
__host__ __device__ inline int route_splits(int D)
{
    for (int s = kRouteSplit; s > 1; s >>= 1)
        if (D % (64 * s) == 0) return s;
    return 1;
}

// ---------------------------------------------------------------------------
// Top-K of every token: one wave per token, its logits (the slices' partial
// logits added in slice order, also stored to logits[t]) in LDS; K rounds of
// the wave's largest remaining key (larger logit first, the lower index on a
// tie), then the softmax over the selected logits.
__global__ void __launch_bounds__(256) k_topk_b(BatchArgs a, int splits)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int t = blockIdx.x * 4 + wave;
    const int E = a.E, K = a.K, T = a.T;
    __shared__ float lg[4][4096];
    if (t >= T) return;  // whole waves leave; no block barrier follows
    for (int e0 = 0; e0 < E; e0 += 64 * 8) {
        float v[8][kRouteSplit];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int e = e0 + lane + 64 * u;
#pragma unroll
            for (int sl = 0; sl < kRouteSplit; ++sl)
                v[u][sl] = e < E && sl < splits ? a.lpart[((size_t)sl * T + t) * E + e] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int e = e0 + lane + 64 * u;
            float sum = v[u][0];
#pragma unroll
            for (int sl = 1; sl < kRouteSplit; ++sl)
                if (sl < splits) sum += v[u][sl];
            if (e < E) {
                lg[wave][e] = sum;
                a.logits[(size_t)t * E + e] = sum;
            }
        }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_wave_barrier();
    uint64_t taken = 0;  // bit j: element lane + 64 j selected
    int idx[kMaxTopK];
    float vals[kMaxTopK], w[kMaxTopK];
#pragma unroll
    for (int k = 0; k < kMaxTopK; ++k) {
        idx[k] = -1;
        vals[k] = -INFINITY;
        if (k >= K) continue;
        uint64_t best = 0ull;
        for (int jj = 0, e = lane; e < E; ++jj, e += 64)
            if (!((taken >> jj) & 1ull)) {
                const uint64_t key = route_key(lg[wave][e], e);
                best = key > best ? key : best;
            }
        const uint64_t m = wave_max_key(best);
        const int e = key_index(m);
        if ((e & 63) == lane) taken |= 1ull << (e >> 6);
        idx[k] = e;
        vals[k] = key_value(m);
    }
    topk_weights(vals, K, w);
    if (lane < K) {
#pragma unroll
        for (int k = 0; k < kMaxTopK; ++k)
            if (k == lane) {
                a.topk_idx[(size_t)t * K + k] = idx[k];
                a.topk_w[(size_t)t * K + k] = w[k];
            }
    }
}

// Exclusive prefix sums of three arrays v0, v1, v2 [0..n) in place
// (n <= 4 * blockDim.x), their totals in tot[]; one block.  Each thread sums
// 4 consecutive entries, a wave scan (shuffles) runs over the threads' sums,
// then every thread adds the totals of the waves before its own (one
// barrier).  wsum: LDS [blockDim.x / 64][3].
__device__ __forceinline__ void block_exscan3(int *v0, int *v1, int *v2, int n, int (*wsum)[3], int (&tot)[3])
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = blockDim.x >> 6;
    int *const v[3] = {v0, v1, v2};
    int loc[3][4], run[3], inc[3];
#pragma unroll
    for (int c = 0; c < 3; ++c) {
        run[c] = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int i = 4 * tid + q;
            loc[c][q] = run[c];
            run[c] += i < n ? v[c][i] : 0;
        }
        inc[c] = run[c];
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1)
#pragma unroll
        for (int c = 0; c < 3; ++c) {
            const int y = __shfl_up(inc[c], off, 64);
            if (lane >= off) inc[c] += y;
        }
    if (lane == 63)
#pragma unroll
        for (int c = 0; c < 3; ++c) wsum[wave][c] = inc[c];
    __syncthreads();
    int before[3] = {0, 0, 0};
#pragma unroll
    for (int c = 0; c < 3; ++c) tot[c] = 0;
    for (int w = 0; w < nw; ++w)
#pragma unroll
        for (int c = 0; c < 3; ++c) {
            if (w < wave) before[c] += wsum[w][c];
            tot[c] += wsum[w][c];
        }
#pragma unroll
    for (int c = 0; c < 3; ++c)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int i = 4 * tid + q;
            if (i < n) v[c][i] = before[c] + (inc[c] - run[c]) + loc[c][q];
        }
    __syncthreads();
}

// One block of 1024 threads: the token -> expert grouping of the
// selections: count[e], offset[e] (exclusive prefix sums), the pair
// permutation perm[pos] = t*K + k sorted by (expert, pair index), its
// inverse, the active experts in ascending order and, among them, those
// with at least kMfmaMin tokens; and the matrix-core kernels' dense work
// list: every (such expert, or the shared expert when T >= kMfmaMin; tile of
// 16 of its tokens).
__global__ void __launch_bounds__(1024) k_group(BatchArgs a)
{
    const int tid = threadIdx.x;
    const int T = a.T, K = a.K, E = a.E, P = T * K;
    __shared__ int s_idx[64 * kMaxTopK];
    __shared__ int s_count[4096];
    __shared__ int s_off[4096];
    __shared__ int s_flag[4096];
    __shared__ int s_big[4096];
    __shared__ int wsum[16][3];
    __shared__ int s_bigl[4096];
    for (int p = tid; p < P; p += 1024) s_idx[p] = a.topk_idx[p];
    for (int e = tid; e < E; e += 1024) s_count[e] = 0;
    __syncthreads();
    for (int p = tid; p < P; p += 1024) {
        const int e = s_idx[p];
        if (e >= 0 && e < E) atomicAdd(&s_count[e], 1);
        else atomicOr(a.flags, MOE_DEVERR_EXPERT_RANGE);
    }
    __syncthreads();
    for (int e = tid; e < E; e += 1024) {
        s_off[e] = s_count[e];
        s_flag[e] = s_count[e] > 0;
        s_big[e] = s_count[e] >= kMfmaMin;
        a.count[e] = s_count[e];
    }
    __syncthreads();
    int tot[3];
    block_exscan3(s_off, s_flag, s_big, E, wsum, tot);
    for (int e = tid; e < E; e += 1024) {
        a.offset[e] = s_off[e];
        if (s_count[e]) a.act[s_flag[e]] = e;
        if (s_count[e] >= kMfmaMin) {
            a.big[s_big[e]] = e;
            s_bigl[s_big[e]] = e;
        }
    }
    if (tid == 0) {
        a.offset[E] = tot[0];
        *a.n_act = tot[1];
        *a.n_big = tot[2];
    }
    __syncthreads();
    if (tid == 0) {
        int w = 0;
        for (int ii = 0; ii < tot[2]; ++ii)
            for (int tt = 0; 16 * tt < s_count[s_bigl[ii]]; ++tt) a.mwork[w++] = ii << 2 | tt;
        if (a.src.n_slots > K && T >= kMfmaMin)
            for (int tt = 0; 16 * tt < T; ++tt) a.mwork[w++] = tot[2] << 2 | tt;
        *a.n_mwork = w;
    }
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

// Item ii of the matrix-core work list: expert big[ii], or the shared
// expert for ii == n_big.
__device__ __forceinline__ Item big_item_of(const BatchArgs &a, int ii, int nbig)
{
    Item r;
    if (ii < nbig) {
        const int e = a.big[ii];
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
__global__ void __launch_bounds__(1024) k_combine_b(BatchArgs a)
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
    constexpr int PER = 8;  // D <= 8192
    float rv[PER];
    float ss = 0.f;
    // the combine of the token's rows first (the outputs never alias y),
    // summed in slot order, then residual and norm; each slot's rows are
    // loaded together
#pragma unroll
    for (int j = 0; j < PER; ++j) rv[j] = 0.f;
    for (int k = 0; k <= K; ++k) {
        const int pk = k < K ? pos[k] : (has_shared ? a.T * K + t : -1);
        if (pk < 0) continue;
        float yv[PER];
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int o = tid + 1024 * j;
            yv[j] = o < D ? a.y[(size_t)pk * D + o] : 0.f;
        }
        if (k < K) {
            const float wk = wts[k];
#pragma unroll
            for (int j = 0; j < PER; ++j) rv[j] += wk * yv[j];
        } else {
#pragma unroll
            for (int j = 0; j < PER; ++j) rv[j] += yv[j];
        }
    }
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int o = tid + 1024 * j;
        if (o >= D) continue;
        if (a.mode == 0) {
            a.yout[(size_t)t * D + o] = rv[j];
        } else {
            const float r = a.resid[(size_t)t * D + o] + rv[j];
            rv[j] = r;
            ss += r * r;
        }
    }
    if (a.mode == 0) return;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int o = tid + 1024 * j;
        if (o < D) a.resid[(size_t)t * D + o] = rv[j];
    }
    ss = group_sum<64>(ss);
    if ((tid & 63) == 0) red[tid >> 6] = ss;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < 16; ++w) tot += red[w];
    const float inv = 1.f / sqrtf(tot / (float)D + a.eps);
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int o = tid + 1024 * j;
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

// One scale group's operands for a wave: the masked codes of M matrices'
// rows (A), the digit words of the three planes (B), the lane's four output
// rows' scale/bias words and the chunk sums of the group.
template <int M>
struct MfStage {
    v4i a[M];
    v4i b0, b1, b2;
    uint32_t sb[M][4];
    float gs;
};

template <int BITS, int M>
__device__ __forceinline__ void mf_load(MfStage<M> &st, const uint8_t *const (&rowq)[M], const uint8_t *const (&sbr)[M],
                                        uint32_t sb_stride, const int *dig, const float *cs, int g, int h)
{
#pragma unroll
    for (int m = 0; m < M; ++m) {
        st.a[m] = mfma_a<BITS>(rowq[m], g, h);
#pragma unroll
        for (int r = 0; r < 4; ++r) st.sb[m][r] = *reinterpret_cast<const uint32_t *>(sbr[m] + (size_t)r * sb_stride + 4 * g);
    }
    st.b0 = mfma_b<BITS>(dig, g, h, 0);
    st.b1 = mfma_b<BITS>(dig, g, h, 1);
    st.b2 = mfma_b<BITS>(dig, g, h, 2);
    st.gs = BITS == 4 ? cs[2 * g] + cs[2 * g + 1] : cs[g];
}

template <int M>
__device__ __forceinline__ void mf_step(const MfStage<M> &st, float inv, float (&acc)[M][4])
{
    const v4i z = {0, 0, 0, 0};
#pragma unroll
    for (int m = 0; m < M; ++m) {
        const v4i c0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(st.a[m], st.b0, z, 0, 0, 0);
        const v4i c1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(st.a[m], st.b1, z, 0, 0, 0);
        const v4i c2 = __builtin_amdgcn_mfma_i32_16x16x64_i8(st.a[m], st.b2, z, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            acc[m][r] = fmaf(bf16_lo(st.sb[m][r]) * inv, plane_sum(c0, c1, c2, r), acc[m][r]);
            acc[m][r] = fmaf(bf16_hi(st.sb[m][r]), st.gs, acc[m][r]);
        }
    }
}

// A wave's share of the contraction of one 16-row tile (M matrices) with
// one 16-vector tile: scale groups g0, g0 + gs, ... below ng, in batches of
// NB groups whose loads are all issued before the batch's arithmetic.
template <int BITS, int M, int NB>
__device__ __forceinline__ void mf_tile(const uint8_t *const (&rowq)[M], const uint8_t *const (&sbr)[M], uint32_t sb_stride,
                                        const int *dig, const float *cs, float inv, int g0, int gs, int ng, int h,
                                        float (&acc)[M][4])
{
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[m][r] = 0.f;
    for (int gb = g0; gb < ng; gb += NB * gs) {
        MfStage<M> st[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b)
            if (gb + b * gs < ng) mf_load<BITS, M>(st[b], rowq, sbr, sb_stride, dig, cs, gb + b * gs, h);
#pragma unroll
        for (int b = 0; b < NB; ++b)
            if (gb + b * gs < ng) mf_step<M>(st[b], inv, acc);
    }
}

// The partial tiles of the block's KS waves, added in wave order into wave
// 0's lanes.
template <int M, int KS>
__device__ __forceinline__ void mf_reduce(float (&acc)[M][4], float (*part)[M][64][4])
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (wave > 0) {
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r) part[wave - 1][m][lane][r] = acc[m][r];
    }
    __syncthreads();
    if (wave == 0) {
        for (int w = 0; w < KS - 1; ++w)
#pragma unroll
            for (int m = 0; m < M; ++m)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[m][r] += part[w][m][lane][r];
    }
    __syncthreads();
}

constexpr int kMfWaves = 8;  // waves per matrix-core block (scale groups split over them)

// Gate/up: a block unit is one 16-row tile of an item's gate and up
// matrices x one tile of 16 of its tokens; the block's kMfWaves waves take
// every kMfWaves-th scale group and their partial sums meet in LDS.
template <int BITS>
__global__ void __launch_bounds__(64 * kMfWaves) k_gate_up_m(BatchArgs a)
{
    using C = Codes<BITS>;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r16 = lane & 15, h = lane >> 4;
    const int D = a.D, I = a.I;
    const int nbig = *a.n_big, nwork = *a.n_mwork;
    const int rtiles = I / 16;  // I is a multiple of 64
    const int ng = D / kGroup, nchunks = D * BITS / 128;
    const int xdw = nchunks * C::DW;
    const uint64_t mat_q = (uint64_t)I * D * BITS / 8, row_q = (uint64_t)D * BITS / 8;
    const uint64_t sb0 = 3 * mat_q, mat_sb = (uint64_t)I * ng * 4;
    __shared__ float part[kMfWaves - 1][2][64][4];
    for (int u = blockIdx.x; u < nwork * rtiles; u += gridDim.x) {
        const int wk = a.mwork[u / rtiles], ii = wk >> 2;
        const int i0 = (u % rtiles) * 16, j0 = (wk & 3) * 16;
        const Item it = big_item_of(a, ii, nbig);
        const int jt = j0 + r16;
        const bool tok_ok = jt < it.n;
        const int tok = token_of(a, it, tok_ok ? jt : j0);
        const uint8_t *const rowq[2] = {it.blob + (uint64_t)(i0 + r16) * row_q, it.blob + mat_q + (uint64_t)(i0 + r16) * row_q};
        const uint8_t *const sbr[2] = {it.blob + sb0 + (uint64_t)(i0 + 4 * h) * ng * 4,
                                       it.blob + sb0 + mat_sb + (uint64_t)(i0 + 4 * h) * ng * 4};
        float acc[2][4];
        mf_tile<BITS, 2, 2>(rowq, sbr, ng * 4, a.xdig + (size_t)tok * xdw, a.xcsum + (size_t)tok * nchunks, a.xinv[tok], wave,
                            kMfWaves, ng, h, acc);
        mf_reduce<2, kMfWaves>(acc, part);
        if (wave == 0 && tok_ok) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float gg = acc[0][r], uu = acc[1][r];
                a.h[(size_t)(it.pos0 + jt) * I + i0 + 4 * h + r] = gg / (1.f + expf(-gg)) * uu;
            }
        }
    }
}

// Down: a block unit is one 16-row tile of an item's down matrix x one tile
// of 16 of its positions (digit tables of h), scale groups split over the
// waves as above.
template <int BITS>
__global__ void __launch_bounds__(64 * kMfWaves) k_down_m(BatchArgs a)
{
    using C = Codes<BITS>;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r16 = lane & 15, h = lane >> 4;
    const int D = a.D, I = a.I;
    const int nbig = *a.n_big, nwork = *a.n_mwork;
    const int rtiles = D / 16;  // D is a multiple of 64
    const int ng = I / kGroup, nchunks = I * BITS / 128;
    const int hdw = nchunks * C::DW;
    const uint64_t mat_q = (uint64_t)I * D * BITS / 8, row_q = (uint64_t)I * BITS / 8;
    const uint64_t sbd = 3 * mat_q + 2 * ((uint64_t)D * ng * 4);
    __shared__ float part[kMfWaves - 1][1][64][4];
    for (int u = blockIdx.x; u < nwork * rtiles; u += gridDim.x) {
        const int wk = a.mwork[u / rtiles], ii = wk >> 2;
        const int o0 = (u % rtiles) * 16, j0 = (wk & 3) * 16;
        const Item it = big_item_of(a, ii, nbig);
        const int jt = j0 + r16;
        const bool ok = jt < it.n;
        const int pos = it.pos0 + (ok ? jt : j0);
        const uint8_t *const rowq[1] = {it.blob + 2 * mat_q + (uint64_t)(o0 + r16) * row_q};
        const uint8_t *const sbr[1] = {it.blob + sbd + (uint64_t)(o0 + 4 * h) * ng * 4};
        float acc[1][4];
        mf_tile<BITS, 1, 8>(rowq, sbr, ng * 4, a.hdig + (size_t)pos * hdw, a.hcsum + (size_t)pos * nchunks, a.hinv[pos], wave,
                            kMfWaves, ng, h, acc);
        mf_reduce<1, kMfWaves>(acc, part);
        if (wave == 0 && ok) {
#pragma unroll
            for (int r = 0; r < 4; ++r) a.y[(size_t)(it.pos0 + jt) * D + o0 + 4 * h + r] = acc[0][r];
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
        constexpr int R = 4;
        if (cpl <= 1) hipLaunchKernelGGL((k_gate_up_b<BITS, 1, R>), dim3(1024), dim3(256), 0, s, a);
        else if constexpr (BITS == 4) {
            if (cpl <= 2) hipLaunchKernelGGL((k_gate_up_b<BITS, 2, 2>), dim3(1024), dim3(256), 0, s, a);
            else hipLaunchKernelGGL((k_gate_up_b<BITS, 4, 1>), dim3(1024), dim3(256), 0, s, a);
        } else {
            hipLaunchKernelGGL((k_gate_up_b<BITS, 2, 4>), dim3(1024), dim3(256), 0, s, a);
        }
        if (a.T >= kMfmaMin) hipLaunchKernelGGL((k_gate_up_m<BITS>), dim3(1024), dim3(64 * kMfWaves), 0, s, a);
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
        if (a.T >= kMfmaMin) hipLaunchKernelGGL((k_down_m<BITS>), dim3(1024), dim3(64 * kMfWaves), 0, s, a);
        break;
    }
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_batch_route(const BatchArgs &a, int do_topk, hipStream_t s)
{
    if (do_topk) {
        const int splits = route_splits(a.D);
        hipLaunchKernelGGL(k_route_m, dim3(splits * ((a.E + 15) / 16) * ((a.T + 15) / 16)), dim3(256), 0, s, a, splits);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(k_topk_b, dim3((a.T + 3) / 4), dim3(256), 0, s, a, splits);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k_group, dim3(1), dim3(1024), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_batch_experts(const BatchArgs &a, int bits, hipStream_t s)
{
    for (int stage = 0; stage < 4; ++stage) {
        hipError_t e = bits == 4 ? batch_bits<4>(a, stage, s) : batch_bits<2>(a, stage, s);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k_combine_b, dim3(a.T), dim3(1024), 0, s, a);
    return hipGetLastError();
}

}  // namespace moe
