// moe_batch.hip -- the MoE block for a batch of T > 1 tokens.
//
// Batching must not change the arithmetic of a token (the pages run one
// token at a time, hakusoku.com "パイプライン概要"); what it changes is how
// often an expert's weights are read.  Tokens are grouped by expert so that
// every selected expert's rows are fetched once per step and applied to all
// of that expert's tokens:
//
//   k_route_m      partial logits of every token over kRouteSplit slices of
//                  the hidden dimension (fp32 matrix cores), and the
//                  tokens' activations as digit words, one fixed-point step
//                  per scale group (k_xdigits alone when routing is given)
//   k_topk_b       the logits (slices added in order), per-token top-K and
//                  softmax weights (one wave per token); up to 512 experts
//                  its last block also does k_group's work
//   k_group        the grouping: count[e], offset[e] (exclusive prefix
//                  sum), the pair permutation perm[pos] = t*K + k sorted by
//                  (expert, pair index), its inverse, the list of active
//                  experts and the expert kernels' work list (expert, tile
//                  of 16 of its tokens)
//   k_expert_mm<0> per active expert (and the shared expert, all tokens):
//                  gate/up rows x that expert's tokens on the matrix cores,
//                  SwiGLU -> h[pos] as digit words, one step per scale group
//   k_expert_mm<1> per active expert: down rows x its positions' h -> y[pos]
//   k_combine_b    per token, in slot order: sum_k w_k y[pos(t,k)] + the
//                  shared expert's y, then (layer mode) residual + RMSNorm
//
// Every step is deterministic (no float atomics, fixed summation orders).
#include <type_traits>

#include "moe_device.h"

namespace moe {
namespace {

using namespace dev;

// ---------------------------------------------------------------------------
// Digit words of activations, one fixed-point step per (vector, scale group
// of 64 values): the rule of a whole-vector table (largest magnitude times
// 2^k below 2^22) applied to each group's own range.  The 16 lanes of a DPP
// row convert one group: lane q takes the four values that share digit word
// (code word q / SUBS, sub q % SUBS) of each plane.  A group's words are
// kGroupWords consecutive ints (its chunks' digit words, plane-major within
// a chunk), so a vector's groups are kGroupWords apart.
constexpr int kGroupWords = 48;  // digit words per scale group (any bit width)

template <int BITS>
__device__ __forceinline__ int group_value(int q, int j)
{
    using C = Codes<BITS>;
    return (q / C::SUBS) * C::PER_WORD + q % C::SUBS + C::SUBS * j;
}

// v: lane q's four values (group_value(q, 0..3)); dig: the group's words;
// lane 0 writes the group's sum of values and its step 2^-k.
template <int BITS>
__device__ __forceinline__ void group_digits(const float v[4], int q, int *dig, float *gsum, float *ginv)
{
    using C = Codes<BITS>;
    static_assert(C::DW * (kGroup / C::CODES) == kGroupWords && kGroup / 4 == 16, "16 lanes per scale group");
    const float mx = group_max<16>(fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3]))));
    const float sm = group_sum<16>((v[0] + v[1]) + (v[2] + v[3]));
    float mul, inv;
    fixed_scale(mx, mul, inv);
    int w0, w1, w2;
    digit_words(v[0], v[1], v[2], v[3], mul, w0, w1, w2);
    const int kb = q / C::SUBS;
    int *o = dig + (kb / 4) * C::DW + (kb % 4) * C::SUBS + q % C::SUBS;
    o[0] = w0;
    o[C::PW] = w1;
    o[2 * C::PW] = w2;
    if (q == 0) {
        *gsum = sm;
        *ginv = inv;
    }
}

// Scale group g of the activations of tokens t0 + 4 wave + lane / 16 (each
// DPP row one token) -> xdig / xcsum / xinv.
template <int BITS>
__device__ __forceinline__ void x_group_digits(const BatchArgs &a, int t0, int g, int lane, int wave)
{
    const int t = t0 + 4 * wave + (lane >> 4), q = lane & 15, ng = a.D / kGroup;
    if (t >= a.T) return;  // whole DPP rows drop out
    const float *xs = a.x + (size_t)t * a.D + g * kGroup;
    float v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = xs[group_value<BITS>(q, j)];
    const size_t tg = (size_t)t * ng + g;
    group_digits<BITS>(v, q, a.xdig + tg * kGroupWords, a.xcsum + tg, a.xinv + tg);
}

// ---------------------------------------------------------------------------
// Router for T tokens on the matrix cores (fp32): a block owns a tile of 16
// router rows x 16 tokens over one slice of the hidden dimension (slices
// spread the router's bytes over enough CUs); its four waves take every
// fourth 64-column block of the slice, and their partial logits are added
// in order in LDS.  lpart[s][t][e] receives slice s's partial logit.
// v_mfma_f32_16x16x4f32: lane l supplies row (A) / token (B) l % 16 at
// k = l / 16; each lane loads 4 consecutive columns, so 4 instructions
// cover 16 columns (A and B use the same column-to-instruction map).
// The blocks of a (slice, token tile) also convert the slice's scale groups
// of those tokens' activations to digit words, row tile r taking groups r,
// r + row tiles, ...
typedef float v4f __attribute__((ext_vector_type(4)));
template <int BITS>
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
    const int gps = D / splits / kGroup;
    for (int gi = rem / ttiles; gi < gps; gi += rtiles) x_group_digits<BITS>(a, t0, sl * gps + gi, lane, wave);
}

// The activations' digit words alone (routing given by the caller): block
// b converts scale group b % groups of token tile b / groups.
template <int BITS>
__global__ void __launch_bounds__(256) k_xdigits(BatchArgs a)
{
    const int ng = a.D / kGroup;
    x_group_digits<BITS>(a, (blockIdx.x / ng) * 16, blockIdx.x % ng, threadIdx.x & 63, threadIdx.x >> 6);
}

// Hidden-dimension slices of the batched router: kRouteSplit when the
// slices stay multiples of 64 columns.
__host__ __device__ inline int route_splits(int D)
{
    for (int s = kRouteSplit; s > 1; s >>= 1)
        if (D % (64 * s) == 0) return s;
    return 1;
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

// The token -> expert grouping of the selections, by one block, from the
// pair ids in LDS (s_idx[t*K + k]): count[e], offset[e] (exclusive prefix
// sums), the pair permutation perm[pos] = t*K + k sorted by (expert, pair
// index), its inverse, the active experts in ascending order; and the
// expert kernels' dense work list: (item, tile of 16 of its tokens) for
// every active expert in that order (item = its rank) and then the shared
// expert (item n_act).  s_count .. s_nt hold E entries (E <= 4 blockDim);
// wsum: [blockDim / 64][3].
__device__ __forceinline__ void group_pairs(const BatchArgs &a, const int *s_idx, int *s_count, int *s_off, int *s_flag,
                                            int *s_nt, int (*wsum)[3])
{
    const int tid = threadIdx.x, nt = blockDim.x;
    const int T = a.T, K = a.K, E = a.E, P = T * K;
    for (int e = tid; e < E; e += nt) s_count[e] = 0;
    __syncthreads();
    for (int p = tid; p < P; p += nt) {
        const int e = s_idx[p];
        if (e >= 0 && e < E) atomicAdd(&s_count[e], 1);
        else atomicOr(a.flags, MOE_DEVERR_EXPERT_RANGE);
    }
    __syncthreads();
    for (int e = tid; e < E; e += nt) {
        s_off[e] = s_count[e];
        s_flag[e] = s_count[e] > 0;
        s_nt[e] = (s_count[e] + 15) / 16;
        a.count[e] = s_count[e];
    }
    __syncthreads();
    int tot[3];
    block_exscan3(s_off, s_flag, s_nt, E, wsum, tot);
    for (int e = tid; e < E; e += nt) {
        a.offset[e] = s_off[e];
        if (s_count[e]) {
            a.act[s_flag[e]] = e;
            for (int tt = 0; 16 * tt < s_count[e]; ++tt) a.mwork[s_nt[e] + tt] = s_flag[e] << 2 | tt;
        }
    }
    const bool shared = a.src.n_slots > K;
    if (shared && tid < (T + 15) / 16) a.mwork[tot[2] + tid] = tot[1] << 2 | tid;
    if (tid == 0) {
        a.offset[E] = tot[0];
        *a.n_act = tot[1];
        *a.n_mwork = tot[2] + (shared ? (T + 15) / 16 : 0);
    }
    for (int p = tid; p < P; p += nt) {
        const int e = s_idx[p];
        if (e < 0 || e >= E) {
            a.pos_of_pair[p] = -1;
            continue;
        }
        // rank among the expert's pairs: earlier pairs with the same id,
        // four ids per 16-byte LDS read
        int rank = 0, q = 0;
        const int4 *s4 = reinterpret_cast<const int4 *>(s_idx);
#pragma unroll 4
        for (; q + 4 <= p; q += 4) {
            const int4 v = s4[q >> 2];
            rank += (v.x == e) + (v.y == e) + (v.z == e) + (v.w == e);
        }
        for (; q < p; ++q) rank += s_idx[q] == e;
        const int pos = s_off[e] + rank;
        a.perm[pos] = p;
        a.pos_of_pair[p] = pos;
    }
}

// One block of 1024 threads: the grouping of the selections in topk_idx
// (given by the caller, or taken by k_topk_b for more than 512 experts).
__global__ void __launch_bounds__(1024) k_group(BatchArgs a)
{
    __shared__ __align__(16) int s_idx[64 * kMaxTopK];
    __shared__ int s_count[4096];
    __shared__ int s_off[4096];
    __shared__ int s_flag[4096];
    __shared__ int s_nt[4096];
    __shared__ int wsum[16][3];
    for (int p = threadIdx.x; p < a.T * a.K; p += blockDim.x) s_idx[p] = a.topk_idx[p];
    group_pairs(a, s_idx, s_count, s_off, s_flag, s_nt, wsum);
}

// ---------------------------------------------------------------------------
// Top-K of every token: one wave per token, its logits (the slices' partial
// logits added in slice order, also stored to logits[t]) in LDS; K rounds of
// the wave's largest remaining key (larger logit first, the lower index on a
// tie), then the softmax over the selected logits.  With `group` (E <= 512)
// the last block to finish also builds the grouping (k_group's work) from
// every token's selection: the selections go out as agent-scope stores, each
// block counts itself in with an agent-scope atomic once its stores are
// acknowledged, and the last one reads them back at agent scope; it resets
// the counter for the next call.
__global__ void __launch_bounds__(256) k_topk_b(BatchArgs a, int splits, int group)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int t = blockIdx.x * 4 + wave;
    const int E = a.E, K = a.K, T = a.T;
    __shared__ __align__(16) float lg[4][4096];
    __shared__ int s_sel[4][kMaxTopK], s_rdy[4][kMaxTopK];
    __shared__ float s_w[4][kMaxTopK];
    if (t < T) {
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
        if (E <= 64 * 8) {
            // the one-token kernels' selection on 32-bit order keys (same
            // order, ties and weights as below, fewer instructions per round)
            uint32_t ord[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int e = lane + 64 * u;
                ord[u] = e < E ? order_key(__float_as_uint(lg[wave][e])) : 0u;
            }
            topk_select<8>(ord, K, s_sel[wave], s_w[wave], s_rdy[wave], 1, lane);
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
            __builtin_amdgcn_wave_barrier();
            if (lane < K) {
                __hip_atomic_store(a.topk_idx + (size_t)t * K + lane, s_sel[wave][lane], __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
                a.topk_w[(size_t)t * K + lane] = s_w[wave][lane];
            }
        } else {
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
    }
    if (!group) return;  // uniform over the grid
    __shared__ int is_last;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t prev = __hip_atomic_fetch_add(a.grp_arrive, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        is_last = prev == gridDim.x - 1;
    }
    __syncthreads();
    if (!is_last) return;
    // the grouping's LDS in the finished top-K's logit rows (E <= 512):
    // pair ids, then count, offset, flag and tile count of every expert
    int *gs = reinterpret_cast<int *>(&lg[0][0]);
    __shared__ int wsum[4][3];
    for (int p = threadIdx.x; p < T * K; p += blockDim.x)
        gs[p] = __hip_atomic_load(a.topk_idx + p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    group_pairs(a, gs, gs + 64 * kMaxTopK, gs + 64 * kMaxTopK + 512, gs + 64 * kMaxTopK + 1024,
                gs + 64 * kMaxTopK + 1536, wsum);
    if (threadIdx.x == 0) *a.grp_arrive = 0u;
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

__device__ __forceinline__ int token_of(const BatchArgs &a, const Item &it, int j)
{
    return it.slot ? j : a.perm[it.pos0 + j] / a.K;
}

// ---------------------------------------------------------------------------
// Per token: combine in slot order (routed k = 0..K-1, then shared), then
// (mode 1) residual + RMSNorm; one block per token.  PER rows per thread
// (D <= 1024 PER), up to NS slots: every slot's rows, the residual rows and
// gamma are requested before the first sum, so that the block waits for one
// round trip instead of one per slot.
template <int PER, int NS>
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
    float yv[NS][PER], rr[PER], gg[PER];
#pragma unroll
    for (int k = 0; k < NS; ++k) {
        const int pk = k < K ? pos[k] : (k == K && has_shared ? a.T * K + t : -1);
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int o = tid + 1024 * j;
            yv[k][j] = k <= K && pk >= 0 && o < D ? a.y[(size_t)pk * D + o] : 0.f;
        }
    }
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int o = tid + 1024 * j;
        rr[j] = a.mode != 0 && o < D ? a.resid[(size_t)t * D + o] : 0.f;
        gg[j] = a.mode != 0 && o < D ? a.gamma[o] : 0.f;
    }
    float rv[PER];
    float ss = 0.f;
    // the combine of the token's rows first (the outputs never alias y),
    // summed in slot order, then residual and norm
#pragma unroll
    for (int j = 0; j < PER; ++j) rv[j] = 0.f;
#pragma unroll
    for (int k = 0; k < NS; ++k) {
        if (k > K) continue;
        const int pk = k < K ? pos[k] : (has_shared ? a.T * K + t : -1);
        if (pk < 0) continue;
        if (k < K) {
            const float wk = wts[k];
#pragma unroll
            for (int j = 0; j < PER; ++j) rv[j] += wk * yv[k][j];
        } else {
#pragma unroll
            for (int j = 0; j < PER; ++j) rv[j] += yv[k][j];
        }
    }
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int o = tid + 1024 * j;
        if (o >= D) continue;
        if (a.mode == 0) {
            a.yout[(size_t)t * D + o] = rv[j];
        } else {
            const float r = rr[j] + rv[j];
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
        if (o < D) a.xout[(size_t)t * D + o] = rv[j] * inv * gg[j];
    }
}

// ---------------------------------------------------------------------------
// Grouped expert contractions of a batch on the matrix cores, for every
// item (each active routed expert, then the shared expert):
//   MODE 0: the item's gate and up rows (I each) x the digit words of its
//           tokens' activations -> h[pos][i] = silu(g) * u, as digit words
//   MODE 1: its down rows (D) x the digit words of its positions' h
//           -> y[pos][o]
// A block unit is one entry of the work list (item, tile of 16 of its
// vectors) and one group of 64 WT rows; wave w takes WT tiles of 16 rows.
// The contraction runs in stages of SG scale groups: the block loads a
// stage's codes, scale words, digit words, group sums and steps with
// coalesced 16-byte loads into registers while it computes the previous
// stage from LDS.  One v_mfma_i32_16x16x64_i8 per (plane, matrix, scale group) takes
// the vectors' digit words of the plane as A (A-row l % 16, K-slice l / 16)
// and the group's masked codes as B (row l % 16), so a lane's C values are
// its own row's and it needs only that row's scale and bias word.  Vector
// slot t sits at A-row 4 (t % 4) + t / 4, so lane group l / 16 holds vectors
// l / 16 + 4 r: a tile of n vectors uses r < ceil(n / 4) only, and the
// epilogue, compiled for each such count, skips the rest.  The three plane
// sums are exact int32; the group's bf16 scale times the vector's step 2^-k
// for the group multiplies their fp32 combination, and the group's bias the
// vector's sum over the group.
// MODE 0 leaves h as digit words (a unit's 64 rows are one scale group of
// h), so the down rows read them as the gate/up rows read x's.
typedef int v4i __attribute__((ext_vector_type(4)));

// The MFMA A-row (and so C row) of a tile's vector slot t: 4 (t % 4) + t / 4.
// C row 4 h + r of lane group h is vector h + 4 r, so the first n vectors of
// a tile occupy the first ceil(n / 4) of a lane's four outputs.
__device__ __forceinline__ int arow(int t) { return 4 * (t & 3) + (t >> 2); }

template <int BITS, int SG>
struct MmShape {
    static constexpr int GB = 16 * BITS / 2;                       // code bytes per row and scale group
    static constexpr int ROWB = SG * GB + (BITS == 4 ? 32 : 16);   // LDS bytes per code row (padded)
    // LDS words per vector: a stride of 4 banks (mod 64) puts the 16 vectors
    // of a 16-byte digit read on distinct banks
    static constexpr int DIGROW = SG * kGroupWords + 4;
};

// A lane's 16 codes (K-slice h of scale group g) of an LDS code row, one per
// byte, in the order of the digit table's words.
template <int BITS>
__device__ __forceinline__ v4i codes_of(const uint8_t *row, int g, int h)
{
    using C = Codes<BITS>;
    v4i r;
    if constexpr (BITS == 4) {
        const uint2 w = *reinterpret_cast<const uint2 *>(row + 32 * g + 8 * h);
        r[0] = (int)(w.x & C::MASK);
        r[1] = (int)((w.x >> 4) & C::MASK);
        r[2] = (int)(w.y & C::MASK);
        r[3] = (int)((w.y >> 4) & C::MASK);
    } else {
        const uint32_t w = *reinterpret_cast<const uint32_t *>(row + 16 * g + 4 * h);
        r[0] = (int)(w & C::MASK);
        r[1] = (int)((w >> 2) & C::MASK);
        r[2] = (int)((w >> 4) & C::MASK);
        r[3] = (int)((w >> 6) & C::MASK);
    }
    return r;
}
// Digit words of plane p matching codes_of's slice h of group g, from a
// vector's digit words whose groups are kGroupWords apart.
template <int BITS>
__device__ __forceinline__ v4i digits_of(const int *dig, int g, int h, int p)
{
    using C = Codes<BITS>;
    const int *src;
    if constexpr (BITS == 4)
        src = dig + g * kGroupWords + (h >> 1) * C::DW + p * C::PW + 4 * (h & 1);
    else
        src = dig + g * kGroupWords + p * C::PW + 4 * h;
    const int4 v = *reinterpret_cast<const int4 *>(src);
    v4i r;
    r[0] = v.x;
    r[1] = v.y;
    r[2] = v.z;
    r[3] = v.w;
    return r;
}

template <int BITS, int MODE, int WT, int SG>
__global__ void __launch_bounds__(256) k_expert_mm(BatchArgs a)
{
    using C = Codes<BITS>;
    using S = MmShape<BITS, SG>;
    static_assert(C::DW * (kGroup / C::CODES) == kGroupWords, "a scale group's digit words");
    constexpr int M = MODE == 0 ? 2 : 1;
    constexpr int UR = 64 * WT;                               // rows per unit
    constexpr int CQ = UR * SG * S::GB / 16 / 256;            // code int4 per thread, matrix and stage
    constexpr int SQ = UR * SG / 256;                         // scale words per thread, matrix and stage
    constexpr int DQ = 16 * SG * kGroupWords / 4 / 256;       // digit int4 per thread and stage
    static_assert(CQ >= 1 && SQ >= 1 && DQ >= 1 && 16 * SG <= 256, "stage split over 256 threads");
    static_assert(MODE == 1 || UR == kGroup, "a gate/up unit's rows are one scale group of h");
    static_assert(SG % 4 == 0, "bias products take four groups at a time");
    static_assert(UR * SG * S::GB % (16 * 256) == 0 && UR * SG % 256 == 0 && 16 * SG * kGroupWords % 1024 == 0,
                  "whole stage loads per thread");
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r16 = lane & 15, h = lane >> 4;
    const int D = a.D, I = a.I;
    const int rows = MODE == 0 ? I : D, klen = MODE == 0 ? D : I;
    const int ng = klen / kGroup;
    const int rgroups = (rows + UR - 1) / UR, nst = (ng + SG - 1) / SG;
    const int nact = *a.n_act, nunits = *a.n_mwork * rgroups;
    const uint64_t mat_q = (uint64_t)I * D * BITS / 8, row_q = (uint64_t)klen * BITS / 8;
    const uint64_t sb0 = 3 * mat_q + (MODE == 0 ? 0 : 2 * (uint64_t)I * (D / kGroup) * 4);
    const uint64_t mat_sb = (uint64_t)rows * ng * 4;
    const int *dsrc = MODE == 0 ? a.xdig : a.hdig;
    const float *csrc = MODE == 0 ? a.xcsum : a.hcsum;
    const float *isrc = MODE == 0 ? a.xinv : a.hinv;
    __shared__ __align__(16) uint8_t s_code[M][UR][S::ROWB];
    __shared__ uint32_t s_sw[M][SG][UR];               // scale words [group][row]
    __shared__ __align__(16) int s_dig[16][S::DIGROW];
    __shared__ __align__(16) float s_gs[SG][16];       // group sums [group][vector]
    __shared__ __align__(16) float s_inv[SG][16];      // group steps [group][vector]
    __shared__ int s_vec[16];                          // the tile's vectors (token or position), -1 past n
    for (int u = blockIdx.x; u < nunits; u += gridDim.x) {
        const int wk = a.mwork[u / rgroups];
        const Item it = item_of(a, wk >> 2, nact);
        const int j0 = (wk & 3) * 16, row0 = (u % rgroups) * UR;
        // C rows 4 h + r hold vectors h + 4 r: a tile of n vectors fills
        // r = 0 .. ceil(n / 4) - 1, and the epilogue skips the other r
        const int nv = it.n - j0 < 16 ? it.n - j0 : 16;
        const int nr = __builtin_amdgcn_readfirstlane((nv + 3) >> 2);
        __syncthreads();  // the previous unit's readers of LDS are done
        if (tid < 16) {
            const int j = j0 + tid;
            s_vec[tid] = j < it.n ? (MODE == 0 ? token_of(a, it, j) : it.pos0 + j) : -1;
        }
        __syncthreads();
        // one stage's loads into registers (clamped rows, groups and
        // vectors: every load is in bounds).  Codes, scales and digits of
        // groups past ng are never multiplied (the group loop stops at ng),
        // and the outputs of vectors past the tile's are dropped, so the
        // clamped copies are stored as they are.
        // (native vector types: a struct copy would become a memcpy that keeps
        // these arrays in scratch memory)
        v4i rq[M][CQ];
        uint32_t rw[M][SQ];
        v4i rd[DQ];
        float rg = 0.f, ri = 0.f;
        auto load = [&](int g0) {
#pragma unroll
            for (int m = 0; m < M; ++m) {
                const uint8_t *mq = it.blob + (uint64_t)(MODE == 0 ? m : 2) * mat_q;
#pragma unroll
                for (int c = 0; c < CQ; ++c) {
                    const int f = tid + 256 * c, row = f / (SG * S::GB / 16);
                    const int b16 = f - row * (SG * S::GB / 16);
                    const int g = g0 + b16 * 16 / S::GB;
                    const uint64_t rr = row0 + row < rows ? row0 + row : rows - 1;
                    const uint64_t off = (uint64_t)(g < ng ? g : ng - 1) * S::GB + (uint64_t)(b16 * 16) % S::GB;
                    rq[m][c] = *reinterpret_cast<const v4i *>(mq + rr * row_q + off);
                }
                const uint8_t *ms = it.blob + sb0 + (uint64_t)m * mat_sb;
#pragma unroll
                for (int c = 0; c < SQ; ++c) {
                    const int f = tid + 256 * c, row = f / SG, g = g0 + (f - row * SG);
                    const uint64_t rr = row0 + row < rows ? row0 + row : rows - 1;
                    rw[m][c] = *reinterpret_cast<const uint32_t *>(ms + (rr * ng + (g < ng ? g : ng - 1)) * 4);
                }
            }
#pragma unroll
            for (int c = 0; c < DQ; ++c) {
                const int f = tid + 256 * c, t = f / (SG * kGroupWords / 4);
                const int rem = f - t * (SG * kGroupWords / 4), gl = rem / (kGroupWords / 4);
                const int w4 = rem - gl * (kGroupWords / 4), g = g0 + gl, vec = s_vec[t];
                const int vc = vec >= 0 ? vec : 0, gc = g < ng ? g : ng - 1;
                rd[c] = *reinterpret_cast<const v4i *>(dsrc + ((size_t)vc * ng + gc) * kGroupWords + 4 * w4);
            }
            {
                const int tt = tid & (16 * SG - 1);
                const int t = tt / SG, gl = tt - t * SG, g = g0 + gl, vec = s_vec[t];
                const int vc = vec >= 0 ? vec : 0, gc = g < ng ? g : ng - 1;
                rg = csrc[(size_t)vc * ng + gc];
                ri = isrc[(size_t)vc * ng + gc];
            }
        };
        auto store = [&](int g0) {
#pragma unroll
            for (int m = 0; m < M; ++m) {
#pragma unroll
                for (int c = 0; c < CQ; ++c) {
                    const int f = tid + 256 * c, row = f / (SG * S::GB / 16);
                    const int b16 = f - row * (SG * S::GB / 16);
                    *reinterpret_cast<v4i *>(&s_code[m][row][16 * b16]) = rq[m][c];
                }
#pragma unroll
                for (int c = 0; c < SQ; ++c) {
                    const int f = tid + 256 * c, row = f / SG, gl = f - row * SG;
                    s_sw[m][gl][row] = rw[m][c];
                }
            }
#pragma unroll
            for (int c = 0; c < DQ; ++c) {
                const int f = tid + 256 * c, t = f / (SG * kGroupWords / 4);
                const int rem = f - t * (SG * kGroupWords / 4);
                *reinterpret_cast<v4i *>(&s_dig[arow(t)][4 * rem]) = rd[c];
            }
            // group sums of groups past ng are zero: the bias products take
            // a stage's groups four at a time
            if (tid < 16 * SG) {
                const int t = tid / SG, gl = tid - t * SG;
                const bool ok = s_vec[t] >= 0 && g0 + gl < ng;
                s_gs[gl][arow(t)] = ok ? rg : 0.f;
                s_inv[gl][arow(t)] = ok ? ri : 0.f;
            }
        };
        float acs[M][WT][4];
        v4f acb[M][WT];
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int wt = 0; wt < WT; ++wt) {
                acb[m][wt] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int r = 0; r < 4; ++r) acs[m][wt][r] = 0.f;
            }
        load(0);
        store(0);
        __syncthreads();
        const int wrow0 = 16 * WT * wave + r16;  // the lane's row in the unit, tile 0
        for (int st = 0; st < nst; ++st) {
            const int g0 = st * SG;
            if (st + 1 < nst) load(g0 + SG);  // in flight while this stage is computed
            const int gn = ng - g0 < SG ? ng - g0 : SG;
            auto group = [&](int gl, auto NRc) {
                constexpr int NR = decltype(NRc)::value;
                v4i da[3];
#pragma unroll
                for (int p = 0; p < 3; ++p) da[p] = digits_of<BITS>(&s_dig[r16][0], gl, h, p);
                const float4 gi = *reinterpret_cast<const float4 *>(&s_inv[gl][4 * h]);
                const float iv[4] = {gi.x, gi.y, gi.z, gi.w};
                const v4i z = {0, 0, 0, 0};
#pragma unroll
                for (int m = 0; m < M; ++m)
#pragma unroll
                    for (int wt = 0; wt < WT; ++wt) {
                        const int wr = wrow0 + 16 * wt;
                        const v4i bq = codes_of<BITS>(&s_code[m][wr][0], gl, h);
                        const float sc = bf16_lo(s_sw[m][gl][wr]);
                        const v4i c0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(da[0], bq, z, 0, 0, 0);
                        const v4i c1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(da[1], bq, z, 0, 0, 0);
                        const v4i c2 = __builtin_amdgcn_mfma_i32_16x16x64_i8(da[2], bq, z, 0, 0, 0);
#pragma unroll
                        for (int r = 0; r < NR; ++r) {
                            float ps;
                            if constexpr (BITS == 2) {
                                // |c0 + 256 c1 + 65536 c2| < 3 * 64 * 2^22 < 2^31: exact in
                                // int32, one rounding to fp32
                                ps = (float)((((c2[r] << 8) + c1[r]) << 8) + c0[r]);
                            } else {
                                // (c0 + 256 c1) is exact in int32 and rounds once to fp32, as
                                // the one-token path's fma(c1, 256, c0) does
                                ps = fmaf((float)c2[r], 65536.f, (float)(c0[r] + (c1[r] << 8)));
                            }
                            acs[m][wt][r] = fmaf(sc * iv[r], ps, acs[m][wt][r]);
                        }
                    }
            };
            auto stage = [&](auto NRc) {
                if (BITS == 2 && gn == SG) {
                    // a whole stage: unrolled, so that one group's LDS reads and
                    // matrix-core work overlap the previous group's (at 4-bit the
                    // unrolled gate/up kernel would need more than 256 VGPRs)
#pragma unroll
                    for (int gl = 0; gl < SG; ++gl) group(gl, NRc);
                } else {
                    for (int gl = 0; gl < gn; ++gl) group(gl, NRc);
                }
            };
            switch (nr) {
            case 1: stage(std::integral_constant<int, 1>{}); break;
            case 2: stage(std::integral_constant<int, 2>{}); break;
            case 3: stage(std::integral_constant<int, 3>{}); break;
            default: stage(std::integral_constant<int, 4>{}); break;
            }
            // the stage's bias terms, four groups per v_mfma_f32_16x16x4f32:
            // A = group sums (vector l % 16, group l / 16), B = the rows' bias
            // halves (group l / 16, row l % 16); groups past ng have zero sums
#pragma unroll
            for (int q = 0; q < SG / 4; ++q) {
                const float ga = s_gs[4 * q + h][r16];
#pragma unroll
                for (int m = 0; m < M; ++m)
#pragma unroll
                    for (int wt = 0; wt < WT; ++wt)
                        acb[m][wt] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                            ga, bf16_hi(s_sw[m][4 * q + h][wrow0 + 16 * wt]), acb[m][wt], 0, 0, 0);
            }
            if (st + 1 < nst) {
                __syncthreads();  // every wave is done with this stage
                store(g0 + SG);
                __syncthreads();
            }
        }
        if constexpr (MODE == 0) {
            // h of the unit's 64 rows (one scale group g of h) for its 16
            // positions, through LDS, then as digit words: wave w converts
            // vectors 4 w .. 4 w + 3, one per DPP row
            __shared__ float s_h[16][kGroup + 1];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float g = acs[0][0][r] + acb[0][0][r], uu = acs[1][0][r] + acb[1][0][r];
                s_h[4 * h + r][wrow0] = g / (1.f + expf(-g)) * uu;
            }
            __syncthreads();
            const int t = 4 * wave + h;
            if (s_vec[t] >= 0) {
                float v[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) v[j] = s_h[arow(t)][group_value<BITS>(r16, j)];
                const size_t pg = ((size_t)it.pos0 + j0 + t) * (I / kGroup) + row0 / kGroup;
                group_digits<BITS>(v, r16, a.hdig + pg * kGroupWords, a.hcsum + pg, a.hinv + pg);
            }
        } else {
#pragma unroll
            for (int wt = 0; wt < WT; ++wt) {
                const int row = row0 + wrow0 + 16 * wt;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = h + 4 * r;
                    if (s_vec[t] < 0 || row >= rows) continue;
                    a.y[((size_t)it.pos0 + j0 + t) * D + row] = acs[0][wt][r] + acb[0][wt][r];
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
template <int BITS>
hipError_t batch_bits(const BatchArgs &a, int stage, hipStream_t s)
{
    switch (stage) {
    case 0:  // gate/up: 64-row units, 8 scale groups per stage
        // 512 blocks (two per CU at these kernels' registers); blocks take
        // further units in turn (2048 blocks measured 1 us slower for the
        // down rows of a 32-token step, 256 blocks 9 us slower)
        hipLaunchKernelGGL((k_expert_mm<BITS, 0, 1, 8>), dim3(512), dim3(256), 0, s, a);
        break;
    case 1:  // down: 128-row units (the digit tables of h shared by more rows)
        hipLaunchKernelGGL((k_expert_mm<BITS, 1, 2, (BITS == 4 ? 4 : 8)>), dim3(512), dim3(256), 0, s, a);
        break;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_batch_route(const BatchArgs &a, int do_topk, int bits, hipStream_t s)
{
    const int ttiles = (a.T + 15) / 16;
    if (do_topk) {
        const int splits = route_splits(a.D);
        const dim3 grid(splits * ((a.E + 15) / 16) * ttiles);
        if (bits == 4)
            hipLaunchKernelGGL(k_route_m<4>, grid, dim3(256), 0, s, a, splits);
        else
            hipLaunchKernelGGL(k_route_m<2>, grid, dim3(256), 0, s, a, splits);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        // up to 512 experts the top-K kernel's last block also groups
        const int group = a.E <= 512;
        hipLaunchKernelGGL(k_topk_b, dim3((a.T + 3) / 4), dim3(256), 0, s, a, splits, group);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if (group) return hipSuccess;
    } else {
        const dim3 grid(ttiles * (a.D / kGroup));
        if (bits == 4)
            hipLaunchKernelGGL(k_xdigits<4>, grid, dim3(256), 0, s, a);
        else
            hipLaunchKernelGGL(k_xdigits<2>, grid, dim3(256), 0, s, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k_group, dim3(1), dim3(1024), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_batch_experts(const BatchArgs &a, int bits, hipStream_t s)
{
    for (int stage = 0; stage < 2; ++stage) {
        hipError_t e = bits == 4 ? batch_bits<4>(a, stage, s) : batch_bits<2>(a, stage, s);
        if (e != hipSuccess) return e;
    }
    // rows per thread and slots of the combine
    const int ns = a.K + (a.src.n_slots > a.K ? 1 : 0);
    if (a.D <= 4096 && ns <= 5)
        hipLaunchKernelGGL((k_combine_b<4, 5>), dim3(a.T), dim3(1024), 0, s, a);
    else if (a.D <= 4096)
        hipLaunchKernelGGL((k_combine_b<4, kMaxSlots>), dim3(a.T), dim3(1024), 0, s, a);
    else
        hipLaunchKernelGGL((k_combine_b<8, kMaxSlots>), dim3(a.T), dim3(1024), 0, s, a);
    return hipGetLastError();
}

}  // namespace moe
