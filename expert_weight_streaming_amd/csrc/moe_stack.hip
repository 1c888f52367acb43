// moe_stack.hip -- a stack of MoE layers (batch 1) in one persistent launch.
//
// Per token and layer the pages' engine routes, fetches the selected
// experts, runs them, and hands the combined, normalised result to the
// next layer (hakusoku.com, "パイプライン概要" and "主要技術"; toolarium.ru,
// "Оптимизации, которые сработали").  Here every layer of a token runs in
// one launch of one 512-thread block per CU, and a layer is three phases
// separated by grid barriers:
//
//   A  x_l = RMSNorm(r_l) * gamma_{l-1} (every block, from the residual rows
//      the previous layer published), its digit table, router rows
//                                                            -> barrier
//   B  top-K in every block (no broadcast round trip), the shared expert's
//      gate/up rows beside the top-K's final merge, then the routed
//      experts' gate/up rows                                 -> barrier
//   C  h of every slot and its digit tables in LDS; down rows of all slots,
//      combined in slot order, plus the residual; per-block sum of squares
//                                                            -> barrier
//
// The weights a phase reads never depend on that phase's activations, so
// each wave issues its weight loads as early as the data dependencies allow
// and holds them in registers across barriers:
//   - the next layer's router rows are issued between arriving at the
//     layer's last barrier and waiting for it, the shared expert's gate/up
//     rows likewise at the first barrier, the routed down rows at the
//     second (so that the routed gate/up rows before it have the memory
//     system to themselves).
// Arrival waits for the block's stores, which must not queue behind a
// prefetch, so every prefetch is issued after an arrival.
// With one unit of work per wave at the pages' shape (hidden 4096, 512
// experts, K=4 + shared, inter 1024: 2048 waves), every phase is a single
// round of loads.  Larger shapes loop; the first unit is the prefetched one.
//
// Arithmetic per layer is that of moe_layer_step's definition: every sum
// runs in a fixed order (no float atomics), every block derives the same
// RMS factor from the same partial sums in the same order, so results are
// deterministic and a stack launch equals the same layers launched one by
// one, bit for bit.
#include "moe_device.h"

#ifndef MOE_STACK_BITS
#error "compile with -DMOE_STACK_BITS=4 or 2"
#endif

namespace moe {
namespace {

using namespace dev;

constexpr int NT = kStackThreads;  // threads per block
constexpr int NWB = NT / 64;       // waves per block
constexpr int RN = 4;              // router float4 per lane and round
constexpr int RSL = 4;             // waves per router row
constexpr int RPB = NWB / RSL;     // router rows per block and round

// The RMS factor from this thread's share t of the per-block partial sums
// of squares (thread q holds blocks q, q + NT, ...): every block adds the
// same values in the same order, so every block gets the same factor.
// Uses red[0..NWB).
__device__ __forceinline__ float rms_inv(float t, int D, float eps, float *red)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    t = group_sum<64>(t);
    if (lane == 0) red[wave] = t;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < NWB; ++w) tot += red[w];
    __syncthreads();
    return 1.f / sqrtf(tot / (float)D + eps);
}

constexpr int RV = 4;  // residual float4 per thread: D / 4 <= RV * NT

// Values that the compiler must not keep live across the layer loop: a
// persistent kernel's loop body would otherwise have every lane-dependent
// address of every phase hoisted out of it, all live at once.
__device__ __forceinline__ int opaque_v(int v)
{
    asm volatile("" : "+v"(v));
    return v;
}
// The kernel's arguments, read in place from the kernarg segment (scalar
// loads) and re-read per layer instead of being held in registers.
typedef const __attribute__((address_space(4))) StackArgs *KArgs;
__device__ __forceinline__ KArgs kargs()
{
    KArgs p = (KArgs)__builtin_amdgcn_kernarg_segment_ptr();
    asm volatile("" : "+s"(p));
    return p;
}
__device__ __forceinline__ StackLayer layer_of(KArgs A, int l)
{
    StackLayer y;
    y.router = A->layer[l].router;
    y.gamma = A->layer[l].gamma;
    y.experts = A->layer[l].experts;
    y.shared = A->layer[l].shared;
    y.slab = A->layer[l].slab;
    return y;
}

template <int BITS, int GCPL, int LPR, int DCPL, int MAXS>
__global__ void __launch_bounds__(NT) k_stack(StackArgs args)
{
    using C = Codes<BITS>;
    constexpr int RPU = 64 / LPR;  // down rows per wave unit
    extern __shared__ __align__(16) unsigned char smem[];

    // The barrier slots of a workspace belong to one grid size.
    const uint32_t hdr = __hip_atomic_load(args.hdr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (hdr != 0u && hdr != gridDim.x) {
        if (threadIdx.x == 0 && blockIdx.x == 0) atomicOr(args.flags, MOE_DEVERR_WORKSPACE);
        return;
    }
    GridBar g;
    g.slots = args.slots;
    g.base = __hip_atomic_load(args.slots + blockIdx.x * kSlotWords, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    g.nb = gridDim.x;
    g.flags = args.flags;
    uint32_t bar = 0;

    RtRegs<RN> ra;
    GuRegs<BITS, GCPL, 1> ga;
    // Router loads of a layer: this wave's slice of row b + NB*rs (the first
    // round of the layer's router rows).
    auto prefetch_router = [&](KArgs A, int l) {
        const int tid = opaque_v(threadIdx.x), lane = tid & 63;
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int NB = gridDim.x, b = blockIdx.x;
        const int D = A->D, E = A->E;
        const int nc4 = D / 4, Q = (nc4 + RSL - 1) / RSL, rs = wave / RSL, sw = wave % RSL;
        const StackLayer Ly = layer_of(A, l);
        const int e = b + NB * rs;
        rt_load<RN>(ra, e < E ? Ly.router + (size_t)e * D : nullptr, sw * Q, min(nc4, sw * Q + Q), lane);
    };
    prefetch_router(kargs(), 0);

    for (int l = 0; l < args.n_layers; ++l) {
        KArgs A = kargs();
        const int tid = opaque_v(threadIdx.x), lane = tid & 63;
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int NB = gridDim.x, b = blockIdx.x;
        const int gw = wave * NB + b, GW = NB * NWB;
        const int D = A->D, E = A->E, K = A->K, I = A->I, S = A->n_slots;
        const uint64_t bb = A->blob_bytes;
        const StackLayer Ly = layer_of(A, l);

        const StackLds lo = stack_lds(D, E, I, S, BITS);
        float *xs = reinterpret_cast<float *>(smem + lo.xs);
        int *dig = reinterpret_cast<int *>(smem + lo.dig);
        float *csum = reinterpret_cast<float *>(smem + lo.csum);
        float *lg = reinterpret_cast<float *>(smem + lo.u);  // logits in phase B ...
        float *hs = reinterpret_cast<float *>(smem + lo.u);  // ... h in phase C
        int *hdig = reinterpret_cast<int *>(smem + lo.hdig);
        float *hcsum = reinterpret_cast<float *>(smem + lo.hcsum);
        float *misc = reinterpret_cast<float *>(smem + lo.misc);
        float *red = misc;                                              // [16]
        float *rpart = misc + 16;                                       // [8]
        int *ncand = reinterpret_cast<int *>(misc + 24);                // [1]
        int *sel = reinterpret_cast<int *>(misc + 32);                  // [8]
        float *selw = misc + 40;                                        // [8]
        float *hmul = misc + 48;                                        // [16]
        float *hinv = misc + 64;                                        // [16]
        float *sspart = misc + 80;                                      // [16]
        uint64_t *wmax = reinterpret_cast<uint64_t *>(misc + 96);       // [8]
        uint64_t *sk = reinterpret_cast<uint64_t *>(misc + 112);        // [8]
        uint64_t *cand = reinterpret_cast<uint64_t *>(misc + 128);      // [64]

        // Slot k's blob of this layer (sel[] holds the layer's selection).
        auto blob_k = [&](int k) -> const uint8_t * {
            if (Ly.slab) return Ly.slab + (uint64_t)k * bb;
            if (k >= K) return Ly.shared;
            const int e = __builtin_amdgcn_readfirstlane(sel[k]);
            if (e < 0 || e >= E) {
                atomicOr(A->flags, MOE_DEVERR_EXPERT_RANGE);
                return nullptr;
            }
            return Ly.experts + (uint64_t)e * bb;
        };

        // ---- phase A: the layer's input activation
        if (l == 0) {
            for (int d4 = tid; d4 < D / 4; d4 += NT) {
                const float4 xv = reinterpret_cast<const float4 *>(A->x)[d4];
                reinterpret_cast<float4 *>(xs)[d4] = xv;
                if (A->record && b == 0) {
                    reinterpret_cast<float4 *>(A->record)[d4] = reinterpret_cast<const float4 *>(A->resid)[d4];
                    reinterpret_cast<float4 *>(A->record + D)[d4] = xv;
                }
            }
        } else {
            // the previous layer's residual rows and partial sums of squares
            // in one round trip
            float t = 0.f;
            for (int q = tid; q < NB; q += NT) t += xload(A->ss + q);
            float4 rv[RV];
#pragma unroll
            for (int j = 0; j < RV; ++j) {
                const int d4 = tid + j * NT;
                rv[j] = d4 < D / 4 ? xload4(A->rbuf, 4 * d4) : make_float4(0.f, 0.f, 0.f, 0.f);
            }
            const float inv = rms_inv(t, D, A->eps, red);
            const float4 *gm = reinterpret_cast<const float4 *>(A->layer[l - 1].gamma);
#pragma unroll
            for (int j = 0; j < RV; ++j) {
                const int d4 = tid + j * NT;
                if (d4 >= D / 4) continue;
                const float4 r = rv[j];
                const float4 gv = gm[d4];
                const float4 xv = make_float4(r.x * inv * gv.x, r.y * inv * gv.y, r.z * inv * gv.z, r.w * inv * gv.w);
                reinterpret_cast<float4 *>(xs)[d4] = xv;
                if (A->record && b == 0) {
                    reinterpret_cast<float4 *>(A->record + (size_t)l * 2 * D)[d4] = r;
                    reinterpret_cast<float4 *>(A->record + (size_t)l * 2 * D + D)[d4] = xv;
                }
            }
        }
        __syncthreads();
        const float xinv = block_digit_table<BITS>(xs, D, dig, csum, red);

        // router rows: RSL waves per row, RPB rows per block and round
        {
            const int nc4 = D / 4, Q = (nc4 + RSL - 1) / RSL, rs = wave / RSL, sw = wave % RSL;
            for (int j = 0; b + NB * RPB * j < E; ++j) {
                const int e = b + NB * (RPB * j + rs);
                float acc = 0.f;
                for (int c0 = 0; c0 < Q; c0 += 64 * RN) {
                    const int c_lo = sw * Q + c0, c_hi = min(nc4, sw * Q + Q);
                    if (j > 0 || c0 > 0) rt_load<RN>(ra, e < E ? Ly.router + (size_t)e * D : nullptr, c_lo, c_hi, lane);
                    acc += rt_finish<RN>(ra, xs, c_lo, c_hi, lane);
                }
                acc = group_sum<64>(acc);
                if (lane == 0) rpart[wave] = acc;
                __syncthreads();
                if (tid < RPB) {
                    const int ee = b + NB * (RPB * j + tid);
                    if (ee < E) {
                        float v = rpart[tid * RSL];
#pragma unroll
                        for (int q = 1; q < RSL; ++q) v += rpart[tid * RSL + q];
                        xstore(A->logits + ee, v);
                    }
                }
                __syncthreads();
            }
        }

        // barrier 1; the shared expert's gate/up rows (needed in phase B, by
        // waves 1..NWB-1) are requested between arrival and wait
        grid_arrive(g, ++bar);
        const uint8_t *sh = S > K ? (Ly.slab ? Ly.slab + (uint64_t)K * bb : Ly.shared) : nullptr;
        const int su0 = b + NB * (wave - 1);  // first shared unit of waves >= 1
        gu_load<BITS, GCPL, 1>(ga, wave > 0 && su0 < I ? sh : nullptr, D, I, su0, lane);
        grid_wait(g, bar);

        // ---- phase B: top-K, then the routed gate/up rows
        for (int e = tid; e < E; e += NT) lg[e] = xload(A->logits + e);
        __syncthreads();
        block_topk_fast<NWB>(lg, E, K, cand, wmax, sk, ncand, sel, selw);
        if (b == 0 && tid < K) {
            A->topk_idx[l * K + tid] = sel[tid];
            A->topk_w[l * K + tid] = selw[tid];
        }
        const int upe = (I + 1) / 2;  // routed gate/up units per expert (2 rows)
        const int nd = (D + RPU - 1) / RPU;
        GuRegs<BITS, GCPL, 2> gb;
        {
            const int k = gw / upe;
            gu_load<BITS, GCPL, 2>(gb, gw < K * upe ? blob_k(k) : nullptr, D, I, (gw - k * upe) * 2, lane);
        }
        // the shared expert's gate/up rows (loaded at barrier 1) while the
        // routed rows are in flight
        if (S > K && wave > 0) {
            float *hsh = A->h + (size_t)K * I;
            for (int u = su0, j = 0; u < I; u += NB * (NWB - 1), ++j) {
                if (j > 0) gu_load<BITS, GCPL, 1>(ga, sh, D, I, u, lane);
                gu_finish<BITS, GCPL, 1>(ga, dig, csum, xinv, D, I, u, lane, hsh);
            }
        }
        for (int u = gw, j = 0; u < K * upe; u += GW, ++j) {
            const int k = u / upe, i0 = (u - k * upe) * 2;
            if (j > 0) gu_load<BITS, GCPL, 2>(gb, blob_k(k), D, I, i0, lane);
            gu_finish<BITS, GCPL, 2>(gb, dig, csum, xinv, D, I, i0, lane, A->h + (size_t)k * I);
        }
        // barrier 2; the down rows of every slot (needed right after it)
        // stream in while the block waits
        grid_arrive(g, ++bar);
        DnRegs<BITS, DCPL> dn[MAXS];
#pragma unroll
        for (int k = 0; k < MAXS; ++k)
            dn_load<BITS, LPR, DCPL>(dn[k], (k < S && gw < nd) ? blob_k(k) : nullptr, D, I, gw * RPU, lane);
        grid_wait(g, bar);

        // ---- phase C: h of every slot into LDS and its digit tables
        const int cpk = I / C::CODES;  // h chunks per slot
        for (int q = tid; q < S * I / 4; q += NT) reinterpret_cast<float4 *>(hs)[q] = xload4(A->h, 4 * q);
        __syncthreads();
        for (int k = wave; k < S; k += NWB) {
            float m = 0.f;
            for (int i = lane; i < I; i += 64) m = fmaxf(m, fabsf(hs[k * I + i]));
            m = group_max<64>(m);
            if (lane == 0) {
                float mul, inv;
                fixed_scale(m, mul, inv);
                hmul[k] = mul;
                hinv[k] = inv;
            }
        }
        __syncthreads();
        for (int t = tid; t < S * cpk * 4 * C::SUBS; t += NT) {
            const int kc = t / (4 * C::SUBS), r = t - kc * 4 * C::SUBS;
            const int kw = r / C::SUBS, s = r - kw * C::SUBS;
            const float mul = hmul[kc / cpk];
            const float *v = hs + kc * C::CODES + kw * C::PER_WORD + s;
            int *o = hdig + kc * C::DW + kw * C::SUBS + s;
            digit_words(v[0], v[C::SUBS], v[2 * C::SUBS], v[3 * C::SUBS], mul, o[0], o[C::PW], o[2 * C::PW]);
        }
        chunk_sums<BITS>(hs, S * cpk, hcsum);
        __syncthreads();

        // down rows of all slots, combined in slot order, plus the residual
        float ssacc = 0.f;
        for (int u = gw, j = 0; u < nd; u += GW, ++j) {
            const int o0 = u * RPU, o = o0 + lane / LPR;
            const bool owner = lane % LPR == 0 && o < D;
            float r = 0.f;
            if (owner) r = l == 0 ? A->resid[o] : xload(A->rbuf + o);
            if (j > 0) {
#pragma unroll
                for (int k = 0; k < MAXS; ++k) dn_load<BITS, LPR, DCPL>(dn[k], k < S ? blob_k(k) : nullptr, D, I, o0, lane);
            }
            // slot partials weighted per lane, in slot order, then one
            // reduction over the row's lanes
            float c = 0.f;
#pragma unroll
            for (int k = 0; k < MAXS; ++k) {
                if (k >= S) continue;
                const float y = dn_part<BITS, LPR, DCPL>(dn[k], hdig + k * cpk * C::DW, hcsum + k * cpk, hinv[k], I, lane);
                c = fmaf(k < K ? selw[k] : 1.f, y, c);
            }
            c = group_sum<LPR>(c);
            if (owner) {
                const float rn = r + c;
                xstore(A->rbuf + o, rn);
                ssacc = fmaf(rn, rn, ssacc);
            }
        }
        ssacc = group_sum<64>(ssacc);
        if (lane == 0) sspart[wave] = ssacc;
        __syncthreads();
        if (tid == 0) {
            float t = 0.f;
#pragma unroll
            for (int w = 0; w < NWB; ++w) t += sspart[w];
            xstore(A->ss + b, t);
        }
        grid_arrive(g, ++bar);
        if (l + 1 < A->n_layers) prefetch_router(A, l + 1);
        grid_wait(g, bar);
    }

    // ---- the stack's output: residual stream and its normalisation
    {
        KArgs A = kargs();
        const int tid = threadIdx.x, NB = gridDim.x, b = blockIdx.x, D = A->D, L = A->n_layers;
        float *red = reinterpret_cast<float *>(smem + stack_lds(D, A->E, A->I, A->n_slots, BITS).misc);
        float t = 0.f;
        for (int q = tid; q < NB; q += NT) t += xload(A->ss + q);
        const float inv = rms_inv(t, D, A->eps, red);
        const float4 *gm = reinterpret_cast<const float4 *>(A->layer[L - 1].gamma);
        for (int d4 = b * NT + tid; d4 < D / 4; d4 += NB * NT) {
            const float4 r = xload4(A->rbuf, 4 * d4);
            const float4 gv = gm[d4];
            const float4 xv = make_float4(r.x * inv * gv.x, r.y * inv * gv.y, r.z * inv * gv.z, r.w * inv * gv.w);
            reinterpret_cast<float4 *>(A->resid)[d4] = r;
            reinterpret_cast<float4 *>(A->x)[d4] = xv;
            if (A->record) {
                reinterpret_cast<float4 *>(A->record + (size_t)L * 2 * D)[d4] = r;
                reinterpret_cast<float4 *>(A->record + (size_t)L * 2 * D + D)[d4] = xv;
            }
        }
        if (tid == 0 && b == 0) __hip_atomic_store(A->hdr, (uint32_t)NB, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Launch plan per instantiation and device: one block per CU when the
// kernel needs no scratch and one block with this LDS fits a CU.
struct StackPlanCache {
    int ready = 0, vgprs = 0, scratch = 0, n_cu = 0;
};

template <int GCPL, int LPR, int DCPL, int MAXS>
hipError_t stack_launch(const StackArgs *a, int D, int E, int I, int S, hipStream_t s, LayerPlan *p)
{
    auto kern = k_stack<MOE_STACK_BITS, GCPL, LPR, DCPL, MAXS>;
    static StackPlanCache cache[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    StackPlanCache c = dev < 64 ? cache[dev] : StackPlanCache{};
    if (!c.ready) {
        hipFuncAttributes attr;
        if ((e = hipFuncGetAttributes(&attr, reinterpret_cast<const void *>(kern))) != hipSuccess) return e;
        c.vgprs = attr.numRegs;
        c.scratch = (int)attr.localSizeBytes;
        if ((e = hipDeviceGetAttribute(&c.n_cu, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
        // allow up to the CU's 160 KB of LDS; should the runtime refuse, the
        // occupancy query below decides
        if (hipFuncSetAttribute(reinterpret_cast<const void *>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                160 * 1024) != hipSuccess)
            (void)hipGetLastError();
        c.ready = 1;
        if (dev < 64) cache[dev] = c;
    }
    const StackLds lo = stack_lds(D, E, I, S, MOE_STACK_BITS);
    int per_cu = 0;
    if (lo.total <= 160u * 1024u &&
        (e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void *>(kern), NT, lo.total)) !=
            hipSuccess)
        return e;
    p->block = NT;
    p->per_cu = per_cu;
    p->n_cu = c.n_cu;
    p->vgprs = c.vgprs;
    p->scratch = c.scratch;
    p->grid = (c.scratch == 0 && per_cu >= 1 && lo.total <= 160u * 1024u) ? (c.n_cu < kMaxLayerBlocks ? c.n_cu : kMaxLayerBlocks) : 0;
    if (!a) return hipSuccess;
    if (p->grid == 0) return hipErrorNotSupported;
    hipLaunchKernelGGL(kern, dim3(p->grid), dim3(NT), lo.total, s, *a);
    return hipGetLastError();
}

// Shape -> instantiation.  Gate/up: GCPL chunks per lane and row.  Down: the
// smallest power-of-two LPR >= the row's chunks (8..64), DCPL chunks per lane.
template <int GCPL>
hipError_t stack_g(const StackArgs *a, int D, int E, int I, int S, hipStream_t s, LayerPlan *p)
{
    const int nch = I * MOE_STACK_BITS / 128;
    const bool wide = S > 5;
#define MOE_S(LPR_, DCPL_)                                                                                              \
    return wide ? stack_launch<GCPL, LPR_, DCPL_, kMaxSlots>(a, D, E, I, S, s, p)                                       \
                : stack_launch<GCPL, LPR_, DCPL_, 5>(a, D, E, I, S, s, p);
    if (nch <= 8) MOE_S(8, 1)
    if (nch <= 16) MOE_S(16, 1)
    if (nch <= 32) MOE_S(32, 1)
    if (nch <= 64) MOE_S(64, 1)
    MOE_S(64, 2)
#undef MOE_S
}

}  // namespace

#if MOE_STACK_BITS == 4
hipError_t stack_bits4(const StackArgs *a, int D, int E, int I, int S, hipStream_t s, LayerPlan *p)
#else
hipError_t stack_bits2(const StackArgs *a, int D, int E, int I, int S, hipStream_t s, LayerPlan *p)
#endif
{
    const int nch = D * MOE_STACK_BITS / 128;
    if (nch <= 64) return stack_g<1>(a, D, E, I, S, s, p);
    if constexpr (MOE_STACK_BITS == 4) {
        if (nch <= 128) return stack_g<2>(a, D, E, I, S, s, p);
        return stack_g<4>(a, D, E, I, S, s, p);
    } else {
        return stack_g<2>(a, D, E, I, S, s, p);
    }
}

}  // namespace moe
