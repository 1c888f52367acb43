// moe_stack.hip -- a stack of MoE layers (batch 1) in one persistent launch.
//
// Per token and layer the pages' engine routes, fetches the selected
// experts, runs them, and hands the combined, normalised result to the
// next layer (hakusoku.com, "パイプライン概要" and "主要技術"; toolarium.ru,
// "Оптимизации, которые сработали").  Here every layer of a token runs in
// one launch of one 512-thread block per CU, and every wave of a block
// takes part in every phase:
//
//   A  x_l = RMSNorm(r_l) * gamma_{l-1} in every block, from the residual
//      rows and sums of squares the previous layer published, and x_l's
//      digit table; the block's router rows (four waves per row); the
//      logits go out tagged
//   B  wave 0 polls the logits and takes the top-K, publishing each
//      selected index (LDS) as soon as its round ends; waves 1.. run the
//      shared expert's gate/up rows (loaded a layer ahead) meanwhile; then
//      every wave its unit of routed gate/up rows as soon as its slot's
//      expert is known; h goes out tagged and the down rows of every slot
//      are requested
//   C  h of every slot, polled, as digit tables; the next layer's router
//      and shared rows are requested; down rows of all slots, combined in
//      slot order; r' = r + c for the block's rows and the block's sum of
//      squares go out tagged
//
// Blocks never meet at a grid barrier.  Every value handed from block to
// block (logits, h, residual rows, sums of squares) is a 64-bit word that
// carries the epoch of the exchange that produced it (tag_store); a reader
// polls the words it needs until each carries the expected epoch.  A
// producer therefore never waits for its own stores to be acknowledged,
// and a consumer waits only for the values it reads.  Epochs grow by three
// per layer and carry over from launch to launch through per-block slots
// in the workspace, so nothing is ever reset.  Inside a block every
// barrier is LDS-only.
//
// Digit tables are built in registers with one fixed-point step per
// 16-byte code chunk (chunk_digits_lane): no block-wide maximum, no LDS
// pass over the activations.
//
// Arithmetic per layer is that of moe_layer_step's definition: every sum
// runs in a fixed order (no float atomics), every block and every wave
// derives the same RMS factor from the same partial sums in the same order,
// and one top-K per block from the same logits, so results are
// deterministic and equal, bit for bit, from launch to launch.
#include "moe_device.h"

#ifndef MOE_STACK_BITS
#error "compile with -DMOE_STACK_BITS=4 or 2"
#endif

namespace moe {
namespace {

using namespace dev;

constexpr int NT = kStackThreads;  // threads per block
constexpr int NWB = NT / 64;       // waves per block
constexpr int RN = kRouterRN;      // router float4 per lane and load round
constexpr int RSL = kRouterSlices; // waves per router row
constexpr int RPB = NWB / RSL;     // router rows per block and round
constexpr int XV = 2;              // x float4 per thread and round
constexpr int HV = 3;              // h float4 per thread and round
constexpr int KPL = 8;             // top-K keys per lane: E <= 512
constexpr uint32_t kTagSpins = 1u << 16;  // polls of an exchange before it is given up (error flag)

// Timeline builds (-DMOE_STACK_PROBE): lane 0 of every wave stores the
// device's constant-rate clock (s_memrealtime) at fixed points of each
// layer into args.probe; other builds compile the points away.
#ifdef MOE_STACK_PROBE
#define MOE_PROBE(P)                                                                                                   \
    do {                                                                                                               \
        if (A->probe && (threadIdx.x & 63) == 0)                                                                       \
            A->probe[(((size_t)l * gridDim.x + blockIdx.x) * NWB + (threadIdx.x >> 6)) * kProbePoints + (P)] =         \
                __builtin_amdgcn_s_memrealtime();                                                                      \
    } while (0)
#else
#define MOE_PROBE(P) ((void)0)
#endif

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
// TBL: the launch has layers in address-table mode (a separate
// instantiation, so that the other launches pay nothing for it)
template <bool TBL>
__device__ __forceinline__ StackLayer layer_of(KArgs A, int l)
{
    StackLayer y;
    y.router = A->layer[l].router;
    y.gamma = A->layer[l].gamma;
    y.experts = A->layer[l].experts;
    y.addr = TBL ? A->layer[l].addr : nullptr;
    y.shared = A->layer[l].shared;
    y.slab = A->layer[l].slab;
    return y;
}

// Per-layer LDS views.
struct Views {
    float *xs, *rs, *csum, *xcinv, *u, *hcsum, *hcinv, *yh, *misc;
    int *dig, *hdig;
};
template <int BITS>
__device__ __forceinline__ Views views(unsigned char *smem, int D, int E, int I, int S)
{
    const StackLds lo = stack_lds(D, E, I, S, BITS);
    Views v;
    v.xs = reinterpret_cast<float *>(smem + lo.xs);
    v.rs = reinterpret_cast<float *>(smem + lo.rs);
    v.dig = reinterpret_cast<int *>(smem + lo.dig);
    v.csum = reinterpret_cast<float *>(smem + lo.csum);
    v.xcinv = reinterpret_cast<float *>(smem + lo.xcinv);
    v.u = reinterpret_cast<float *>(smem + lo.u);  // router partials (A), combined rows (C)
    v.hdig = reinterpret_cast<int *>(smem + lo.hdig);
    v.hcsum = reinterpret_cast<float *>(smem + lo.hcsum);
    v.hcinv = reinterpret_cast<float *>(smem + lo.hcinv);
    v.yh = reinterpret_cast<float *>(smem + lo.yh);
    v.misc = reinterpret_cast<float *>(smem + lo.misc);
    return v;
}

// Slot k's blob of layer Ly under the selection sel (LDS).
template <bool TBL>
__device__ __forceinline__ const uint8_t *slot_blob(KArgs A, const StackLayer &Ly, const int *sel, int k)
{
    const uint64_t bb = A->blob_bytes;
    if (Ly.slab) return Ly.slab + (uint64_t)k * bb;
    if (k >= A->K) return Ly.shared;
    const int e = __builtin_amdgcn_readfirstlane(sel[k]);
    if (e < 0 || e >= A->E) {
        atomicOr(A->flags, MOE_DEVERR_EXPERT_RANGE);
        return nullptr;
    }
    if constexpr (TBL)
        if (Ly.addr) return reinterpret_cast<const uint8_t *>(Ly.addr[e]);
    return Ly.experts + (uint64_t)e * bb;
}
__device__ __forceinline__ const uint8_t *shared_blob(KArgs A, const StackLayer &Ly)
{
    if (A->n_slots <= A->K) return nullptr;
    return Ly.slab ? Ly.slab + (uint64_t)A->K * A->blob_bytes : Ly.shared;
}

// Residual rows and per-block sums of squares of the previous layer, from
// their tagged words: polls until every word this thread reads carries
// epoch `tag`.  rv[j] receives float4 q0 + tid + j*NT of the residual; the
// return value is this lane's share of the NB partial sums (blocks
// 4*lane + 256*i .. +3, added in that order).  Every wave polls and adds the
// same way.
template <int NV>
__device__ __forceinline__ float poll_residual(KArgs A, int q0, int D, int NB, uint32_t tag, bool with_ss, float4 (&rv)[NV])
{
    const int tid = threadIdx.x, lane = tid & 63;
    constexpr int SI = kMaxLayerBlocks / 256;
    uint4 sa[SI], sc[SI], ra[NV], rc[NV];
    bool ns[SI], nr[NV];
#pragma unroll
    for (int i = 0; i < SI; ++i) {
        ns[i] = with_ss && 256 * i + 4 * lane < NB;
        sa[i] = sc[i] = make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        nr[j] = q0 + tid + j * NT < D / 4;
        ra[j] = rc[j] = make_uint4(0, 0, 0, 0);
    }
    for (uint32_t spins = 0;;) {
        bool ok = true;
#pragma unroll
        for (int i = 0; i < SI; ++i) {
            const int p = 256 * i + 4 * lane;
            const uint4 a = tag_load2_if(A->tss, p, ns[i]), c = tag_load2_if(A->tss, p + 2, ns[i]);
            const bool g = (p >= NB || a.y == tag) && (p + 1 >= NB || a.w == tag) && (p + 2 >= NB || c.y == tag) &&
                           (p + 3 >= NB || c.w == tag);
            if (ns[i]) {
                sa[i] = a;
                sc[i] = c;
                ok &= g;
                ns[i] = !g;
            }
        }
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int q = q0 + tid + j * NT;
            const uint4 a = tag_load2_if(A->tres, 4 * q, nr[j]), c = tag_load2_if(A->tres, 4 * q + 2, nr[j]);
            const bool g = a.y == tag && a.w == tag && c.y == tag && c.w == tag;
            if (nr[j]) {
                ra[j] = a;
                rc[j] = c;
                ok &= g;
                nr[j] = !g;
            }
        }
        if (__all(ok)) break;
        __builtin_amdgcn_s_sleep(1);
        if (++spins == kTagSpins) {
            atomicOr(A->flags, MOE_DEVERR_BARRIER_TIMEOUT);
            break;
        }
    }
    float t = 0.f;
#pragma unroll
    for (int i = 0; i < SI; ++i) {
        const int p = 256 * i + 4 * lane;
        if (256 * i < NB) {
            t += p < NB ? __uint_as_float(sa[i].x) : 0.f;
            t += p + 1 < NB ? __uint_as_float(sa[i].z) : 0.f;
            t += p + 2 < NB ? __uint_as_float(sc[i].x) : 0.f;
            t += p + 3 < NB ? __uint_as_float(sc[i].z) : 0.f;
        }
    }
#pragma unroll
    for (int j = 0; j < NV; ++j)
        rv[j] = make_float4(__uint_as_float(ra[j].x), __uint_as_float(ra[j].z), __uint_as_float(rc[j].x),
                            __uint_as_float(rc[j].z));
    return with_ss ? t : 0.f;
}

template <int BITS, int GCPL, int RX, int LPR, int DCPL, int MAXS, bool TBL>
__global__ void __launch_bounds__(NT) k_stack(StackArgs args)
{
    using C = Codes<BITS>;
    constexpr int RPU = 64 / LPR;  // down rows per wave unit
    extern __shared__ __align__(16) unsigned char smem[];

    // The epochs of a workspace belong to one grid size.
    const uint32_t hdr = __hip_atomic_load(args.hdr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (hdr != 0u && hdr != gridDim.x) {
        if (threadIdx.x == 0 && blockIdx.x == 0) atomicOr(args.flags, MOE_DEVERR_WORKSPACE);
        return;
    }
    // Epochs: the exchanges of layer l carry base + 3l + 1 (logits), + 2 (h)
    // and + 3 (residual rows and sums of squares); every block starts from
    // the epoch the previous launch on this workspace ended with.
    const uint32_t base = __hip_atomic_load(args.slots + blockIdx.x * kSlotWords, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    {
        KArgs A = kargs();
        const Views v = views<BITS>(smem, A->D, A->E, A->I, A->n_slots);
        if (threadIdx.x < 8) reinterpret_cast<int *>(v.misc)[16 + threadIdx.x] = 0;
        __syncthreads();
    }

    // One layer ahead: this wave's slice of the layer's first round of
    // router rows (row b + NB*rs, slice sw) and, for waves 1.., its shared
    // gate/up row (unit (wave-1)*NB + b, if the expert has that many rows;
    // wave 0 takes the top-K instead).
    RtRegs<RN> ra;
    GuRegs<BITS, GCPL, 1> ga;
    auto prefetch = [&](KArgs A, int l) {
        const int tid = opaque_v(threadIdx.x), lane = tid & 63;
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int NB = gridDim.x, b = blockIdx.x;
        const int D = A->D, E = A->E, I = A->I;
        const int rs = wave / RSL, sw = wave % RSL;
        const StackLayer Ly = layer_of<TBL>(A, l);
        const int e = b + NB * rs;
        router_slice_load<RN>(ra, e < E && !Ly.slab ? Ly.router + (size_t)e * D : nullptr, D, sw, lane);
        const int su = (wave - 1) * NB + b;
        gu_load<BITS, GCPL, 1>(ga, wave > 0 && su < I ? shared_blob(A, Ly) : nullptr, D, I, su, lane);
    };
    prefetch(kargs(), 0);

    const int n_layers = kargs()->n_layers;
    for (int l = 0; l < n_layers; ++l) {
        KArgs A = kargs();
        const int tid = opaque_v(threadIdx.x), lane = tid & 63;
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int NB = gridDim.x, b = blockIdx.x;
        const int gw = wave * NB + b, GW = NWB * NB;
        const int D = A->D, E = A->E, K = A->K, I = A->I, S = A->n_slots;
        const StackLayer Ly = layer_of<TBL>(A, l);
        const Views v = views<BITS>(smem, D, E, I, S);
        int *sel = reinterpret_cast<int *>(v.misc);  // the block's selection [8]
        float *selw = v.misc + 8;                     // and its weights [8]
        int *rdy = reinterpret_cast<int *>(v.misc) + 16;  // selection k published: rdy[k] == l + 1
        const int cpk = I / C::CODES;                 // h chunks per slot
        const int nd = (D + RPU - 1) / RPU;           // down units
        const uint32_t t_log = base + 3u * l + 1u, t_h = t_log + 1u, t_res = t_log + 2u;
        MOE_PROBE(0);

        // ---- phase A: x_l, r_l and x_l's digit table
        {
            const float4 *gm = l > 0 ? reinterpret_cast<const float4 *>(A->layer[l - 1].gamma) : nullptr;
            const float4 *r_src = reinterpret_cast<const float4 *>(A->resid);
            const float4 *x_src = reinterpret_cast<const float4 *>(A->x);
            float inv = 1.f;
            for (int q0 = 0; q0 < D / 4; q0 += NT * XV) {
                float4 rv[XV], gv[XV];
#pragma unroll
                for (int j = 0; j < XV; ++j) {
                    const int q = q0 + tid + j * NT;
                    gv[j] = make_float4(0.f, 0.f, 0.f, 0.f);
                    rv[j] = gv[j];
                    if (q < D / 4) {
                        gv[j] = l == 0 ? x_src[q] : gm[q];
                        if (l == 0) rv[j] = r_src[q];
                    }
                }
                if (l > 0) {
                    // the residual rows and sums of squares of layer l-1
                    const float t = poll_residual<XV>(A, q0, D, NB, t_res - 3u, q0 == 0, rv);
                    if (q0 == 0) inv = 1.f / sqrtf(group_sum<64>(t) / (float)D + A->eps);
                    if (q0 == 0) MOE_PROBE(1);
                }
#pragma unroll
                for (int j = 0; j < XV; ++j) {
                    const int q = q0 + tid + j * NT;
                    const bool ok = q < D / 4;
                    const float4 r = rv[j], gq = gv[j];
                    const float4 xv = l == 0 ? gq
                                             : make_float4(r.x * inv * gq.x, r.y * inv * gq.y, r.z * inv * gq.z,
                                                           r.w * inv * gq.w);
                    if (ok) {
                        reinterpret_cast<float4 *>(v.xs)[q] = xv;
                        reinterpret_cast<float4 *>(v.rs)[q] = r;
                        if (A->record && b == 0) {
                            reinterpret_cast<float4 *>(A->record + (size_t)l * 2 * D)[q] = r;
                            reinterpret_cast<float4 *>(A->record + (size_t)l * 2 * D + D)[q] = xv;
                        }
                    }
                    chunk_digits_lane<BITS>(xv, q, ok, v.dig, v.csum, v.xcinv);
                }
            }
        }
        MOE_PROBE(2);
        lds_barrier();

        // router rows: RSL waves per row, RPB rows per block and round, the
        // slices added in a fixed order; the logits go out tagged.  A
        // streamed layer (slab) takes the routing its slab was filled for
        // and computes no logits.
        const int nr = b < E && !Ly.slab ? (E - b + NB * RPB - 1) / (NB * RPB) : 0;
        {
            const int rsr = wave / RSL, sw = wave % RSL;
            for (int j = 0; j < nr; ++j) {
                const int e = b + NB * (RPB * j + rsr);
                const float acc = router_slice<RN>(ra, j == 0, e < E ? Ly.router + (size_t)e * D : nullptr, v.xs, D, sw, lane);
                if (lane == 0) v.u[j * NWB + wave] = acc;
            }
        }
        MOE_PROBE(3);
        lds_barrier();
        for (int t = tid; t < nr * RPB; t += NT) {
            const int j = t / RPB, rr = t - j * RPB;
            const int e = b + NB * (RPB * j + rr);
            if (e < E) {
                float s = v.u[j * NWB + rr * RSL];
#pragma unroll
                for (int q = 1; q < RSL; ++q) s += v.u[j * NWB + rr * RSL + q];
                tag_store(A->tlog + e, s, t_log);
            }
        }
        MOE_PROBE(4);

        // ---- phase B: wave 0 polls the logits and takes the top-K, each
        // selected index published as soon as it is known; waves 1.. run the
        // shared expert's gate/up rows (loaded a layer ahead) meanwhile, then
        // every wave its unit of routed gate/up rows (RX rows) as soon as its
        // slot's expert is known
        if (wave == 0) {
            if (Ly.slab) {
                // streamed: the slab holds the experts of topk_idx (in that
                // order, e.g. as moe_route chose them); take that routing as it is
                if (lane < K) {
                    sel[lane] = A->topk_idx[l * K + lane];
                    selw[lane] = A->topk_w[l * K + lane];
                }
                __builtin_amdgcn_wave_barrier();
                if (lane < K) __hip_atomic_store(rdy + lane, l + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
            } else {
                // the top-K is on every layer's critical path: its wave goes
                // ahead of the shared gate/up wave on the same SIMD
                __builtin_amdgcn_s_setprio(3);
                wave_topk_global<KPL>(A->tlog, t_log, E, K, sel, selw, rdy, l + 1, lane, A->flags);
                __builtin_amdgcn_s_setprio(0);
                if (b == 0 && lane < K) {
                    A->topk_idx[l * K + lane] = sel[lane];
                    A->topk_w[l * K + lane] = selw[lane];
                }
            }
        } else if (const uint8_t *sh = shared_blob(A, Ly)) {
            for (int u = (wave - 1) * NB + b, j = 0; u < I; u += (NWB - 1) * NB, ++j) {
                if (j > 0) gu_load<BITS, GCPL, 1>(ga, sh, D, I, u, lane);
                float hv[1];
                gu_finish_c<BITS, GCPL, 1>(ga, v.dig, v.csum, v.xcinv, D, lane, hv);
                if (lane == 0) tag_store(A->th + (size_t)K * I + u, hv[0], t_h);
            }
        }
        MOE_PROBE(5);
        {
            const int upe = (I + RX - 1) / RX;
            for (int u = gw; u < K * upe; u += GW) {
                const int k = u / upe, i0 = (u - k * upe) * RX;
                if (TBL ? !Ly.slab : Ly.experts != nullptr) wait_selected(rdy, k, l + 1, A->flags);
                GuRegs<BITS, GCPL, RX> gb;
                gu_load<BITS, GCPL, RX>(gb, slot_blob<TBL>(A, Ly, sel, k), D, I, i0, lane);
                float hv[RX];
                gu_finish_c<BITS, GCPL, RX>(gb, v.dig, v.csum, v.xcinv, D, lane, hv);
                if (lane == 0) {
#pragma unroll
                    for (int r = 0; r < RX; ++r)
                        if (i0 + r < I) tag_store(A->th + (size_t)k * I + i0 + r, hv[r], t_h);
                }
            }
        }
        MOE_PROBE(6);
        // Down units: when at most half the waves have one (wide row units),
        // wave w and its helper w + NWB/2 share a unit: the partner takes
        // slots [0, ka), the helper slots [ka, S) and hands its per-lane slot
        // partials over through LDS, so the partner's slot-order combine is
        // the same arithmetic as one wave's.
        static_assert(NWB == 8 && kMaxSlots - (kMaxSlots + 1) / 2 <= 4, "helper partials are [4 waves][4 slots]");
        // (only units of four or more rows, LPR <= 16, have the split: with
        // one- and two-row units the plain path measured faster or the
        // registers did not allow it)
        constexpr bool kSplit = LPR <= 16;
        const bool split = kSplit && 2 * nd <= GW;
        const int half = NWB / 2;
        const bool helper = split && wave >= half;
        const int ud = split ? (wave % half) * NB + b : gw;  // this wave's (first) down unit
        const int ka = (S + 1) / 2;
        const int k_lo = helper ? ka : 0, k_hi = split && !helper ? ka : S;
        // the down rows of every slot (first round): they stream while the
        // other blocks finish their gate/up rows
        DnRegs<BITS, DCPL> dn[MAXS];
        if (TBL ? !Ly.slab : Ly.experts != nullptr) wait_selected(rdy, K - 1, l + 1, A->flags);
#pragma unroll
        for (int k = 0; k < MAXS; ++k)
            dn_load<BITS, LPR, DCPL>(dn[k], (k >= k_lo && k < k_hi && ud < nd) ? slot_blob<TBL>(A, Ly, sel, k) : nullptr, D,
                                     I, ud * RPU, lane);
        MOE_PROBE(7);

        // ---- phase C: h of every slot (polled until all of it carries this
        // layer's epoch) as digit tables; then the next layer's router and
        // shared rows are requested
        {
            const int n4 = S * I / 4;
            for (int q0 = 0; q0 < n4; q0 += NT * HV) {
                float4 hv[HV];
                bool nh[HV];
#pragma unroll
                for (int j = 0; j < HV; ++j) {
                    nh[j] = q0 + tid + j * NT < n4;
                    hv[j] = make_float4(0.f, 0.f, 0.f, 0.f);
                }
                for (uint32_t spins = 0;;) {
                    bool ok = true;
#pragma unroll
                    for (int j = 0; j < HV; ++j) {
                        const int q = q0 + tid + j * NT;
                        const uint4 a = tag_load2_if(A->th, 4 * q, nh[j]), c = tag_load2_if(A->th, 4 * q + 2, nh[j]);
                        const bool g = a.y == t_h && a.w == t_h && c.y == t_h && c.w == t_h;
                        if (nh[j]) {
                            hv[j] = make_float4(__uint_as_float(a.x), __uint_as_float(a.z), __uint_as_float(c.x),
                                                __uint_as_float(c.z));
                            ok &= g;
                            nh[j] = !g;
                        }
                    }
                    if (__all(ok)) break;
                    __builtin_amdgcn_s_sleep(1);
                    if (++spins == kTagSpins) {
                        atomicOr(A->flags, MOE_DEVERR_BARRIER_TIMEOUT);
                        break;
                    }
                }
                if (q0 + NT * HV >= n4 && l + 1 < n_layers) prefetch(A, l + 1);
#pragma unroll
                for (int j = 0; j < HV; ++j) {
                    const int q = q0 + tid + j * NT;
                    chunk_digits_lane<BITS>(hv[j], q, q < n4, v.hdig, v.hcsum, v.hcinv);
                }
            }
        }
        MOE_PROBE(8);
        lds_barrier();
        MOE_PROBE(9);
        // down rows of all slots, combined in slot order into LDS
        if (kSplit && split) {
            // the partner's chain over its own slots, the helper's partials
            // to LDS; then the partner continues the chain with them
            float c = 0.f;
#pragma unroll
            for (int k = 0; k < MAXS; ++k) {
                if (k < k_lo || k >= k_hi || ud >= nd) continue;
                const float y = dn_part_c<BITS, LPR, DCPL>(dn[k], v.hdig + k * cpk * C::DW, v.hcsum + k * cpk,
                                                           v.hcinv + k * cpk, I, lane);
                if (helper)
                    v.yh[((wave - half) * 4 + (k - ka)) * 64 + lane] = y;
                else
                    c = fmaf(k < K ? selw[k] : 1.f, y, c);
            }
            lds_barrier();
            if (!helper && ud < nd) {
                const int o = ud * RPU + lane / LPR;
#pragma unroll
                for (int k = 0; k < MAXS; ++k)
                    if (k >= ka && k < S) c = fmaf(k < K ? selw[k] : 1.f, v.yh[(wave * 4 + (k - ka)) * 64 + lane], c);
                c = group_sum<LPR>(c);
                if (lane % LPR == 0 && o < D) v.u[o] = c;
            }
        } else
        for (int u = gw, j = 0; u < nd; u += GW, ++j) {
            const int o0 = u * RPU, o = o0 + lane / LPR;
            if (j > 0) {
#pragma unroll
                for (int k = 0; k < MAXS; ++k)
                    dn_load<BITS, LPR, DCPL>(dn[k], k < S ? slot_blob<TBL>(A, Ly, sel, k) : nullptr, D, I, o0, lane);
            }
            // slot partials weighted per lane, in slot order, then one
            // reduction over the row's lanes
            float c = 0.f;
#pragma unroll
            for (int k = 0; k < MAXS; ++k) {
                if (k >= S) continue;
                const float y = dn_part_c<BITS, LPR, DCPL>(dn[k], v.hdig + k * cpk * C::DW, v.hcsum + k * cpk,
                                                           v.hcinv + k * cpk, I, lane);
                c = fmaf(k < K ? selw[k] : 1.f, y, c);
            }
            c = group_sum<LPR>(c);
            if (lane % LPR == 0 && o < D) v.u[o] = c;
        }
        MOE_PROBE(10);
        lds_barrier();
        // the block's rows (units b + NB*m): r' = r + c, published tagged with
        // the block's sum of squares
        if (wave == 0) {
            float ssacc = 0.f;
            for (int t = lane;; t += 64) {
                const int m = t / RPU, rr = t - m * RPU;
                const int u = b + NB * m;
                if (u >= nd) break;
                const int o = u * RPU + rr;
                if (o < D) {
                    const float rn = v.rs[o] + v.u[o];
                    tag_store(A->tres + o, rn, t_res);
                    ssacc = fmaf(rn, rn, ssacc);
                }
            }
            ssacc = group_sum<64>(ssacc);
            if (lane == 0) tag_store(A->tss + b, ssacc, t_res);
        }
        MOE_PROBE(11);
        // the block's LDS is rewritten by the next layer
        lds_barrier();
    }

    // ---- the stack's output: residual stream and its normalisation
    {
        KArgs A = kargs();
        const int tid = threadIdx.x, NB = gridDim.x, b = blockIdx.x, D = A->D, L = A->n_layers;
        const uint32_t t_res = base + 3u * L;
        float4 rv[1];
        const float t = poll_residual<1>(A, 0, 0, NB, t_res, true, rv);
        const float inv = 1.f / sqrtf(group_sum<64>(t) / (float)D + A->eps);
        const float4 *gm = reinterpret_cast<const float4 *>(A->layer[L - 1].gamma);
        for (int d4 = b * NT + tid; d4 < D / 4; d4 += NB * NT) {
            float4 r = make_float4(0.f, 0.f, 0.f, 0.f);
            for (uint32_t spins = 0;;) {
                const uint4 a = tag_load2(A->tres, 4 * d4), c = tag_load2(A->tres, 4 * d4 + 2);
                r = make_float4(__uint_as_float(a.x), __uint_as_float(a.z), __uint_as_float(c.x), __uint_as_float(c.z));
                if (a.y == t_res && a.w == t_res && c.y == t_res && c.w == t_res) break;
                __builtin_amdgcn_s_sleep(1);
                if (++spins == kTagSpins) {
                    atomicOr(A->flags, MOE_DEVERR_BARRIER_TIMEOUT);
                    break;
                }
            }
            const float4 gv = gm[d4];
            const float4 xv = make_float4(r.x * inv * gv.x, r.y * inv * gv.y, r.z * inv * gv.z, r.w * inv * gv.w);
            reinterpret_cast<float4 *>(A->resid)[d4] = r;
            reinterpret_cast<float4 *>(A->x)[d4] = xv;
            if (A->record) {
                reinterpret_cast<float4 *>(A->record + (size_t)L * 2 * D)[d4] = r;
                reinterpret_cast<float4 *>(A->record + (size_t)L * 2 * D + D)[d4] = xv;
            }
        }
        if (tid == 0) __hip_atomic_store(A->slots + b * kSlotWords, t_res, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (tid == 0 && b == 0) __hip_atomic_store(A->hdr, (uint32_t)NB, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Launch plan per instantiation and device: one block per CU when the
// kernel needs no scratch and one block with this LDS fits a CU.
struct StackPlanCache {
    int ready = 0, vgprs = 0, scratch = 0, n_cu = 0;
};

template <int GCPL, int RX, int LPR, int DCPL, int MAXS, bool TBL>
hipError_t stack_launch(const StackArgs *a, int D, int E, int I, int S, hipStream_t s, LayerPlan *p)
{
    auto kern = k_stack<MOE_STACK_BITS, GCPL, RX, LPR, DCPL, MAXS, TBL>;
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
    p->grid = (c.scratch == 0 && per_cu >= 1 && lo.total <= 160u * 1024u && E <= 64 * KPL)
                  ? (c.n_cu < kMaxLayerBlocks ? c.n_cu : kMaxLayerBlocks)
                  : 0;
    if (!a) return hipSuccess;
    if (p->grid == 0) return hipErrorNotSupported;
    hipLaunchKernelGGL(kern, dim3(p->grid), dim3(NT), lo.total, s, *a);
    return hipGetLastError();
}

// Shape -> instantiation.  Gate/up: GCPL chunks per lane and row, RX rows
// per wave unit.  Down: the smallest power-of-two LPR >= the row's chunks
// (8..64), DCPL chunks per lane.
template <int GCPL, bool TBL>
hipError_t stack_g(const StackArgs *a, int D, int E, int I, int S, hipStream_t s, LayerPlan *p)
{
    constexpr int RX = GCPL <= 2 ? 2 : 1;
    const int nch = I * MOE_STACK_BITS / 128;
    const bool wide = S > 5;
#define MOE_S(LPR_, DCPL_)                                                                                              \
    return wide ? stack_launch<GCPL, RX, LPR_, DCPL_, kMaxSlots, TBL>(a, D, E, I, S, s, p)                              \
                : stack_launch<GCPL, RX, LPR_, DCPL_, 5, TBL>(a, D, E, I, S, s, p);
    if (nch <= 8) MOE_S(8, 1)
    if (nch <= 16) MOE_S(16, 1)
    if (nch <= 32) MOE_S(32, 1)
    if (nch <= 64) MOE_S(64, 1)
    MOE_S(64, 2)
#undef MOE_S
}

}  // namespace

namespace {
template <bool TBL>
hipError_t stack_bits_t(const StackArgs *a, int D, int E, int I, int S, hipStream_t s, LayerPlan *p)
{
    const int nch = D * MOE_STACK_BITS / 128;
    if (nch <= 64) return stack_g<1, TBL>(a, D, E, I, S, s, p);
    if constexpr (MOE_STACK_BITS == 4) {
        if (nch <= 128) return stack_g<2, TBL>(a, D, E, I, S, s, p);
        return stack_g<4, TBL>(a, D, E, I, S, s, p);
    } else {
        return stack_g<2, TBL>(a, D, E, I, S, s, p);
    }
}
}  // namespace

#if MOE_STACK_BITS == 4
hipError_t stack_bits4(const StackArgs *a, int D, int E, int I, int S, bool tables, hipStream_t s, LayerPlan *p)
#else
hipError_t stack_bits2(const StackArgs *a, int D, int E, int I, int S, bool tables, hipStream_t s, LayerPlan *p)
#endif
{
    return tables ? stack_bits_t<true>(a, D, E, I, S, s, p) : stack_bits_t<false>(a, D, E, I, S, s, p);
}

}  // namespace moe
