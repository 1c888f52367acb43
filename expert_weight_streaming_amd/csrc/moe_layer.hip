// moe_layer.hip -- one MoE layer step (batch 1) in one persistent launch.
//
// The pages' per-layer work (routing projection with the shared expert, the
// softmax/top-K, the expert forward, then combine + residual + norm fused,
// hakusoku.com "パイプライン概要" and "主要技術"; toolarium.ru
// "Оптимизации, которые сработали") has three all-to-all dependencies: top-K
// needs every logit, a down row needs every h, RMSNorm needs every output
// row.  Each becomes a grid barrier inside one launch instead of a kernel
// boundary:
//
//   phase A  router rows (one per wave) and the shared expert's gate/up rows
//            -- neither depends on the routing        -> barrier 1
//   phase B  every block selects the top K from the logits itself (no
//            broadcast round trip), then the routed gate/up rows   -> barrier 2
//   phase C  down rows of all slots for a block's row units, combined in
//            slot order in LDS, residual added, partial sum of squares
//                                                               -> barrier 3
//   phase D  every block sums the partials (fixed order) and normalises its
//            own rows.
//
// Blocks have one wave per slot (K routed + shared).  The grid never exceeds
// the number of blocks that fit on the device at once, so every block is
// resident and the barriers can be waited on.  Waits are bounded: a timeout
// raises MOE_DEVERR_BARRIER_TIMEOUT in the workspace flags and lets every
// wave run to its end.
#include "moe_device.h"

namespace moe {
namespace {

using namespace dev;

constexpr uint32_t kSpinLimit = 1u << 22;
constexpr int kMaxUnits = 8;  // phase-C row units per block

// Grid barrier of one launch.  Every block owns a 64-byte slot holding an
// epoch count; at barrier i a block publishes base + i in its slot and
// waits until every slot of the grid has reached it.  The epochs carry over
// from launch to launch (each launch adds 3), so no counter is ever reset
// and no atomic read-modify-write is contended.  Before publishing, the
// block waits for its own stores to complete; all data crossing a barrier
// is stored and loaded agent-coherently (xstore / xload / xload4).
struct GridBar {
    uint32_t *slots;
    uint32_t base;
    uint32_t nb;
    uint32_t *flags;
};

__device__ __forceinline__ void grid_sync(const GridBar &g, uint32_t i)
{
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    const uint32_t target = g.base + i;
    if (threadIdx.x == 0)
        __hip_atomic_store(g.slots + blockIdx.x * kSlotWords, target, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (threadIdx.x < 64) {
        uint32_t spins = 0;
        for (;;) {
            bool ok = true;
            for (uint32_t j = threadIdx.x; j < g.nb; j += 64)
                ok &= (int32_t)(__hip_atomic_load(g.slots + j * kSlotWords, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) -
                                target) >= 0;
            if (__all(ok)) break;
            __builtin_amdgcn_s_sleep(1);
            if (++spins == kSpinLimit) {
                atomicOr(g.flags, MOE_DEVERR_BARRIER_TIMEOUT);
                break;
            }
        }
    }
    __syncthreads();
}

template <int BITS, int GCPL, int R, int LPR, int DCPL, int STEPS, int MAXW>
__global__ void __launch_bounds__(64 * MAXW) k_layer(LayerArgs a)
{
    constexpr int RPS = 64 / LPR;
    constexpr int RW = RPS * STEPS;
    static_assert(RW <= 64, "one wave finishes the rows");
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int W = blockDim.x >> 6;
    const int NB = gridDim.x;
    const int D = a.D, I = a.I, E = a.E, K = a.K;
    const BlobSrc &src = a.src;

    using C = Codes<BITS>;
    __shared__ __align__(16) float xs[8192];
    __shared__ __align__(16) float lg[4096];
    __shared__ __align__(16) int dig[8192 / C::CODES * C::DW];
    __shared__ float csum[8192 / C::CODES];
    __shared__ float red[16];
    __shared__ float part[kMaxSlots][RW];
    __shared__ float rsave[kMaxUnits][RW];
    __shared__ int sel[kMaxTopK];
    __shared__ float selw[kMaxTopK];
    __shared__ float inv_s;

    // The barrier slots of a workspace belong to one grid size; a launch
    // with another grid on the same workspace stops here.
    const uint32_t hdr = __hip_atomic_load(a.hdr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (hdr != 0u && hdr != (uint32_t)NB) {
        if (tid == 0 && blockIdx.x == 0) atomicOr(a.flags, MOE_DEVERR_WORKSPACE);
        return;
    }
    GridBar g;
    g.slots = a.slots;
    g.base = __hip_atomic_load(a.slots + blockIdx.x * kSlotWords, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    g.nb = NB;
    g.flags = a.flags;

    for (int d = tid; d < D; d += blockDim.x) xs[d] = a.x[d];
    __syncthreads();
    const float xinv = block_digit_table<BITS>(xs, D, dig, csum, red);

    // ---- phase A: router rows + shared gate/up (routing-independent)
    const int gw = wave * NB + blockIdx.x, NW = W * NB;
    const int upe = (I + R - 1) / R;
    const bool has_shared = src.n_slots > K;
    const int nA = E + (has_shared ? upe : 0);
    for (int u = gw; u < nA; u += NW) {
        if (u < E) {
            const float v = wave_router_row(a.router + (size_t)u * D, xs, D, lane);
            if (lane == 0) xstore(a.logits + u, v);
        } else {
            wave_gate_up<BITS, GCPL, R>(blob_of(src, K, -1, a.flags), dig, csum, xinv, D, I, (u - E) * R, lane,
                                        a.h + (size_t)K * I);
        }
    }
    grid_sync(g, 1);

    // ---- phase B: top-K in every block, then routed gate/up
    for (int e = tid; e < E; e += blockDim.x) lg[e] = xload(a.logits + e);
    __syncthreads();
    if (wave == 0) {
        int idx[kMaxTopK];
        float vals[kMaxTopK], w[kMaxTopK];
        wave_topk(lg, E, K, lane, idx, vals);
        topk_weights(vals, K, w);
        if (lane == 0) {
#pragma unroll
            for (int k = 0; k < kMaxTopK; ++k) {
                if (k >= K) continue;
                sel[k] = idx[k];
                selw[k] = w[k];
                if (blockIdx.x == 0) {
                    a.topk_idx[k] = idx[k];
                    a.topk_w[k] = w[k];
                }
            }
        }
    }
    __syncthreads();
    for (int u = gw; u < K * upe; u += NW) {
        const int k = u / upe, i0 = (u - k * upe) * R;
        const uint8_t *blob = blob_of(src, k, sel[k], a.flags);
        float *h = a.h + (size_t)k * I;
        if (!blob) {
            if (lane < R && i0 + lane < I) xstore(h + i0 + lane, 0.f);
            continue;
        }
        wave_gate_up<BITS, GCPL, R>(blob, dig, csum, xinv, D, I, i0, lane, h);
    }
    grid_sync(g, 2);

    // ---- phase C: down rows of every slot, combine, residual
    const int units = (D + RW - 1) / RW;
    const uint8_t *myblob = blob_of(src, wave, wave < K ? sel[wave] : -1, a.flags);
    const float wk = wave < K ? selw[wave] : 1.f;
    float ssacc = 0.f;
    int j = 0;
    for (int u = blockIdx.x; u < units; u += NB, ++j) {
        const int o0 = u * RW;
        float out[STEPS];
        wave_down<BITS, LPR, DCPL, STEPS, true>(myblob, a.h + (size_t)wave * I, D, I, o0, lane, out);
        if (lane % LPR == 0) {
#pragma unroll
            for (int s = 0; s < STEPS; ++s) part[wave][s * RPS + lane / LPR] = myblob ? wk * out[s] : 0.f;
        }
        __syncthreads();
        if (wave == 0) {
            const int o = o0 + lane;
            float v = 0.f;
            if (lane < RW && o < D) {
                float c = 0.f;
                for (int q = 0; q < W; ++q) c += part[q][lane];
                const float r = a.resid[o] + c;
                a.resid[o] = r;
                rsave[j][lane] = r;
                v = r * r;
            }
            ssacc += group_sum<64>(v);
        }
        __syncthreads();
    }
    if (tid == 0) xstore(a.ss + blockIdx.x, ssacc);
    grid_sync(g, 3);

    // ---- phase D: RMSNorm of the block's own rows
    if (wave == 0) {
        float t = 0.f;
        for (int b = lane; b < NB; b += 64) t += xload(a.ss + b);
        t = group_sum<64>(t);
        if (lane == 0) inv_s = 1.f / sqrtf(t / (float)D + a.eps);
    }
    __syncthreads();
    const float inv = inv_s;
    j = 0;
    for (int u = blockIdx.x; u < units; u += NB, ++j) {
        const int o = u * RW + lane;
        if (wave == 0 && lane < RW && o < D) a.x[o] = rsave[j][lane] * inv * a.gamma[o];
    }
    if (tid == 0 && blockIdx.x == 0)
        __hip_atomic_store(a.hdr, (uint32_t)NB, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

constexpr int kGateUpRowsFused = 2;

// Grid of the fused kernel on the current device: as many blocks as fit on
// the device at once (at most 2 per CU) by the runtime's occupancy figure
// and by the kernel's own register count, or 0 when the instantiation needs
// scratch memory (scratch limits how many waves are resident).  `cache` is
// private to one instantiation.
inline hipError_t fused_plan(const void *kern, int n_slots, LayerPlan (*cache)[kMaxSlots + 1], LayerPlan *p)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 64 && cache[dev][n_slots].block) {
        *p = cache[dev][n_slots];
        return hipSuccess;
    }
    LayerPlan q;
    q.block = 64 * n_slots;
    hipFuncAttributes attr;
    if ((e = hipFuncGetAttributes(&attr, kern)) != hipSuccess) return e;
    q.vgprs = attr.numRegs;
    q.scratch = (int)attr.localSizeBytes;
    if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&q.per_cu, kern, q.block, 0)) != hipSuccess) return e;
    if ((e = hipDeviceGetAttribute(&q.n_cu, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
    // Waves per SIMD that the registers allow (512 VGPRs per lane, granules of
    // 8, at most 8 waves).  A block's waves are placed on the CU's 4 SIMDs
    // starting from the same SIMD, so the busiest SIMD holds ceil(W/4) waves
    // of each block: two 5-wave blocks need 4 wave slots on one SIMD.  The
    // runtime's occupancy figure has been seen to overstate this.
    const int regs = q.vgprs < 8 ? 8 : (q.vgprs + 7) / 8 * 8;
    int wps = 512 / regs;
    if (wps > 8) wps = 8;
    const int per_simd = (n_slots + 3) / 4;
    int fit = wps / per_simd;
    if (fit > q.per_cu) fit = q.per_cu;
    if (fit > 2) fit = 2;
    if (q.scratch == 0 && fit >= 1 && q.n_cu >= 1) {
        q.grid = fit * q.n_cu;
        if (q.grid > kMaxLayerBlocks) q.grid = kMaxLayerBlocks;
    }
    if (dev < 64) cache[dev][n_slots] = q;
    *p = q;
    return hipSuccess;
}

template <int BITS, int GCPL, int LPR, int DCPL, int MAXW>
hipError_t layer_launch_w(const LayerArgs *a_in, int n_slots, hipStream_t s, LayerPlan *p)
{
    constexpr int STEPS = (8 * LPR / 64) < 1 ? 1 : (8 * LPR / 64);
    constexpr int RW = (64 / LPR) * STEPS;
    auto kern = k_layer<BITS, GCPL, kGateUpRowsFused, LPR, DCPL, STEPS, MAXW>;
    static LayerPlan cache[64][kMaxSlots + 1];
    hipError_t e = fused_plan(reinterpret_cast<const void *>(kern), n_slots, cache, p);
    if (e != hipSuccess || !a_in) return e;
    if (p->grid == 0) return hipErrorNotSupported;
    const int units = (a_in->D + RW - 1) / RW;
    if ((units + p->grid - 1) / p->grid > kMaxUnits) return hipErrorNotSupported;
    hipLaunchKernelGGL(kern, dim3(p->grid), dim3(p->block), 0, s, *a_in);
    return hipGetLastError();
}

// Blocks of up to 5 waves (K <= 4 plus a shared expert) get their own launch
// bound, so the compiler may give each wave up to 256 VGPRs.
template <int BITS, int GCPL, int LPR, int DCPL>
hipError_t layer_launch(const LayerArgs *a_in, hipStream_t s, LayerPlan *p)
{
    const int n_slots = a_in ? a_in->src.n_slots : p->block / 64;
    if (n_slots <= 5) return layer_launch_w<BITS, GCPL, LPR, DCPL, 5>(a_in, n_slots, s, p);
    return layer_launch_w<BITS, GCPL, LPR, DCPL, kMaxSlots>(a_in, n_slots, s, p);
}

// Select the instantiation for (D, I, bits) and either launch (a != NULL) or
// only fill the plan.
template <int BITS, int GCPL>
hipError_t layer_gcpl(int I, const LayerArgs *a, hipStream_t s, LayerPlan *p)
{
    const DownShape d = down_shape(I, BITS);
#define MOE_L(LPR_)                                                                                                     \
    case LPR_:                                                                                                          \
        return d.cpl <= 1 ? layer_launch<BITS, GCPL, LPR_, 1>(a, s, p) : layer_launch<BITS, GCPL, LPR_, 2>(a, s, p);
    switch (d.lpr) {
        MOE_L(1)
        MOE_L(2)
        MOE_L(4)
        MOE_L(8)
        MOE_L(16)
        MOE_L(32)
        MOE_L(64)
    }
#undef MOE_L
    return hipErrorInvalidValue;
}

template <int BITS>
hipError_t layer_bits(int D, int I, const LayerArgs *a, hipStream_t s, LayerPlan *p)
{
    const int cpl = (D * BITS / 128 + 63) / 64;
    if (cpl <= 1) return layer_gcpl<BITS, 1>(I, a, s, p);
    if constexpr (BITS == 2) return layer_gcpl<BITS, 2>(I, a, s, p);
    else {
        if (cpl <= 2) return layer_gcpl<BITS, 2>(I, a, s, p);
        return layer_gcpl<BITS, 4>(I, a, s, p);
    }
}

}  // namespace

hipError_t launch_layer(const LayerArgs &a, int bits, hipStream_t s, int *grid)
{
    LayerPlan p;
    hipError_t e = bits == 4 ? layer_bits<4>(a.D, a.I, &a, s, &p) : layer_bits<2>(a.D, a.I, &a, s, &p);
    *grid = p.grid;
    return e;
}

hipError_t plan_layer(int D, int I, int bits, int n_slots, LayerPlan *p)
{
    p->block = 64 * n_slots;
    return bits == 4 ? layer_bits<4>(D, I, nullptr, nullptr, p) : layer_bits<2>(D, I, nullptr, nullptr, p);
}

}  // namespace moe
