// moe_kernels.hip -- the separately launched kernels of moe_route and
// moe_expert_forward (batch 1):
//   k_route      router GEMV (fp32) + top-K + softmax over the selection,
//                the top-K done by the last workgroup to finish;
//   k_gate_up    dequantised gate/up GEMV for every selected expert and the
//                shared expert, SwiGLU fused, h kept in the workspace;
//   k_down       dequantised down GEMV for all slots of one output row block,
//                weighted combine in slot order.
// moe_layer_step and moe_stack_step run the same building blocks fused in
// one persistent launch (moe_stack.hip).
#include "moe_device.h"

namespace moe {
namespace {

using namespace dev;

// Router: kRouterSlices waves per row (router_slice, the same reduction as
// the fused stack kernel's router, so that both give the same logits bit for
// bit), two rows per 512-thread block.  The last block to arrive selects the
// top K and writes the weights (topk_select for E <= 512, the stack kernel's
// selection; wave_topk beyond).
constexpr int kRouteThreads = 512;
constexpr int kRouteRows = kRouteThreads / 64 / kRouterSlices;

__global__ void __launch_bounds__(kRouteThreads) k_route(RouteArgs a)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int rr = wave / kRouterSlices, sw = wave % kRouterSlices;
    const int row = blockIdx.x * kRouteRows + rr;
    __shared__ float part[kRouteThreads / 64];
    __shared__ int is_last;
    {
        RtRegs<kRouterRN> r;
        const float acc = router_slice<kRouterRN>(r, false, row < a.E ? a.router + (size_t)row * a.D : nullptr, a.x,
                                                  a.D, sw, lane);
        if (lane == 0) part[wave] = acc;
    }
    __syncthreads();
    if (tid < kRouteRows && blockIdx.x * kRouteRows + tid < a.E) {
        float s = part[tid * kRouterSlices];
#pragma unroll
        for (int q = 1; q < kRouterSlices; ++q) s += part[tid * kRouterSlices + q];
        xstore(a.logits + blockIdx.x * kRouteRows + tid, s);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
        const uint32_t prev = __hip_atomic_fetch_add(a.counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        is_last = prev == gridDim.x - 1;
    }
    __syncthreads();
    if (!is_last || wave != 0) return;

    if (a.E <= 64 * 8) {
        __shared__ int sel[kMaxTopK], rdy[kMaxTopK];
        __shared__ float selw[kMaxTopK];
        uint32_t ord[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int e = lane + 64 * j;
            ord[j] = e < a.E ? order_key(__float_as_uint(xload(a.logits + e))) : 0u;
        }
        topk_select<8>(ord, a.K, sel, selw, rdy, 1, lane);
        __builtin_amdgcn_wave_barrier();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        if (lane < a.K) {
            a.topk_idx[lane] = sel[lane];
            a.topk_w[lane] = selw[lane];
        }
    } else {
        __shared__ float lg[4096];
        for (int e = lane; e < a.E; e += 64) lg[e] = xload(a.logits + e);
        __builtin_amdgcn_wave_barrier();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        int idx[kMaxTopK];
        float vals[kMaxTopK], w[kMaxTopK];
        wave_topk(lg, a.E, a.K, lane, idx, vals);
        if (lane == 0) {
            topk_weights(vals, a.K, w);
#pragma unroll
            for (int k = 0; k < kMaxTopK; ++k) {
                if (k >= a.K) continue;
                a.topk_idx[k] = idx[k];
                a.topk_w[k] = w[k];
            }
        }
    }
    if (lane == 0) *a.counter = 0u;
}

constexpr int kGateUpRows = 2;  // rows per wave unit

// Gate/up: blocks_per_slot blocks per slot, each staging x and its digit
// table in LDS once and then walking its share of the slot's rows in wave
// units of kGateUpRows rows.
template <int BITS, int CPL>
__global__ void __launch_bounds__(256) k_gate_up(GateUpArgs a)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int slot = blockIdx.x / a.blocks_per_slot;
    const int rb = blockIdx.x - slot * a.blocks_per_slot;
    __shared__ __align__(16) float xs[8192];
    __shared__ __align__(16) int dig[8192 / 32 * 24];
    __shared__ float csum[8192 / 32];
    __shared__ float red[16];
    for (int d = threadIdx.x; d < a.D; d += blockDim.x) xs[d] = a.x[d];
    __syncthreads();
    const float inv = block_digit_table<BITS>(xs, a.D, dig, csum, red);

    const int32_t e = slot < a.src.top_k && !a.src.slab ? a.topk_idx[slot] : -1;
    const uint8_t *blob = blob_of(a.src, slot, e, a.flags);
    float *h = a.h + (size_t)slot * a.I;
    const int units = (a.I + kGateUpRows - 1) / kGateUpRows;
    for (int u = rb * 4 + wave; u < units; u += a.blocks_per_slot * 4) {
        const int i0 = u * kGateUpRows;
        if (!blob) {
            if (lane < kGateUpRows && i0 + lane < a.I) h[i0 + lane] = 0.f;
            continue;
        }
        wave_gate_up<BITS, CPL, kGateUpRows>(blob, dig, csum, inv, a.D, a.I, i0, lane, h);
    }
}

// Down + combine: one block per RW output rows, one wave per slot.  Partial
// rows meet in LDS and are summed in slot order (routed 0..K-1, then shared).
// Layer mode adds the residual, keeps a per-block sum of squares, and the
// last block to arrive applies RMSNorm to every row.
template <int BITS, int LPR, int CPL, int STEPS>
__global__ void __launch_bounds__(64 * kMaxSlots) k_down(DownArgs a)
{
    constexpr int RPS = 64 / LPR;
    constexpr int RW = RPS * STEPS;
    static_assert(RW <= 64, "one wave finishes the rows");
    const int tid = threadIdx.x, lane = tid & 63, k = tid >> 6;
    const int o0 = blockIdx.x * RW;
    __shared__ float part[kMaxSlots][RW];
    __shared__ int is_last;
    __shared__ float inv_s;

    const int32_t e = k < a.src.top_k && !a.src.slab ? a.topk_idx[k] : -1;
    const uint8_t *blob = blob_of(a.src, k, e, a.flags);
    const float wk = k < a.src.top_k ? a.topk_w[k] : 1.f;
    float out[STEPS];
    wave_down<BITS, LPR, CPL, STEPS, false>(blob, a.h + (size_t)k * a.I, a.D, a.I, o0, lane, out);
    if (lane % LPR == 0) {
#pragma unroll
        for (int s = 0; s < STEPS; ++s) part[k][s * RPS + lane / LPR] = blob ? wk * out[s] : 0.f;
    }
    __syncthreads();
    if (k == 0) {
        const int o = o0 + lane;
        float v = 0.f;
        if (lane < RW && o < a.D) {
            float c = 0.f;
            for (int j = 0; j < a.src.n_slots; ++j) c += part[j][lane];
            if (a.mode == 0) {
                a.y[o] = c;
            } else {
                const float r = a.resid[o] + c;
                xstore(a.resid + o, r);
                v = r * r;
            }
        }
        if (a.mode == 1) {
            v = group_sum<64>(v);
            if (lane == 0) xstore(a.ss + blockIdx.x, v);
        }
    }
    if (a.mode == 0) return;

    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
        const uint32_t prev = __hip_atomic_fetch_add(a.counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        is_last = prev == gridDim.x - 1;
    }
    __syncthreads();
    if (!is_last) return;
    if (k == 0) {
        float t = 0.f;
        for (int b = lane; b < (int)gridDim.x; b += 64) t += xload(a.ss + b);
        t = group_sum<64>(t);
        if (lane == 0) {
            inv_s = 1.f / sqrtf(t / (float)a.D + a.eps);
            *a.counter = 0u;
        }
    }
    __syncthreads();
    // RMSNorm of every row: all loads of a thread first, then the stores
    const float inv = inv_s;
    constexpr int kPer = 8;
    for (int o0b = 0; o0b < a.D; o0b += (int)blockDim.x * kPer) {
        float rv[kPer], gv[kPer];
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int o = o0b + j * (int)blockDim.x + tid;
            rv[j] = o < a.D ? xload(a.resid + o) : 0.f;
            gv[j] = o < a.D ? a.gamma[o] : 0.f;
        }
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int o = o0b + j * (int)blockDim.x + tid;
            if (o < a.D) a.x[o] = rv[j] * inv * gv[j];
        }
    }
}

template <int BITS, int CPL>
hipError_t gate_up_cpl(const GateUpArgs &a, hipStream_t s)
{
    dim3 grid(a.blocks_per_slot * a.src.n_slots);
    hipLaunchKernelGGL((k_gate_up<BITS, CPL>), grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

template <int BITS>
hipError_t gate_up_bits(const GateUpArgs &a, hipStream_t s)
{
    const int cpl = (a.D * BITS / 128 + 63) / 64;  // hidden <= 8192: 4-bit <= 4, 2-bit <= 2
    if (cpl <= 1) return gate_up_cpl<BITS, 1>(a, s);
    if constexpr (BITS == 2) return gate_up_cpl<BITS, 2>(a, s);
    else {
        if (cpl <= 2) return gate_up_cpl<BITS, 2>(a, s);
        return gate_up_cpl<BITS, 4>(a, s);
    }
}

template <int BITS, int LPR, int CPL, int STEPS>
hipError_t down_launch(const DownArgs &a, hipStream_t s)
{
    constexpr int RW = (64 / LPR) * STEPS;
    dim3 grid((a.D + RW - 1) / RW);
    hipLaunchKernelGGL((k_down<BITS, LPR, CPL, STEPS>), grid, dim3(64 * a.src.n_slots), 0, s, a);
    return hipGetLastError();
}

template <int BITS, int LPR>
hipError_t down_lpr(const DownArgs &a, int cpl, hipStream_t s)
{
    constexpr int STEPS = (16 * LPR / 64) < 1 ? 1 : ((16 * LPR / 64) > 8 ? 8 : (16 * LPR / 64));
    if (cpl <= 1) return down_launch<BITS, LPR, 1, STEPS>(a, s);
    return down_launch<BITS, LPR, 2, STEPS>(a, s);
}

template <int BITS>
hipError_t down_bits(const DownArgs &a, hipStream_t s)
{
    const DownShape d = down_shape(a.I, BITS);
    switch (d.lpr) {
    case 1: return down_lpr<BITS, 1>(a, d.cpl, s);
    case 2: return down_lpr<BITS, 2>(a, d.cpl, s);
    case 4: return down_lpr<BITS, 4>(a, d.cpl, s);
    case 8: return down_lpr<BITS, 8>(a, d.cpl, s);
    case 16: return down_lpr<BITS, 16>(a, d.cpl, s);
    case 32: return down_lpr<BITS, 32>(a, d.cpl, s);
    default: return down_lpr<BITS, 64>(a, d.cpl, s);
    }
}

}  // namespace

DownShape down_shape(int I, int bits)
{
    const int nchunks = I * bits / 128;
    int lpr = 1;
    while (lpr * 2 <= nchunks && lpr < 64) lpr *= 2;
    DownShape d;
    d.lpr = lpr;
    d.cpl = (nchunks + lpr - 1) / lpr;
    return d;
}

// About 512 blocks in all, each with at least one wave unit per wave.
int gate_up_blocks_per_slot(int I, int n_slots)
{
    const int most = (I + 4 * kGateUpRows - 1) / (4 * kGateUpRows);
    int b = 512 / (n_slots > 0 ? n_slots : 1);
    if (b < 1) b = 1;
    return b < most ? b : most;
}

int down_blocks(int D, int I, int bits)
{
    const DownShape d = down_shape(I, bits);
    int steps = 16 * d.lpr / 64;
    steps = steps < 1 ? 1 : (steps > 8 ? 8 : steps);
    const int rw = (64 / d.lpr) * steps;
    return (D + rw - 1) / rw;
}

hipError_t launch_route(const RouteArgs &a, hipStream_t s)
{
    hipLaunchKernelGGL(k_route, dim3((a.E + kRouteRows - 1) / kRouteRows), dim3(kRouteThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_gate_up(const GateUpArgs &a, int bits, hipStream_t s)
{
    return bits == 4 ? gate_up_bits<4>(a, s) : gate_up_bits<2>(a, s);
}

hipError_t launch_down(const DownArgs &a, int bits, hipStream_t s)
{
    return bits == 4 ? down_bits<4>(a, s) : down_bits<2>(a, s);
}

}  // namespace moe
