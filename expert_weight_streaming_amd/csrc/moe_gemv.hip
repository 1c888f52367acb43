// moe_gemv.hip -- the dequantised expert GEMVs of a range of resident
// experts against one activation vector, with no routing and no combine:
// the matrix-vector kernel that the pages measure on its own against the
// memory bandwidth (hakusoku.com, 「Apple Siliconにおけるメモリ制約」), in the
// FMA-rewritten dequant form (toolarium.ru, «Оптимизации, которые
// сработали»; here as exact integer digit-plane dot products per 64-column
// group, the same inner loops as the fused stack kernel: gu_finish_c,
// dn_part_c).
//
// One launch.  A workgroup runs whole experts: the gate/up rows (SwiGLU
// applied, h kept in LDS), then h's digit table, then the down rows; so h
// never leaves the chip and every byte of the range's blobs is read once.
// Inside an expert, wave w takes row units w, w + 8, ..., so that the eight
// waves read neighbouring rows at any time.  A wave holds one unit (one
// gate/up row pair, or 8 to 16 down rows) at a time, so that the kernel fits
// 128 registers and four waves run per SIMD: while one computes, the loads
// of the others are in flight (measured faster than two units in flight per
// wave at two waves per SIMD).
#include "moe_device.h"

namespace moe {
namespace {

using namespace dev;

constexpr int NT = 512;
constexpr int NW = NT / 64;

// LDS: x's digit table (dig, csum, cinv), h (fp32 [I]) and h's digit table
// (hdig, hcsum, hcinv); byte offsets, 16-byte aligned.
struct GemvLds {
    uint32_t dig, csum, cinv, hs, hdig, hcsum, hcinv, total;
};
__host__ __device__ inline GemvLds gemv_lds(int D, int I, int bits)
{
    const uint32_t codes = 128 / bits, dw = 4 * (8 / bits) * 3;
    const uint32_t xc = (uint32_t)D / codes, hc = (uint32_t)I / codes;
    GemvLds l;
    uint32_t o = 0;
    auto take = [&](uint32_t &f, uint32_t bytes) {
        f = o;
        o = (o + bytes + 15u) & ~15u;
    };
    take(l.dig, xc * dw * 4);
    take(l.csum, xc * 4);
    take(l.cinv, xc * 4);
    take(l.hs, (uint32_t)I * 4);
    take(l.hdig, hc * dw * 4);
    take(l.hcsum, hc * 4);
    take(l.hcinv, hc * 4);
    l.total = o;
    return l;
}

// A vector of n fp32 values (n a multiple of the chunk width; global or
// LDS) as a digit table with one fixed-point step per chunk.  Called by the
// whole workgroup.
template <int BITS>
__device__ __forceinline__ void digit_table(const float *v, int n, int *dig, float *csum, float *cinv)
{
    const int n4 = n / 4;
    for (int q0 = 0; q0 < n4; q0 += NT) {
        const int q = q0 + (int)threadIdx.x;
        const float4 f = q < n4 ? reinterpret_cast<const float4 *>(v)[q] : make_float4(0.f, 0.f, 0.f, 0.f);
        chunk_digits_lane<BITS>(f, q, q < n4, dig, csum, cinv);
    }
}

// S down row groups of one wave unit (RPU = 64/LPR rows each, rows o0 +
// s*RPU + lane/LPR), loaded together.
template <int BITS, int DCPL, int S>
struct DnUnit {
    DnRegs<BITS, DCPL> d[S];
};

template <int BITS, int LPR, int DCPL, int S>
__device__ __forceinline__ void dn_unit_load(DnUnit<BITS, DCPL, S> &u, const uint8_t *blob, int D, int I, int o0,
                                             int lane)
{
    constexpr int RPU = 64 / LPR;
#pragma unroll
    for (int s = 0; s < S; ++s) dn_load<BITS, LPR, DCPL>(u.d[s], blob, D, I, o0 + s * RPU, lane);
}

// The unit's rows against h's digit table (LDS), each chunk's digits read
// once for all S groups; row sums in rows o0 + s*RPU + lane/LPR.
template <int BITS, int LPR, int DCPL, int S>
__device__ __forceinline__ void dn_unit_finish(const DnUnit<BITS, DCPL, S> &u, const int *hdig, const float *hcsum,
                                               const float *hcinv, int I, int D, int o0, int lane, float *yn)
{
    using C = Codes<BITS>;
    constexpr int RPU = 64 / LPR;
    const int nchunks = I * BITS / 128;
    const int lc = lane % LPR;
    float t[S];
#pragma unroll
    for (int s = 0; s < S; ++s) t[s] = 0.f;
#pragma unroll
    for (int m = 0; m < DCPL; ++m) {
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
            const float cs = hcsum[c], ci = hcinv[c];
#pragma unroll
            for (int s = 0; s < S; ++s) {
                const float qh = qdot<BITS>(u.d[s].q[m], dg);
                t[s] = fmaf(bf16_lo(u.d[s].sb[m]) * ci, qh, t[s]);
                t[s] = fmaf(bf16_hi(u.d[s].sb[m]), cs, t[s]);
            }
        }
    }
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const float r = group_sum<LPR>(t[s]);
        const int o = o0 + s * RPU + lane / LPR;
        if (lane % LPR == 0 && o < D) yn[o] = r;
    }
}

// Waves per SIMD the compiler must leave room for: four (at most 128
// registers), or one for gate/up rows of more than 2 KB, whose registers do
// not fit that.
template <int BITS, int GCPL>
constexpr int gemv_waves() { return GCPL >= 4 || (BITS == 2 && GCPL >= 2) ? 1 : 4; }

template <int BITS, int GCPL, int R, int LPR, int DCPL>
__global__ void __launch_bounds__(NT, (gemv_waves<BITS, GCPL>())) k_expert_gemv(GemvArgs a)
{
    constexpr int RPU = 64 / LPR;  // down rows per row group
    // row groups per down unit: up to 16 rows, at most 4 chunks per lane
    constexpr int S0 = 16 / RPU > 0 ? 16 / RPU : 1;
    constexpr int S = S0 * DCPL > 4 ? 4 / DCPL : S0;
    constexpr int RPD = RPU * S;   // rows per down unit
    extern __shared__ __align__(16) unsigned char smem[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int D = a.D, I = a.I;
    const GemvLds lo = gemv_lds(D, I, BITS);
    int *dig = reinterpret_cast<int *>(smem + lo.dig);
    float *csum = reinterpret_cast<float *>(smem + lo.csum);
    float *cinv = reinterpret_cast<float *>(smem + lo.cinv);
    float *hs = reinterpret_cast<float *>(smem + lo.hs);
    int *hdig = reinterpret_cast<int *>(smem + lo.hdig);
    float *hcsum = reinterpret_cast<float *>(smem + lo.hcsum);
    float *hcinv = reinterpret_cast<float *>(smem + lo.hcinv);

    digit_table<BITS>(a.x, D, dig, csum, cinv);
    lds_barrier();

    const int ngu = (I + R - 1) / R;          // gate/up units of an expert
    const int ndn = (D + RPD - 1) / RPD;      // down units
    for (int n = blockIdx.x; n < a.count; n += gridDim.x) {
        const uint8_t *blob = a.experts + (uint64_t)(a.first + n) * a.blob_bytes;
        float *hn = a.h + (size_t)n * I;
        float *yn = a.y + (size_t)n * D;
        // gate/up rows
        for (int u = wave; u < ngu; u += NW) {
            GuRegs<BITS, GCPL, R> g;
            gu_load<BITS, GCPL, R>(g, blob, D, I, u * R, lane);
            float hv[R];
            gu_finish_c<BITS, GCPL, R>(g, dig, csum, cinv, D, lane, hv);
            if (lane == 0) {
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const int i = u * R + r;
                    if (i < I) {
                        hs[i] = hv[r];
                        hn[i] = hv[r];
                    }
                }
            }
        }
        // the first down unit is requested before h is complete
        DnUnit<BITS, DCPL, S> d;
        if (wave < ndn) dn_unit_load<BITS, LPR, DCPL, S>(d, blob, D, I, wave * RPD, lane);
        lds_barrier();
        digit_table<BITS>(hs, I, hdig, hcsum, hcinv);
        lds_barrier();
        for (int u = wave; u < ndn; u += NW) {
            if (u > wave) dn_unit_load<BITS, LPR, DCPL, S>(d, blob, D, I, u * RPD, lane);
            dn_unit_finish<BITS, LPR, DCPL, S>(d, hdig, hcsum, hcinv, I, D, u * RPD, lane, yn);
        }
    }
}

struct GemvPlanCache {
    int ready = 0, n_cu = 0, per_cu = 0, vgprs = 0, scratch = 0;
};

template <int BITS, int GCPL, int R, int LPR, int DCPL>
hipError_t gemv_launch(const GemvArgs &a, hipStream_t s, LayerPlan *p)
{
    auto kern = k_expert_gemv<BITS, GCPL, R, LPR, DCPL>;
    static GemvPlanCache cache[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const GemvLds lo = gemv_lds(a.D, a.I, BITS);
    GemvPlanCache c = dev < 64 ? cache[dev] : GemvPlanCache{};
    if (!c.ready) {
        hipFuncAttributes attr;
        if ((e = hipFuncGetAttributes(&attr, reinterpret_cast<const void *>(kern))) != hipSuccess) return e;
        c.vgprs = attr.numRegs;
        c.scratch = (int)attr.localSizeBytes;
        if ((e = hipDeviceGetAttribute(&c.n_cu, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
        if (hipFuncSetAttribute(reinterpret_cast<const void *>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                160 * 1024) != hipSuccess)
            (void)hipGetLastError();
        c.ready = 1;
    }
    // occupancy depends on this shape's LDS
    if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&c.per_cu, reinterpret_cast<const void *>(kern), NT,
                                                          lo.total)) != hipSuccess)
        return e;
    if (dev < 64) cache[dev] = c;
    // instantiations that spill to scratch memory are not run
    if (c.per_cu < 1 || c.scratch > 0) return hipErrorNotSupported;
    int grid = c.n_cu * c.per_cu;
    if (grid > a.count) grid = a.count;
    if (p) {
        p->grid = grid;
        p->block = NT;
        p->per_cu = c.per_cu;
        p->n_cu = c.n_cu;
        p->vgprs = c.vgprs;
        p->scratch = c.scratch;
    }
    hipLaunchKernelGGL(kern, dim3(grid), dim3(NT), lo.total, s, a);
    return hipGetLastError();
}

template <int BITS, int GCPL, int R>
hipError_t gemv_dn(const GemvArgs &a, hipStream_t s, LayerPlan *p)
{
    const DownShape d = down_shape(a.I, BITS);
#define MOE_G(LPR_)                                                                                                    \
    case LPR_:                                                                                                         \
        return d.cpl <= 1 ? gemv_launch<BITS, GCPL, R, LPR_, 1>(a, s, p) : gemv_launch<BITS, GCPL, R, LPR_, 2>(a, s, p);
    switch (d.lpr) {
        MOE_G(1)
        MOE_G(2)
        MOE_G(4)
        MOE_G(8)
        MOE_G(16)
        MOE_G(32)
    default:
        return d.cpl <= 1 ? gemv_launch<BITS, GCPL, R, 64, 1>(a, s, p) : gemv_launch<BITS, GCPL, R, 64, 2>(a, s, p);
    }
#undef MOE_G
}

template <int BITS>
hipError_t gemv_bits(const GemvArgs &a, hipStream_t s, LayerPlan *p)
{
    const int nch = a.D * BITS / 128;  // 16-byte chunks of a gate/up row
    if (nch <= 64) return gemv_dn<BITS, 1, 2>(a, s, p);
    if (nch <= 128) return gemv_dn<BITS, 2, 1>(a, s, p);
    if constexpr (BITS == 4) return gemv_dn<BITS, 4, 1>(a, s, p);
    return hipErrorNotSupported;
}

}  // namespace

hipError_t launch_expert_gemv(const GemvArgs &a, int bits, hipStream_t s, LayerPlan *p)
{
    return bits == 4 ? gemv_bits<4>(a, s, p) : gemv_bits<2>(a, s, p);
}

}  // namespace moe
