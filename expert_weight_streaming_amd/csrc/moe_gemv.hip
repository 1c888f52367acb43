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
// waves read neighbouring rows at any time.  A wave's registers hold one
// unit (one gate/up row pair, or 8 to 16 down rows), so that the kernel fits
// 128 registers and four waves run per SIMD.  At the pages' layer shape
// (k_expert_gemv_st) the next unit streams into an LDS stage while the
// current one is computed, and h and y leave the chip in one coalesced pass
// per expert; other shapes take k_expert_gemv, whose units are loaded
// straight into registers.
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

// ---------------------------------------------------------------------------
// The same GEMVs with the next unit's weights in flight while a wave
// computes.  A wave's registers hold one unit (the 128-register budget of
// four waves per SIMD leaves no room for a second), so the next unit is
// requested straight into LDS (buffer loads with the LDS destination: no
// registers, no waiting at issue): per wave one stage of up to four
// 16-byte chunks and four scale/bias words per lane.  The unit in the stage
// is copied into registers (vmcnt(0) first: only the stage's loads and the
// h stores are outstanding then), the stage is refilled with the unit
// after, and the copied unit is computed while that refill streams.  The
// tables live in fixed-size LDS arrays, distinct objects from the stage, so
// that the compiler sees that the tables' reads do not depend on the stage's
// loads and puts no wait for them in front of the arithmetic.  Capacity:
// D <= 4096, I <= 1024 (the pages' layer shape; others take k_expert_gemv).
constexpr int kStDmax = 4096, kStImax = 1024, kStSlots = 4;

#define MOE_LDSP(p) ((__attribute__((address_space(3))) void *)(p))

// wait for every outstanding vector-memory operation of the wave (gfx9
// s_waitcnt: vmcnt 0, expcnt and lgkmcnt left open)
__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// wait for every outstanding LDS operation of the wave (vmcnt left open)
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

template <int BITS>
struct StLds {
    using C = Codes<BITS>;
    static constexpr int XCH = kStDmax * BITS / 128, HCH = kStImax * BITS / 128;
    int dig[XCH * C::DW];
    float csum[XCH], cinv[XCH];
    float h[kStImax];
    float y[kStDmax];
    int hdig[HCH * C::DW];
    float hcsum[HCH], hcinv[HCH];
};

// gate/up unit (rows i0 .. i0+R-1) -> stage: slot (m*R + r)*2 + mat
template <int BITS, int CPL, int R>
__device__ __forceinline__ void gu_stage(__amdgpu_buffer_rsrc_t rs, uint4 (*sq)[64], uint32_t (*ssb)[64], int D, int I,
                                         int i0, int lane)
{
    static_assert(CPL * R * 2 <= kStSlots, "stage slots");
    const int nchunks = D * BITS / 128;
    const uint32_t mat_q = (uint32_t)I * D * BITS / 8, row_q = (uint32_t)D * BITS / 8;
    const uint32_t sb0 = 3 * mat_q, mat_sb = (uint32_t)I * (D / kGroup) * 4, row_sb = (uint32_t)(D / kGroup) * 4;
#pragma unroll
    for (int m = 0; m < CPL; ++m) {
        const int c = lane + 64 * m;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int i = i0 + r;
            if (i >= I || c >= nchunks) continue;
#pragma unroll
            for (int mat = 0; mat < 2; ++mat)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, MOE_LDSP(&sq[(m * R + r) * 2 + mat][0]), 16,
                                                         (uint32_t)c * 16, mat * mat_q + (uint32_t)i * row_q, 0, 0);
        }
    }
    // a row's scale/bias words (D/64 <= 64 of them), word l in lane l, in
    // slot r*2 + mat
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int i = i0 + r;
        if (i >= I || lane >= D / kGroup) continue;
#pragma unroll
        for (int mat = 0; mat < 2; ++mat)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, MOE_LDSP(&ssb[r * 2 + mat][0]), 4, (uint32_t)lane * 4,
                                                     sb0 + mat * mat_sb + (uint32_t)i * row_sb, 0, 0);
    }
}

template <int BITS, int CPL, int R>
__device__ __forceinline__ void gu_unstage(GuRegs<BITS, CPL, R> &g, const uint4 (*sq)[64], const uint32_t (*ssb)[64],
                                           int D, int I, int i0, int lane)
{
    const int nchunks = D * BITS / 128;
    using C = Codes<BITS>;
#pragma unroll
    for (int m = 0; m < CPL; ++m) {
        const int c = lane + 64 * m;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const bool ok = i0 + r < I && c < nchunks;
#pragma unroll
            for (int mat = 0; mat < 2; ++mat) {
                g.q[m][r][mat] = ok ? sq[(m * R + r) * 2 + mat][lane] : make_uint4(0, 0, 0, 0);
                g.sb[m][r][mat] = ok ? ssb[r * 2 + mat][c * C::CODES / kGroup] : 0u;
            }
        }
    }
}

// down unit (S row groups of RPU rows from o0) -> stage: slot s*DCPL + m
template <int BITS, int LPR, int DCPL, int S>
__device__ __forceinline__ void dn_stage(__amdgpu_buffer_rsrc_t rs, uint4 (*sq)[64], uint32_t (*ssb)[64], int D, int I,
                                         int o0, int lane)
{
    constexpr int RPU = 64 / LPR;
    static_assert(S * DCPL <= kStSlots, "stage slots");
    const int nchunks = I * BITS / 128, lc = lane % LPR;
    const uint32_t mat_q = (uint32_t)I * D * BITS / 8, row_q = (uint32_t)I * BITS / 8;
    const uint32_t sbd = 3 * mat_q + 2 * ((uint32_t)D * (I / kGroup) * 4), row_sb = (uint32_t)(I / kGroup) * 4;
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const int os = o0 + s * RPU;
        const int o = os + lane / LPR;
#pragma unroll
        for (int m = 0; m < DCPL; ++m) {
            const int c = lc + LPR * m;
            if (o >= D || c >= nchunks) continue;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, MOE_LDSP(&sq[s * DCPL + m][0]), 16,
                                                     (uint32_t)(lane / LPR) * row_q + (uint32_t)c * 16,
                                                     2 * mat_q + (uint32_t)os * row_q, 0, 0);
        }
    }
    // the scale/bias words of the unit's rows (contiguous in the blob, I/64
    // per row, at most 64 * S * DCPL): word w in lane w % 64 of slot w / 64;
    // words of rows past D are not requested
    const int rows = D - o0 < RPU * S ? D - o0 : RPU * S;
    const int nw = rows * (I / kGroup);
#pragma unroll
    for (int q = 0; q < S * DCPL; ++q) {
        if (64 * q >= nw) break;
        if (64 * q + lane < nw)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, MOE_LDSP(&ssb[q][0]), 4, (uint32_t)(64 * q + lane) * 4,
                                                     sbd + (uint32_t)o0 * row_sb, 0, 0);
    }
}

template <int BITS, int LPR, int DCPL, int S>
__device__ __forceinline__ void dn_unstage(DnUnit<BITS, DCPL, S> &u, const uint4 (*sq)[64], const uint32_t (*ssb)[64],
                                           int D, int I, int o0, int lane)
{
    constexpr int RPU = 64 / LPR;
    const int nchunks = I * BITS / 128, lc = lane % LPR;
    using C = Codes<BITS>;
    const int *sbw = reinterpret_cast<const int *>(ssb);
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const int o = o0 + s * RPU + lane / LPR;
#pragma unroll
        for (int m = 0; m < DCPL; ++m) {
            const int c = lc + LPR * m;
            const bool ok = o < D && c < nchunks;
            u.d[s].q[m] = ok ? sq[s * DCPL + m][lane] : make_uint4(0, 0, 0, 0);
            u.d[s].sb[m] = ok ? (uint32_t)sbw[(o - o0) * (I / kGroup) + c * C::CODES / kGroup] : 0u;
        }
    }
}

template <int BITS, int GCPL, int R, int LPR, int DCPL>
__global__ void __launch_bounds__(NT, 4) k_expert_gemv_st(GemvArgs a)
{
    constexpr int RPU = 64 / LPR;
    constexpr int S0 = 16 / RPU > 0 ? 16 / RPU : 1;
    constexpr int S = S0 * DCPL > 4 ? 4 / DCPL : S0;
    constexpr int RPD = RPU * S;
    __shared__ __align__(16) StLds<BITS> t;
    __shared__ __align__(16) uint4 s_q[NW][kStSlots][64];
    __shared__ __align__(16) uint32_t s_sb[NW][kStSlots][64];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int D = a.D, I = a.I;
    uint4 (*sq)[64] = s_q[wave];
    uint32_t (*ssb)[64] = s_sb[wave];

    digit_table<BITS>(a.x, D, t.dig, t.csum, t.cinv);
    lds_barrier();

    const int ngu = (I + R - 1) / R;
    const int ndn = (D + RPD - 1) / RPD;
    for (int n = blockIdx.x; n < a.count; n += gridDim.x) {
        const uint8_t *blob = a.experts + (uint64_t)(a.first + n) * a.blob_bytes;
        const __amdgpu_buffer_rsrc_t rs = blob_rsrc(blob);
        float *hn = a.h + (size_t)n * I;
        float *yn = a.y + (size_t)n * D;
        if (wave < ngu) gu_stage<BITS, GCPL, R>(rs, sq, ssb, D, I, wave * R, lane);
        for (int u = wave; u < ngu; u += NW) {
            GuRegs<BITS, GCPL, R> g;
            wait_vm0();
            gu_unstage<BITS, GCPL, R>(g, sq, ssb, D, I, u * R, lane);
            wait_lgkm0();
            if (u + NW < ngu) gu_stage<BITS, GCPL, R>(rs, sq, ssb, D, I, (u + NW) * R, lane);
            float hv[R];
            gu_finish_c<BITS, GCPL, R>(g, t.dig, t.csum, t.cinv, D, lane, hv);
            if (lane == 0) {
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const int i = u * R + r;
                    if (i < I) t.h[i] = hv[r];
                }
            }
        }
        // the first down unit streams while h is completed and converted
        if (wave < ndn) dn_stage<BITS, LPR, DCPL, S>(rs, sq, ssb, D, I, wave * RPD, lane);
        lds_barrier();
        digit_table<BITS>(t.h, I, t.hdig, t.hcsum, t.hcinv);
        for (int i = threadIdx.x; i < I; i += NT) hn[i] = t.h[i];
        lds_barrier();
        for (int u = wave; u < ndn; u += NW) {
            DnUnit<BITS, DCPL, S> d;
            wait_vm0();
            dn_unstage<BITS, LPR, DCPL, S>(d, sq, ssb, D, I, u * RPD, lane);
            wait_lgkm0();
            if (u + NW < ndn) dn_stage<BITS, LPR, DCPL, S>(rs, sq, ssb, D, I, (u + NW) * RPD, lane);
            dn_unit_finish<BITS, LPR, DCPL, S>(d, t.hdig, t.hcsum, t.hcinv, I, D, u * RPD, lane, t.y);
        }
        // y leaves in one coalesced pass (no stores between a wave's stage
        // refills, whose wait would also wait for them)
        lds_barrier();
        for (int o = threadIdx.x; o < D; o += NT) yn[o] = t.y[o];
    }
}

struct GemvPlanCache {
    int ready = 0, n_cu = 0, per_cu = 0, vgprs = 0, scratch = 0;
};

// One kernel instantiation's launch: its attributes are read once per
// device; the grid fills every CU at the occupancy this shape's LDS allows.
template <typename Kern>
hipError_t gemv_run(Kern kern, GemvPlanCache *cache, uint32_t lds_bytes, const GemvArgs &a, hipStream_t s,
                    LayerPlan *p)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    GemvPlanCache c = dev < 64 ? cache[dev] : GemvPlanCache{};
    if (!c.ready) {
        hipFuncAttributes attr;
        if ((e = hipFuncGetAttributes(&attr, reinterpret_cast<const void *>(kern))) != hipSuccess) return e;
        c.vgprs = attr.numRegs;
        c.scratch = (int)attr.localSizeBytes;
        if ((e = hipDeviceGetAttribute(&c.n_cu, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
        if (lds_bytes > 0 && hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024) != hipSuccess)
            (void)hipGetLastError();
        c.ready = 1;
    }
    // occupancy depends on this shape's LDS
    if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&c.per_cu, reinterpret_cast<const void *>(kern), NT,
                                                          lds_bytes)) != hipSuccess)
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
    hipLaunchKernelGGL(kern, dim3(grid), dim3(NT), lds_bytes, s, a);
    return hipGetLastError();
}

template <int BITS, int GCPL, int R, int LPR, int DCPL>
hipError_t gemv_launch(const GemvArgs &a, hipStream_t s, LayerPlan *p)
{
    constexpr int RPU = 64 / LPR;
    constexpr int S0 = 16 / RPU > 0 ? 16 / RPU : 1;
    constexpr int S = S0 * DCPL > 4 ? 4 / DCPL : S0;
    // the staged kernel where its fixed tables hold the shape and a unit
    // fits its stage
    if constexpr (GCPL * R * 2 <= kStSlots && S * DCPL <= kStSlots && gemv_waves<BITS, GCPL>() == 4) {
        // (a down unit's scale/bias words must fit the stage's 64 * S * DCPL
        // words, which holds whenever its LPR * DCPL lanes cover a row)
        if (a.D <= kStDmax && a.I <= kStImax && RPU * S * (a.I / kGroup) <= 64 * S * DCPL) {
            static GemvPlanCache cache[64];
            return gemv_run(k_expert_gemv_st<BITS, GCPL, R, LPR, DCPL>, cache, 0u, a, s, p);
        }
    }
    static GemvPlanCache cache[64];
    return gemv_run(k_expert_gemv<BITS, GCPL, R, LPR, DCPL>, cache, gemv_lds(a.D, a.I, BITS).total, a, s, p);
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
