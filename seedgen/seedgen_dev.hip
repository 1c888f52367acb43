// seedgen_dev.hip -- device twin of the expert-blob generator in seedgen.c.
//
// Writes, directly into HBM, the same bytes sg_blob() writes on the host, so
// that multi-GB expert arenas need not cross PCIe.  It holds no MoE
// arithmetic: SplitMix64 outputs (Steele, Lea, Flood, OOPSLA 2014) used
// counter-style, uniform draws rounded to bf16.  Every fp32 step of the
// uniform mapping is a separately rounded multiply and add (contraction off
// here and in the build flags), matching the host's -ffp-contract=off build.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kGolden = 0x9E3779B97F4A7C15ULL;

__device__ __host__ inline uint64_t mix64(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

__device__ __host__ inline uint64_t stream_key(uint64_t seed, uint64_t layer, uint64_t expert, uint64_t stream)
{
    uint64_t k = mix64(seed + kGolden);
    k = mix64(k ^ (layer + 1) * 0xD1B54A32D192ED03ULL);
    k = mix64(k ^ (expert + 1) * 0xABC98388FB8FAC03ULL);
    k = mix64(k ^ (stream + 1) * 0x8CB92BA72F3D8DD7ULL);
    return k;
}

__device__ inline uint32_t bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (u >> 16) | 0x40u;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ inline float unif24(uint32_t u24, float lo, float width)
{
#pragma clang fp contract(off)
    float t = __fmul_rn((float)u24, 1.0f / 16777216.0f);
    return __fadd_rn(lo, __fmul_rn(t, width));
}

struct BlobJob {
    uint64_t seed;
    uint64_t blob_bytes;   // distance between consecutive blobs in dst
    uint64_t q_pairs;      // 64-bit outputs in the q region (2 words each)
    uint64_t n_groups;     // group words in the sb region
    int32_t layer, expert0;
    float s_lo, s_w, b_lo, b_w;
};

// blockIdx.y = blob number within the launch; expert id = expert0 + blockIdx.y,
// or the fixed id `expert0` when ids_fixed is set (the shared blob).
__global__ void __launch_bounds__(256) blob_kernel(BlobJob job, int ids_fixed, uint8_t *dst)
{
    const uint32_t b = blockIdx.y;
    const uint64_t expert = (uint64_t)(uint32_t)(ids_fixed ? job.expert0 : job.expert0 + (int32_t)b);
    uint8_t *blob = dst + (uint64_t)b * job.blob_bytes;
    const uint64_t kq = stream_key(job.seed, (uint64_t)job.layer, expert, 0);
    const uint64_t ks = stream_key(job.seed, (uint64_t)job.layer, expert, 1);
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    const uint64_t t0 = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    uint2 *q = reinterpret_cast<uint2 *>(blob);
    for (uint64_t p = t0; p < job.q_pairs; p += stride) {
        uint64_t z = mix64(kq + (p + 1) * kGolden);
        q[p] = make_uint2((uint32_t)z, (uint32_t)(z >> 32));
    }
    uint32_t *sb = reinterpret_cast<uint32_t *>(blob + job.q_pairs * 8);
    for (uint64_t n = t0; n < job.n_groups; n += stride) {
        uint64_t z = mix64(ks + (n + 1) * kGolden);
        float s = unif24((uint32_t)(z >> 40), job.s_lo, job.s_w);
        float bb = unif24((uint32_t)(z >> 8) & 0xFFFFFFu, job.b_lo, job.b_w);
        sb[n] = bf16_rne(s) | (bf16_rne(bb) << 16);
    }
}

}  // namespace

extern "C" {

// Fill n_blobs consecutive canonical blobs at dst (device pointer, blobs
// blob_bytes apart) for experts expert0 .. expert0+n_blobs-1 of `layer`
// (or n_blobs copies of expert0's blob when ids_fixed != 0).  Returns the
// hipError_t of the launch (0 on success).  Asynchronous on `stream`.
int sg_dev_blobs(uint64_t seed, int32_t layer, int32_t expert0, int32_t n_blobs, int32_t ids_fixed,
                 int32_t D, int32_t I, int32_t bits, int32_t group,
                 float s_lo, float s_hi, float b_lo, float b_hi, void *dst, void *stream)
{
    if (n_blobs <= 0 || D <= 0 || I <= 0 || group <= 0 || (bits != 2 && bits != 4) || !dst) return -1;
    const uint64_t n = 3ull * (uint64_t)D * (uint64_t)I;
    if ((n * (uint64_t)bits) % 64 != 0 || n % (uint64_t)group != 0) return -1;
    BlobJob job;
    job.seed = seed;
    job.q_pairs = n * (uint64_t)bits / 64;
    job.n_groups = n / (uint64_t)group;
    job.blob_bytes = job.q_pairs * 8 + job.n_groups * 4;
    job.layer = layer;
    job.expert0 = expert0;
    volatile float sw = s_hi - s_lo, bw = b_hi - b_lo;
    job.s_lo = s_lo;
    job.s_w = sw;
    job.b_lo = b_lo;
    job.b_w = bw;
    uint64_t per_blob = job.q_pairs > job.n_groups ? job.q_pairs : job.n_groups;
    uint64_t gx = (per_blob + 255) / 256;
    if (gx > 1024) gx = 1024;
    for (int32_t b0 = 0; b0 < n_blobs; b0 += 65535) {
        int32_t nb = n_blobs - b0 < 65535 ? n_blobs - b0 : 65535;
        BlobJob j = job;
        if (!ids_fixed) j.expert0 = expert0 + b0;
        hipLaunchKernelGGL(blob_kernel, dim3((uint32_t)gx, (uint32_t)nb), dim3(256), 0, (hipStream_t)stream, j,
                           ids_fixed, (uint8_t *)dst + (uint64_t)b0 * job.blob_bytes);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return (int)e;
    }
    return 0;
}

}  // extern "C"
