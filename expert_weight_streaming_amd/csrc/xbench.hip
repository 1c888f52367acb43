// xbench.hip -- latency of the tagged all-gather exchanges of the persistent
// stack kernel, measured alone (a standalone program, not part of libmoe).
//
// One 512-thread block per CU, persistent.  Per iteration every block stores
// its share of W tagged 64-bit words (value low, epoch high; agent-scope
// single-copy atomic stores, as the stack kernel's exchanges), then the
// polling waves load all W words (agent-scope loads, every load of a round in
// flight) until each carries an epoch at least the iteration's.  Blocks that
// do not poll wait for their group's poller to finish the iteration, so that
// every block stores once per exchange.  Each block stamps the device clock
// (s_memrealtime, 100 MHz) after its own store and when its poll completes.
//
// Reported per case: the time from the last block's store to each poller's
// completion (median, 90th percentile, maximum over iterations and pollers),
// the spread of the store times, and the period of one exchange.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#define CK(x)                                                                                                          \
    do {                                                                                                               \
        hipError_t e_ = (x);                                                                                           \
        if (e_ != hipSuccess) {                                                                                        \
            printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__);                                     \
            exit(1);                                                                                                   \
        }                                                                                                              \
    } while (0)

namespace {

constexpr int kIters = 200;
constexpr uint32_t kSpins = 1u << 18;  // polls before a case is given up (flag)
constexpr size_t kDoneWord = 1u << 15;  // pacing words start here (word index)

struct Args {
    uint64_t *buf;           // exchange words, then pacing words
    uint64_t *stamps;        // [kIters][NB][2]
    uint32_t *flags;
    const uint4 *stream;     // background reads by waves 1..7 (or null)
    uint64_t stream_bytes;
    int W;                   // exchanged words
    int map;                 // 0: word w by block w % NB (interleaved); 1: block-contiguous
    int all_waves;           // 0: wave 0 polls all W; 1: every thread polls W / 512
    int pstep;               // blocks b % pstep == 0 poll
};

__device__ __forceinline__ bool tag_ge(uint32_t t, uint32_t want) { return (int32_t)(t - want) >= 0; }

__global__ void __launch_bounds__(512) k_xbench(Args a)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int NB = gridDim.x, b = blockIdx.x, W = a.W, wpb = W / NB;
    const bool poller = b % a.pstep == 0;
    __shared__ int bail;
    if (tid == 0) bail = 0;
    __syncthreads();
    for (int it = 0; it < kIters; ++it) {
        const uint32_t ep = (uint32_t)it + 1u;
        if (tid < wpb) {
            const int w = a.map == 0 ? b + NB * tid : b * wpb + tid;
            __hip_atomic_store(a.buf + w, ((uint64_t)ep << 32) | (uint32_t)(w + it), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
        const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
        bool timeout = false;
        if (!a.all_waves) {
            if (wave == 0 && poller) {
                for (uint32_t spins = 0;;) {
                    uint64_t v[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        v[j] = __hip_atomic_load(a.buf + min(lane + 64 * j, W - 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    bool ok = true;
#pragma unroll
                    for (int j = 0; j < 8; ++j) ok &= tag_ge((uint32_t)(v[j] >> 32), ep);
                    if (__all(ok)) break;
                    __builtin_amdgcn_s_sleep(1);
                    if (++spins == kSpins) {
                        timeout = true;
                        break;
                    }
                }
            } else if (wave > 0 && a.stream) {
                // a weight stream beside the poll: each block reads its slice
                const uint64_t per_block = a.stream_bytes / 16 / NB, chunk = per_block / kIters;
                const uint4 *p = a.stream + (uint64_t)b * per_block;
                uint32_t acc = 0;
                for (uint64_t i = (uint64_t)it * chunk + (tid - 64); i < (uint64_t)(it + 1) * chunk; i += 448) {
                    const uint4 q = p[i];
                    acc ^= q.x ^ q.w;
                }
                if (acc == 0x9E3779B9u) atomicOr(a.flags, 0x100u);  // keeps the loads
            }
        } else {
            const int per = W / 512;  // W a multiple of 512, at most 10 words per thread
            for (uint32_t spins = 0;;) {
                uint64_t v[10];
#pragma unroll
                for (int j = 0; j < 10; ++j)
                    v[j] = __hip_atomic_load(a.buf + min(tid * per + min(j, per - 1), W - 1), __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
                bool ok = true;
#pragma unroll
                for (int j = 0; j < 10; ++j) ok &= tag_ge((uint32_t)(v[j] >> 32), ep);
                if (__all(ok)) break;
                __builtin_amdgcn_s_sleep(1);
                if (++spins == kSpins) {
                    timeout = true;
                    break;
                }
            }
        }
        if (!a.all_waves && a.pstep > 1) {
            // pacing: the group's poller announces the end of its poll
            uint64_t *done = a.buf + kDoneWord + (size_t)(b - b % a.pstep) * 8;
            if (poller) {
                if (tid == 0) __hip_atomic_store(done, (uint64_t)ep << 32, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            } else if (wave == 0) {
                for (uint32_t spins = 0;;) {
                    if (tag_ge((uint32_t)(__hip_atomic_load(done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >> 32), ep)) break;
                    __builtin_amdgcn_s_sleep(1);
                    if (++spins == kSpins) {
                        timeout = true;
                        break;
                    }
                }
            }
        }
        const uint64_t t1 = __builtin_amdgcn_s_memrealtime();
        if (tid == 0) {
            a.stamps[((size_t)it * NB + b) * 2] = t0;
            a.stamps[((size_t)it * NB + b) * 2 + 1] = t1;
        }
        if (timeout) {
            atomicOr(a.flags, 1u);
            if (lane == 0) atomicOr(&bail, 1);
        }
        __syncthreads();
        if (bail) break;
    }
}

struct Case {
    const char *name;
    int W, map, all_waves, pstep, stream;
};

void run(const Case &c, Args a, int NB)
{
    a.W = c.W;
    a.map = c.map;
    a.all_waves = c.all_waves;
    a.pstep = c.pstep;
    if (!c.stream) a.stream = nullptr;
    CK(hipMemset(a.buf, 0, (kDoneWord + 8 * 1024) * 8));
    CK(hipMemset(a.flags, 0, 4));
    hipLaunchKernelGGL(k_xbench, dim3(NB), dim3(512), 0, 0, a);
    CK(hipGetLastError());
    CK(hipDeviceSynchronize());
    uint32_t flags = 0;
    CK(hipMemcpy(&flags, a.flags, 4, hipMemcpyDeviceToHost));
    std::vector<uint64_t> st((size_t)kIters * NB * 2);
    CK(hipMemcpy(st.data(), a.stamps, st.size() * 8, hipMemcpyDeviceToHost));
    std::vector<double> lat, skew, per;
    double prev = -1;
    for (int it = 2; it < kIters; ++it) {
        uint64_t last = 0, first = ~0ull, done = 0;
        for (int b = 0; b < NB; ++b) {
            const uint64_t s0 = st[((size_t)it * NB + b) * 2], s1 = st[((size_t)it * NB + b) * 2 + 1];
            last = std::max(last, s0);
            first = std::min(first, s0);
            if (b % c.pstep == 0) done = std::max(done, s1);
        }
        for (int b = 0; b < NB; b += c.pstep)
            lat.push_back(((double)st[((size_t)it * NB + b) * 2 + 1] - (double)last) * 0.01);
        skew.push_back((double)(last - first) * 0.01);
        if (prev >= 0) per.push_back(((double)done - prev) * 0.01);
        prev = (double)done;
    }
    auto q = [](std::vector<double> v, double f) {
        std::sort(v.begin(), v.end());
        return v[(size_t)(f * (double)(v.size() - 1))];
    };
    printf("| %s | %.2f | %.2f | %.2f | %.2f | %.2f | %s |\n", c.name, q(lat, 0.5), q(lat, 0.9), q(lat, 1.0), q(skew, 0.5),
           q(per, 0.5), flags & 1u ? "timeout" : "ok");
    fflush(stdout);
}

}  // namespace

int main()
{
    int dev = 0, ncu = 0;
    CK(hipGetDevice(&dev));
    CK(hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev));
    const int NB = ncu < 256 ? ncu : 256;
    Args a{};
    CK(hipMalloc(&a.buf, (kDoneWord + 8 * 1024) * 8));
    CK(hipMalloc(&a.stamps, (size_t)kIters * NB * 2 * 8));
    CK(hipMalloc(&a.flags, 4));
    const uint64_t SB = 4ull << 30;
    uint4 *sbuf = nullptr;
    CK(hipMalloc(&sbuf, SB));
    CK(hipMemset(sbuf, 1, SB));
    a.stream = sbuf;
    a.stream_bytes = SB;
    printf("%d CUs, %d blocks x 512 threads, %d exchanges per case; us\n\n", ncu, NB, kIters);
    printf("| case | after last store: median | p90 | max | store spread | period | |\n|---|---:|---:|---:|---:|---:|---|\n");
    const Case cs[] = {
        {"512 words (logits), written interleaved, 256 polling waves", 512, 0, 0, 1, 0},
        {"512 words, block-contiguous writers, 256 polling waves", 512, 1, 0, 1, 0},
        {"512 words, interleaved, 64 polling waves", 512, 0, 0, 4, 0},
        {"512 words, interleaved, 8 polling waves", 512, 0, 0, 32, 0},
        {"512 words, interleaved, 1 polling wave", 512, 0, 0, 256, 0},
        {"512 words, interleaved, 256 polling waves, 4 GiB read beside", 512, 0, 0, 1, 1},
        {"512 words, interleaved, 8 polling waves, 4 GiB read beside", 512, 0, 0, 32, 1},
        {"4096 words (residual rows), block-contiguous, all threads poll", 4096, 1, 1, 1, 0},
        {"4096 words, interleaved writers, all threads poll", 4096, 0, 1, 1, 0},
        {"5120 words (h), block-contiguous, all threads poll", 5120, 1, 1, 1, 0},
    };
    for (const Case &c : cs)
        if (c.W % NB == 0 && (!c.all_waves || c.W % 512 == 0)) run(c, a, NB);
    CK(hipFree(sbuf));
    CK(hipFree(a.buf));
    CK(hipFree(a.stamps));
    CK(hipFree(a.flags));
    return 0;
}
