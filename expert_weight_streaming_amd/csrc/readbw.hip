// readbw.hip -- the HBM read rate a plain streaming read reaches on this
// part (a standalone program, not part of libmoe): the ceiling against which
// the dequant GEMV's rate is read, next to the nominal 8 TB/s.
//
// A 3,623,878,656-byte buffer (512 blobs of a hidden-4096, inter-1024,
// 4-bit expert: the bytes one all-experts GEMV launch reads) is read with
// 16-byte loads and folded into one word per thread, so that no load is
// dead; nothing is written but one word per workgroup when the fold hits a
// marker value that the buffer's contents never produce.  Two access shapes:
//   grid-stride: thread i of the grid reads i, i + G, ... (G = grid threads),
//                U loads of a thread in flight together;
//   contiguous:  workgroup b reads its own contiguous range (as one expert
//                per workgroup in the GEMV), U loads in flight.
// Each case: 3 untimed launches, then 10 launches between two HIP events.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>

#define CHECK(x)                                                                          \
    do {                                                                                  \
        hipError_t e_ = (x);                                                              \
        if (e_ != hipSuccess) {                                                           \
            std::printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__);    \
            std::exit(1);                                                                 \
        }                                                                                 \
    } while (0)

constexpr int kMarker = 0x2468ACE1;  // the fold of an all-0x01 buffer never equals it

template <int U>
__global__ void k_read_strided(const int4 *__restrict__ p, size_t n16, int *out)
{
    int acc = 0;
    const size_t g = (size_t)gridDim.x * blockDim.x;
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i + (U - 1) * g < n16; i += U * g) {
        int4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = p[i + u * g];
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n16; i += g) {
        const int4 v = p[i];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (acc == kMarker) out[blockIdx.x] = acc;
}

template <int U>
__global__ void k_read_contig(const int4 *__restrict__ p, size_t per_block16, int *out)
{
    int acc = 0;
    const int4 *q = p + (size_t)blockIdx.x * per_block16;
    size_t i = threadIdx.x;
    for (; i + (U - 1) * blockDim.x < per_block16; i += U * blockDim.x) {
        int4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = q[i + u * blockDim.x];
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < per_block16; i += blockDim.x) {
        const int4 v = q[i];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (acc == kMarker) out[blockIdx.x] = acc;
}

int main()
{
    const size_t bytes = 3623878656ull, n16 = bytes / 16;
    int4 *p = nullptr;
    int *out = nullptr;
    CHECK(hipMalloc(&p, bytes));
    CHECK(hipMalloc(&out, 1 << 16));  // one word per workgroup: grids up to 16,384
    CHECK(hipMemset(p, 1, bytes));
    hipEvent_t a, b;
    CHECK(hipEventCreate(&a));
    CHECK(hipEventCreate(&b));
    std::printf("| case | grid x threads | loads in flight per thread | us per launch | GB/s | of 8 TB/s |\n");
    std::printf("|---|---:|---:|---:|---:|---:|\n");
    auto run = [&](const char *name, int grid, int threads, int u, auto launch) {
        for (int w = 0; w < 3; ++w) launch();
        CHECK(hipGetLastError());
        CHECK(hipDeviceSynchronize());
        CHECK(hipEventRecord(a, 0));
        for (int it = 0; it < 10; ++it) launch();
        CHECK(hipEventRecord(b, 0));
        CHECK(hipEventSynchronize(b));
        float ms = 0.f;
        CHECK(hipEventElapsedTime(&ms, a, b));
        const double us = ms * 100.0, gbs = bytes / (us * 1e3);
        std::printf("| %s | %d x %d | %d | %.1f | %.0f | %.1f%% |\n", name, grid, threads, u, us, gbs, gbs / 80.0);
        std::fflush(stdout);
    };
    for (int g : {256, 512, 1024, 4096}) {
        run("grid-stride", g, 256, 4, [&] { k_read_strided<4><<<g, 256>>>(p, n16, out); });
        run("grid-stride", g, 512, 8, [&] { k_read_strided<8><<<g, 512>>>(p, n16, out); });
    }
    // contiguous ranges: the grids divide the buffer exactly
    run("contiguous", 512, 512, 4, [&] { k_read_contig<4><<<512, 512>>>(p, n16 / 512, out); });
    run("contiguous", 512, 512, 8, [&] { k_read_contig<8><<<512, 512>>>(p, n16 / 512, out); });
    run("contiguous", 1024, 512, 8, [&] { k_read_contig<8><<<1024, 512>>>(p, n16 / 1024, out); });
    run("contiguous", 4096, 256, 8, [&] { k_read_contig<8><<<4096, 256>>>(p, n16 / 4096, out); });
    CHECK(hipFree(p));
    CHECK(hipFree(out));
    return 0;
}
