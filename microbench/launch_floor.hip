// Launch floor of back-to-back kernels on one stream, on gfx950: what a
// one-kernel-per-step loop at small N pays before doing any arithmetic.
//
// Three kernels, each launched many times in a row and timed with hipEvents:
//   empty  - returns at once;
//   stage  - the memory skeleton of the small-N step: every 256-thread
//            workgroup reads all N bodies through 1024-body LDS tiles (two
//            barriers per tile), reduces the per-thread sums as that kernel
//            does (xor butterfly in each wave, then the wave sums in order)
//            and writes one record per target it owns (4 per workgroup);
//   chain  - the same, reading the bodies the previous launch wrote (two
//            buffers, alternating, like the positions of a step loop), so
//            each launch depends on the last one through memory.
// Output: one JSON line per (kernel, grid) with microseconds per launch.
//
// Build: hipcc --offload-arch=gfx950 -O3 -Xclang -target-feature -Xclang -packed-fp32-ops \
//          microbench/launch_floor.hip -o _build/launch_floor
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>

#define CHECK(x)                                                                        \
    do {                                                                                \
        hipError_t e_ = (x);                                                            \
        if (e_ != hipSuccess) {                                                         \
            fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));              \
            exit(1);                                                                    \
        }                                                                               \
    } while (0)

constexpr int kWG = 256;
constexpr int kTile = 1024;
constexpr int kTargets = 4;  // targets per workgroup

__global__ void __launch_bounds__(kWG) empty_kernel(float4 *out)
{
    // never true for the grids used here; keeps the store (and the argument) alive
    if (blockIdx.x == 0x7fffffff) out[threadIdx.x] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
}

// n >= 1; `out` has at least n records; the grid covers n / kTargets workgroups.
__global__ void __launch_bounds__(kWG) stage_kernel(const float4 *__restrict__ in, int n,
                                                    float4 *__restrict__ out)
{
    __shared__ float4 tile[kTile];
    __shared__ float4 red[kWG / 64][kTargets];
    float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    for (int t0 = 0; t0 < n; t0 += kTile) {
        for (int i = threadIdx.x; i < kTile; i += kWG) {
            const int j = t0 + i;
            tile[i] = in[j < n ? j : n - 1];
        }
        __syncthreads();
        for (int u = 0; u < kTile / kWG; ++u) {
            const float4 b = tile[u * kWG + threadIdx.x];
            acc.x += b.x;
            acc.y += b.y;
            acc.z += b.z;
            acc.w += b.w;
        }
        __syncthreads();
    }
    // the small-N kernel's reduction: an xor butterfly inside each wave over the
    // lanes of one target, then the four wave sums in order
    for (int m = kTargets; m < 64; m <<= 1) {
        acc.x += __shfl_xor(acc.x, m);
        acc.y += __shfl_xor(acc.y, m);
        acc.z += __shfl_xor(acc.z, m);
        acc.w += __shfl_xor(acc.w, m);
    }
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    if (lane < kTargets) red[w][lane] = acc;
    __syncthreads();
    if (threadIdx.x < kTargets) {
        float4 s = red[0][threadIdx.x];
        for (int k = 1; k < kWG / 64; ++k) {
            const float4 b = red[k][threadIdx.x];
            s.x += b.x;
            s.y += b.y;
            s.z += b.z;
            s.w += b.w;
        }
        const int i = blockIdx.x * kTargets + threadIdx.x;
        // scaled back so that the chained buffers stay bounded
        if (i < n) out[i] = make_float4(s.x * 1e-6f, s.y * 1e-6f, s.z * 1e-6f, s.w * 1e-6f);
    }
}

int main(int argc, char **argv)
{
    const int n = argc > 1 ? atoi(argv[1]) : 2048;
    const int reps = 2000, warm = 200;
    if (n < 1 || n > (1 << 20)) {
        fprintf(stderr, "n must be in [1, 2^20]\n");
        return 1;
    }
    float4 *a = nullptr, *b = nullptr;
    CHECK(hipMalloc(&a, (size_t)n * sizeof(float4)));
    CHECK(hipMalloc(&b, (size_t)n * sizeof(float4)));
    CHECK(hipMemset(a, 0, (size_t)n * sizeof(float4)));
    CHECK(hipMemset(b, 0, (size_t)n * sizeof(float4)));
    hipStream_t s;
    CHECK(hipStreamCreate(&s));
    hipEvent_t e0, e1;
    CHECK(hipEventCreate(&e0));
    CHECK(hipEventCreate(&e1));
    const int stage_grid = (n + kTargets - 1) / kTargets;
    const char *names[3] = {"empty", "stage", "chain"};
    for (int kind = 0; kind < 3; ++kind) {
        for (int grid : {1, 64, 256, stage_grid}) {
            if (kind > 0 && grid != stage_grid) continue;  // the skeletons cover all targets
            auto launch = [&](int r) {
                if (kind == 0) {
                    empty_kernel<<<grid, kWG, 0, s>>>(a);
                } else if (kind == 1) {
                    stage_kernel<<<grid, kWG, 0, s>>>(a, n, b);
                } else {
                    const bool even = r % 2 == 0;
                    stage_kernel<<<grid, kWG, 0, s>>>(even ? a : b, n, even ? b : a);
                }
            };
            for (int r = 0; r < warm; ++r) launch(r);
            CHECK(hipGetLastError());
            CHECK(hipEventRecord(e0, s));
            for (int r = 0; r < reps; ++r) launch(r);
            CHECK(hipEventRecord(e1, s));
            CHECK(hipEventSynchronize(e1));
            CHECK(hipGetLastError());
            float ms = 0.0f;
            CHECK(hipEventElapsedTime(&ms, e0, e1));
            printf("{\"kernel\": \"%s\", \"n\": %d, \"grid\": %d, \"workgroup\": %d, "
                   "\"us_per_launch\": %.3f}\n",
                   names[kind], n, grid, kWG, 1000.0 * ms / reps);
        }
    }
    CHECK(hipFree(a));
    CHECK(hipFree(b));
    return 0;
}
