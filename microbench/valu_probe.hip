// Issue-rate probe for the instructions the all-pairs inner step is made of,
// on gfx950: v_fma_f32, v_rsq_f32, and mixes of the two, plus the cost of the
// three source-broadcast paths (LDS uniform reads, v_readlane, scalar loads).
//
// Every kernel runs independent dependency chains per lane (enough of them to
// cover the ALU latency), on a grid of 8 waves per SIMD, for a fixed number of
// iterations. The host times each launch with hipEvents and reads the shader
// clock of one wave (s_memtime against s_memrealtime, the 100 MHz constant
// clock) to turn time into cycles. Output: one JSON line per kernel with
// lane-operations per second and issue cycles per wave-instruction.
//
// Build: hipcc --offload-arch=gfx950 -O3 -Xclang -target-feature -Xclang -packed-fp32-ops \
//          microbench/valu_probe.hip -o _build/valu_probe
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <vector>

#define CHECK(x)                                                                        \
    do {                                                                                \
        hipError_t e_ = (x);                                                            \
        if (e_ != hipSuccess) {                                                         \
            fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));              \
            exit(1);                                                                    \
        }                                                                               \
    } while (0)

constexpr int kChains = 8;

struct Clock {
    unsigned long long c0, c1, r0, r1;
};

__device__ __forceinline__ void clock_begin(Clock *ck)
{
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        ck->r0 = __builtin_amdgcn_s_memrealtime();
        ck->c0 = __builtin_amdgcn_s_memtime();
    }
}

__device__ __forceinline__ void clock_end(Clock *ck)
{
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        ck->c1 = __builtin_amdgcn_s_memtime();
        ck->r1 = __builtin_amdgcn_s_memrealtime();
    }
}

// K FMAs per chain per step, plus one v_rsq_f32 per chain per step when RSQ.
template <int K, bool RSQ>
__global__ void __launch_bounds__(256) mix_kernel(float *out, int iters, float a, Clock *ck)
{
    clock_begin(ck);
    float x[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) x[c] = 1.0f + 1e-3f * (threadIdx.x + c);
    const float b = 0.5f * a;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < kChains; ++c) {
            if constexpr (RSQ) x[c] = __builtin_amdgcn_rsqf(x[c]);  // x stays positive
#pragma unroll
            for (int k = 0; k < K; ++k) x[c] = __builtin_fmaf(x[c], a, b);
        }
    }
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < kChains; ++c) s += x[c];
    out[blockIdx.x * 256 + threadIdx.x] = s;
    clock_end(ck);
}

// Only v_rsq_f32: four dependent rounds over the chains per iteration.
__global__ void __launch_bounds__(256) rsq_kernel(float *out, int iters, float a, Clock *ck)
{
    clock_begin(ck);
    float x[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) x[c] = 1.0f + 1e-3f * (threadIdx.x + c) + a;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
#pragma unroll
            for (int c = 0; c < kChains; ++c) x[c] = __builtin_amdgcn_rsqf(x[c]);
        }
    }
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < kChains; ++c) s += x[c];
    out[blockIdx.x * 256 + threadIdx.x] = s;
    clock_end(ck);
}


// Operand-source variants of a dependent-chain FMA/MUL/SUB stream. OPS:
//   0: v_fma_f32 x, x, a, b with a, b in VGPRs      1: same with a, b from SGPRs
//   2: v_mul_f32 x, x, a (VGPR)                       3: v_sub_f32 x, a, x (VGPR)
//   4: v_sub_f32 x, s, x (SGPR)
template <int OPS>
__global__ void __launch_bounds__(256) op_kernel(float *out, int iters, float a_s, Clock *ck)
{
    clock_begin(ck);
    float x[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) x[c] = 1.0f + 1e-3f * (threadIdx.x + c);
    // lane-varying operands live in VGPRs; a_s/b_s are uniform kernel arguments (SGPRs)
    const float a_v = 0.999f + 1e-9f * threadIdx.x, b_v = 0.5f * a_v;
    const float b_s = 0.5f * a_s;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
#pragma unroll
            for (int c = 0; c < kChains; ++c) {
                if constexpr (OPS == 0) x[c] = __builtin_fmaf(x[c], a_v, b_v);
                if constexpr (OPS == 1) x[c] = __builtin_fmaf(x[c], a_s, b_s);
                if constexpr (OPS == 2) x[c] = x[c] * a_v;
                if constexpr (OPS == 3) x[c] = a_v - x[c];
                if constexpr (OPS == 4) x[c] = a_s - x[c];
            }
        }
    }
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < kChains; ++c) s += x[c];
    out[blockIdx.x * 256 + threadIdx.x] = s;
    clock_end(ck);
}

// rsq interleaved with K independent FMAs of the other chains (no FMA waits on the
// rsq issued just before it), all operands in VGPRs.
template <int K>
__global__ void __launch_bounds__(256) rsq_overlap_kernel(float *out, int iters, float a_s,
                                                          Clock *ck)
{
    clock_begin(ck);
    float x[kChains], y[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) {
        x[c] = 1.0f + 1e-3f * (threadIdx.x + c);
        y[c] = x[c];
    }
    const float a_v = 0.999f + 1e-9f * threadIdx.x, b_v = 0.5f * a_v;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < kChains; ++c) {
            y[c] = __builtin_amdgcn_rsqf(x[c]);
#pragma unroll
            for (int k = 0; k < K; ++k) {
                const int o = (c + 1 + k) % kChains;
                x[o] = __builtin_fmaf(x[o], a_v, b_v);
            }
        }
#pragma unroll
        for (int c = 0; c < kChains; ++c) x[c] = __builtin_fmaf(y[c], a_v, x[c]);
    }
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < kChains; ++c) s += x[c] + y[c];
    out[blockIdx.x * 256 + threadIdx.x] = s;
    clock_end(ck);
}

// The all-pairs inner step itself, operands all in VGPRs (no memory traffic in
// the loop): per interaction 3 sub, 3 FMA (q), rsq, 3 mul, 3 FMA (a) and, with
// POT, 1 FMA (p). MODE 1 replaces the rsq by a multiply, to price the rsq. The
// target drifts by 3 FMAs per 8 interactions so that no work is loop-invariant.
template <bool POT, int MODE>
__global__ void __launch_bounds__(256) pair_kernel(const float4 *src, float *out, int iters,
                                                   float eps2_s, Clock *ck)
{
    clock_begin(ck);
    float4 s[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) s[u] = src[(threadIdx.x + 7 * u) & 255];
    float4 me = src[threadIdx.x & 255];
    float eps2;
    asm volatile("v_mov_b32 %0, %1" : "=v"(eps2) : "s"(eps2_s));
    float ax = 0.0f, ay = 0.0f, az = 0.0f, p = 0.0f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const float dx = s[u].x - me.x, dy = s[u].y - me.y, dz = s[u].z - me.z;
            float q = __builtin_fmaf(dx, dx, eps2);
            q = __builtin_fmaf(dy, dy, q);
            q = __builtin_fmaf(dz, dz, q);
            const float inv = MODE == 0 ? __builtin_amdgcn_rsqf(q) : q * eps2;
            const float mi = s[u].w * inv;
            const float f = mi * (inv * inv);
            ax = __builtin_fmaf(f, dx, ax);
            ay = __builtin_fmaf(f, dy, ay);
            az = __builtin_fmaf(f, dz, az);
            if constexpr (POT) p = __builtin_fmaf(s[u].w, inv, p);
        }
        // move the target a little so nothing above is loop-invariant
        // (3 extra FMAs per 8 interactions)
        me.x = __builtin_fmaf(me.x, eps2, me.y);
        me.y = __builtin_fmaf(me.y, eps2, me.z);
        me.z = __builtin_fmaf(me.z, eps2, me.x);
    }
    out[blockIdx.x * 256 + threadIdx.x] = ax + ay + az + p;
    clock_end(ck);
}

// DPP wave rotation (wave_ror:1: lane l receives lane l-1, lane 0 receives
// lane 63), the cross-lane move a pair-symmetric inner loop would use.
constexpr int kWaveRor1 = 0x13C;

__device__ __forceinline__ float wave_ror1(float v)
{
    // bound_ctrl set: every lane has a source lane under a rotation, so no
    // "old" value is needed
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kWaveRor1, 0xF, 0xF,
                                           true));
}

// Lane-layout check: out[i] = the lane index each lane holds after one rotation.
__global__ void __launch_bounds__(64) ror_layout_kernel(int *out)
{
    const float v = (float)threadIdx.x;
    out[threadIdx.x] = (int)wave_ror1(v);
}

// Throughput of DPP-rotated moves: 8 chains of dependent rotations.
__global__ void __launch_bounds__(256) ror_kernel(float *out, int iters, float a_s, Clock *ck)
{
    clock_begin(ck);
    float x[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) x[c] = 1.0f + 1e-3f * (threadIdx.x + c) + a_s;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
#pragma unroll
            for (int c = 0; c < kChains; ++c) x[c] = wave_ror1(x[c]);
        }
    }
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < kChains; ++c) s += x[c];
    out[blockIdx.x * 256 + threadIdx.x] = s;
    clock_end(ck);
}

struct Result {
    const char *name;
    int k;       // FMAs per chain per step (0 for the rsq-only kernel)
    int rsq;     // v_rsq_f32 per chain per step
    double ms;
    double ghz;                 // measured shader clock
    double waves_override = 0;  // waves in the launch if not 8 per SIMD
};

template <typename F>
Result run(const char *name, int k, int rsq, F launch, Clock *d_ck)
{
    hipEvent_t e0, e1;
    CHECK(hipEventCreate(&e0));
    CHECK(hipEventCreate(&e1));
    launch();  // warm-up
    CHECK(hipDeviceSynchronize());
    CHECK(hipEventRecord(e0, 0));
    launch();
    CHECK(hipEventRecord(e1, 0));
    CHECK(hipEventSynchronize(e1));
    float ms = 0.0f;
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    Clock ck;
    CHECK(hipMemcpy(&ck, d_ck, sizeof ck, hipMemcpyDeviceToHost));
    const double real_s = (double)(ck.r1 - ck.r0) / 100e6;
    const double ghz = real_s > 0 ? (double)(ck.c1 - ck.c0) / real_s / 1e9 : 0.0;
    CHECK(hipEventDestroy(e0));
    CHECK(hipEventDestroy(e1));
    return {name, k, rsq, ms, ghz, 0.0};
}

int main(int argc, char **argv)
{
    int dev = 0;
    CHECK(hipSetDevice(dev));
    hipDeviceProp_t prop;
    CHECK(hipGetDeviceProperties(&prop, dev));
    const int cus = prop.multiProcessorCount;
    const int blocks = cus * 8;  // 8 blocks of 4 waves per CU = 8 waves per SIMD
    const int iters = argc > 1 ? atoi(argv[1]) : 4096;
    float *d_out = nullptr;
    Clock *d_ck = nullptr;
    CHECK(hipMalloc(&d_out, (size_t)blocks * 256 * sizeof(float)));
    CHECK(hipMalloc(&d_ck, sizeof(Clock)));
    const float a = 0.999f;
    std::vector<Result> rs;

#define MIX(NAME, K, R)                                                                     \
    rs.push_back(run(NAME, K, R ? 1 : 0, [&] {                                              \
        hipLaunchKernelGGL((mix_kernel<K, R>), dim3(blocks), dim3(256), 0, 0, d_out, iters, \
                           a, d_ck);                                                       \
    }, d_ck))

    MIX("fma16", 16, false);
    MIX("fma4+rsq", 4, true);
    MIX("fma8+rsq", 8, true);
    MIX("fma12+rsq", 12, true);
    MIX("fma16+rsq", 16, true);
#undef MIX
    rs.push_back(run("rsq", 0, 4, [&] {
        hipLaunchKernelGGL(rsq_kernel, dim3(blocks), dim3(256), 0, 0, d_out, iters, a, d_ck);
    }, d_ck));
#define OP(NAME, O)                                                                         \
    rs.push_back(run(NAME, 16, 0, [&] {                                                     \
        hipLaunchKernelGGL((op_kernel<O>), dim3(blocks), dim3(256), 0, 0, d_out, iters, a,  \
                           d_ck);                                                          \
    }, d_ck))
    OP("fma_vgpr_ops", 0);
    OP("fma_sgpr_ops", 1);
    OP("mul_vgpr", 2);
    OP("sub_vgpr", 3);
    OP("sub_sgpr", 4);
#undef OP
    // one wave per SIMD: same FMA stream, 256 blocks of one wave on 256 CUs x 4 SIMDs
    rs.push_back(run("fma_vgpr_1wave_per_simd", 16, 0, [&] {
        hipLaunchKernelGGL((op_kernel<0>), dim3(cus), dim3(256), 0, 0, d_out, iters, a, d_ck);
    }, d_ck));
    rs.back().waves_override = cus * 4;
#define OV(NAME, K)                                                                         \
    rs.push_back(run(NAME, K + 1, 1, [&] {                                                  \
        hipLaunchKernelGGL((rsq_overlap_kernel<K>), dim3(blocks), dim3(256), 0, 0, d_out,    \
                           iters, a, d_ck);                                                \
    }, d_ck))
    OV("rsq+4fma_interleaved", 4);
    OV("rsq+8fma_interleaved", 8);
    OV("rsq+12fma_interleaved", 12);
#undef OV

    float4 *d_src = nullptr;
    {
        std::vector<float> hs(4 * 256);
        for (int i = 0; i < 4 * 256; ++i) hs[i] = (i % 4 == 3) ? 1e-3f : 0.01f * ((i * 37) % 101 - 50);
        CHECK(hipMalloc(&d_src, hs.size() * sizeof(float)));
        CHECK(hipMemcpy(d_src, hs.data(), hs.size() * sizeof(float), hipMemcpyHostToDevice));
    }
    // pair kernels: k counts VALU per interaction, rsq 1; one "chain" = one interaction
    // (8 per iteration, matching kChains)
#define PAIR(NAME, POT, MODE, K, R)                                                          \
    rs.push_back(run(NAME, K, R, [&] {                                                       \
        hipLaunchKernelGGL((pair_kernel<POT, MODE>), dim3(blocks), dim3(256), 0, 0, d_src,    \
                           d_out, iters, 1e-4f, d_ck);                                       \
    }, d_ck))
    // 3 drift FMAs per 8 interactions are counted as 3/8 of a VALU op each
    PAIR("pair_pot_rsq", true, 0, 13, 1);
    PAIR("pair_nopot_rsq", false, 0, 12, 1);
    PAIR("pair_pot_mul_instead_of_rsq", true, 1, 14, 0);
#undef PAIR
    rs.push_back(run("dpp_wave_ror1_mov", 16, 0, [&] {
        hipLaunchKernelGGL(ror_kernel, dim3(blocks), dim3(256), 0, 0, d_out, iters, a, d_ck);
    }, d_ck));
    {
        int *d_lanes = nullptr;
        int h_lanes[64];
        CHECK(hipMalloc(&d_lanes, sizeof h_lanes));
        hipLaunchKernelGGL(ror_layout_kernel, dim3(1), dim3(64), 0, 0, d_lanes);
        CHECK(hipMemcpy(h_lanes, d_lanes, sizeof h_lanes, hipMemcpyDeviceToHost));
        CHECK(hipFree(d_lanes));
        int ok = 1;
        for (int l = 0; l < 64; ++l) ok &= h_lanes[l] == (l + 63) % 64;
        printf("{\"check\": \"wave_ror1 lane layout (lane l gets lane l-1)\", \"ok\": %s, "
               "\"lane0\": %d, \"lane1\": %d, \"lane63\": %d}\n",
               ok ? "true" : "false", h_lanes[0], h_lanes[1], h_lanes[63]);
    }
    const double waves = (double)blocks * 4, simds = cus * 4.0;
    for (const Result &r : rs) {
        const double s = r.ms / 1e3;
        // SIMD cycles spent per wave per iteration, at the measured clock
        const double wv = r.waves_override > 0 ? r.waves_override : waves;
        const double cyc_iter = s * r.ghz * 1e9 * simds / (wv * iters);
        // split into 4 cycles per wave64 FMA (16-lane SIMD) and the remainder per rsq
        const double fma_cyc = 4.0 * r.k * kChains;
        const double per_rsq = r.rsq ? (cyc_iter - fma_cyc) / (r.rsq * kChains) : 0.0;
        const double lane_ops = (double)(r.k + r.rsq) * kChains * iters * wv * 64.0;
        const double per_instr = cyc_iter / ((r.k + r.rsq) * kChains);
        printf("{\"kernel\": \"%s\", \"ms\": %.3f, \"shader_ghz\": %.3f, "
               "\"lane_ops_per_s\": %.4e, \"simd_cycles_per_wave_iter\": %.2f, "
               "\"cycles_per_wave_instr\": %.3f, \"cycles_per_rsq_if_rest_4\": %.2f}\n",
               r.name, r.ms, r.ghz, lane_ops / s, cyc_iter, per_instr, per_rsq);
    }
    printf("{\"device\": \"%s\", \"cus\": %d, \"blocks\": %d, \"iters\": %d}\n", prop.name, cus,
           blocks, iters);
    CHECK(hipFree(d_src));
    CHECK(hipFree(d_out));
    CHECK(hipFree(d_ck));
    return 0;
}
