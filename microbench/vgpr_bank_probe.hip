// Issue cost of VALU instructions by the VGPR banks of their source operands on
// gfx950 (MI355X). A VGPR's bank is its register number mod 4. Each kernel runs
// one inline-asm loop of 64 FMAs on fixed registers (v32..v71, initialised to
// 0.5 inside the same asm statement) into 8 independent accumulators, so the
// only difference between kernels is which banks the operands come from. The
// kernels touch no memory but out[block * 256 + thread] and clk[0..1].
//
//   hipcc --offload-arch=gfx950 -O3 -Xclang -target-feature -Xclang -packed-fp32-ops \
//         microbench/vgpr_bank_probe.hip -o _build/vgpr_bank_probe
//   ./_build/vgpr_bank_probe [iterations]
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>

#define CHECK(x)                                                                   \
    do {                                                                           \
        hipError_t e_ = (x);                                                       \
        if (e_ != hipSuccess) {                                                    \
            std::fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));           \
            std::exit(1);                                                          \
        }                                                                          \
    } while (0)

// v_fmac_f32 acc, a, b into the 8 accumulators v40, v44, ..., v68 (all bank 0;
// fmac reads its destination as the addend).
#define FMAC8(a, b)                                                                \
    "v_fmac_f32 v40, " a ", " b "\n"                                               \
    "v_fmac_f32 v44, " a ", " b "\n"                                               \
    "v_fmac_f32 v48, " a ", " b "\n"                                               \
    "v_fmac_f32 v52, " a ", " b "\n"                                               \
    "v_fmac_f32 v56, " a ", " b "\n"                                               \
    "v_fmac_f32 v60, " a ", " b "\n"                                               \
    "v_fmac_f32 v64, " a ", " b "\n"                                               \
    "v_fmac_f32 v68, " a ", " b "\n"
// v_fma_f32 dst, a, b, c into the same 8 destinations (three separate sources).
#define FMA8(a, b, c)                                                              \
    "v_fma_f32 v40, " a ", " b ", " c "\n"                                         \
    "v_fma_f32 v44, " a ", " b ", " c "\n"                                         \
    "v_fma_f32 v48, " a ", " b ", " c "\n"                                         \
    "v_fma_f32 v52, " a ", " b ", " c "\n"                                         \
    "v_fma_f32 v56, " a ", " b ", " c "\n"                                         \
    "v_fma_f32 v60, " a ", " b ", " c "\n"                                         \
    "v_fma_f32 v64, " a ", " b ", " c "\n"                                         \
    "v_fma_f32 v68, " a ", " b ", " c "\n"
#define X8(s) s s s s s s s s  // 64 instructions per loop trip

#define INIT4(r) "v_mov_b32 v" #r ", 0.5\n"
#define INIT_ALL                                                                   \
    INIT4(32) INIT4(33) INIT4(34) INIT4(35) INIT4(36) INIT4(37) INIT4(40)         \
    INIT4(41) INIT4(44) INIT4(48) INIT4(52) INIT4(56) INIT4(60) INIT4(64) INIT4(68)

#define CLOBBERS                                                                   \
    "v32", "v33", "v34", "v35", "v36", "v37", "v40", "v41", "v44", "v48", "v52",  \
        "v56", "v60", "v64", "v68", "s40", "scc"

#define PROBE(name, body)                                                          \
    __global__ void __launch_bounds__(256) name(float *out, int iters,             \
                                                unsigned long long *clk)           \
    {                                                                              \
        unsigned long long t0 = 0, r0 = 0;                                         \
        const bool timer = blockIdx.x == 0 && threadIdx.x == 0;                    \
        if (timer) {                                                               \
            t0 = __builtin_amdgcn_s_memtime();                                     \
            r0 = __builtin_amdgcn_s_memrealtime();                                 \
        }                                                                          \
        float res;                                                                 \
        asm volatile(INIT_ALL "s_mov_b32 s40, %1\n"                                \
                              "1:\n" body "s_sub_u32 s40, s40, 1\n"                \
                              "s_cmp_lg_u32 s40, 0\n"                              \
                              "s_cbranch_scc1 1b\n"                                \
                              "v_add_f32 %0, v40, v44\n"                           \
                     : "=v"(res)                                                   \
                     : "s"(iters)                                                  \
                     : CLOBBERS);                                                  \
        out[blockIdx.x * 256 + threadIdx.x] = res;                                 \
        if (timer) {                                                               \
            clk[0] = __builtin_amdgcn_s_memtime() - t0;                            \
            clk[1] = __builtin_amdgcn_s_memrealtime() - r0;                        \
        }                                                                          \
    }

// fmac: sources are the accumulator (bank 0) and a, b
PROBE(k_banks_0_1_2, X8(FMAC8("v33", "v34")))  // three banks
PROBE(k_banks_0_1_0, X8(FMAC8("v33", "v36")))  // two in bank 0
PROBE(k_banks_0_1_1, X8(FMAC8("v33", "v37")))  // two in bank 1
PROBE(k_banks_0_0_0, X8(FMAC8("v32", "v36")))  // three in bank 0
// fma: three sources, destination not read
PROBE(k_fma_banks_1_2_3, X8(FMA8("v33", "v34", "v35")))
PROBE(k_fma_banks_1_1_1, X8(FMA8("v33", "v37", "v41")))

int main(int argc, char **argv)
{
    const int grid = 2048;  // 8 waves per SIMD requested on 256 CUs
    const int iters = argc > 1 ? std::atoi(argv[1]) : 2048;
    if (iters < 1) return 1;
    float *out;
    unsigned long long *clk;
    CHECK(hipMalloc(&out, grid * 256 * sizeof(float)));
    CHECK(hipMalloc(&clk, 2 * sizeof(unsigned long long)));
    hipEvent_t a, b;
    CHECK(hipEventCreate(&a));
    CHECK(hipEventCreate(&b));
    struct K {
        const char *name;
        void (*fn)(float *, int, unsigned long long *);
    } ks[] = {{"fmac acc b0, src b1 b2", k_banks_0_1_2},  {"fmac acc b0, src b1 b0", k_banks_0_1_0},
              {"fmac acc b0, src b1 b1", k_banks_0_1_1},  {"fmac acc b0, src b0 b0", k_banks_0_0_0},
              {"fma src b1 b2 b3", k_fma_banks_1_2_3},    {"fma src b1 b1 b1", k_fma_banks_1_1_1}};
    std::printf("| operands | ms | shader GHz | cycles / wave instr |\n|---|---|---|---|\n");
    for (const K &k : ks) {
        float ms = 0.0f;
        unsigned long long c[2] = {0, 0};
        for (int rep = 0; rep < 3; ++rep) {  // the last of three runs is reported
            CHECK(hipEventRecord(a));
            k.fn<<<grid, 256>>>(out, iters, clk);
            CHECK(hipGetLastError());
            CHECK(hipEventRecord(b));
            CHECK(hipEventSynchronize(b));
            CHECK(hipEventElapsedTime(&ms, a, b));
            CHECK(hipMemcpy(c, clk, sizeof(c), hipMemcpyDeviceToHost));
        }
        // s_memrealtime ticks at 100 MHz
        const double ghz = c[1] ? 0.1 * (double)c[0] / (double)c[1] : 0.0;
        const double per_simd = (double)grid * 4 * iters * 64 / (256.0 * 4);
        std::printf("| %s | %.3f | %.3f | %.3f |\n", k.name, ms, ghz,
                    ms * 1e-3 * ghz * 1e9 / per_simd);
    }
    CHECK(hipDeviceSynchronize());
    return 0;
}
