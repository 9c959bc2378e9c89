// Host-side driver for the sanitizer test: every C ABI entry point called with
// arguments that its checks reject before any HIP call (so no GPU is needed).
// Built with AddressSanitizer and UndefinedBehaviorSanitizer on the host code
// only; exits non-zero if a call returns anything but the expected code or
// leaves no error text.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "nbody.h"

static int failures = 0;

static void expect(const char *what, int rc, int want)
{
    const char *msg = nbody_last_error();
    if (rc != want || (want != NBODY_OK && (!msg || !*msg))) {
        std::printf("FAIL %s: rc=%d want=%d msg=%s\n", what, rc, want, msg ? msg : "(null)");
        ++failures;
    }
}

int main()
{
    // fake, aligned device addresses: never dereferenced (the checks fail first)
    nbody_f4 *A = (nbody_f4 *)(uintptr_t)(1u << 20);
    nbody_f4 *B = (nbody_f4 *)(uintptr_t)(1u << 28);
    float *C = (float *)(uintptr_t)(1u << 29);
    const float nan = std::nanf("");

    expect("accel N<0", nbody_accel(A, -1, 1e-4f, B, nullptr, nullptr), NBODY_EINVAL);
    expect("accel N>2^30", nbody_accel(A, (int64_t(1) << 30) + 1, 1e-4f, B, nullptr, nullptr),
           NBODY_EINVAL);
    expect("accel pos NULL", nbody_accel(nullptr, 16, 1e-4f, B, nullptr, nullptr), NBODY_EINVAL);
    expect("accel eps2 NaN", nbody_accel(A, 16, nan, B, nullptr, nullptr), NBODY_EINVAL);
    expect("accel eps2 0", nbody_accel(A, 16, 0.0f, B, nullptr, nullptr), NBODY_EINVAL);
    expect("accel misaligned", nbody_accel((nbody_f4 *)((char *)A + 4), 16, 1e-4f, B, nullptr,
                                           nullptr), NBODY_EALIGN);
    expect("accel overlap", nbody_accel(A, 16, 1e-4f, A + 1, nullptr, nullptr), NBODY_EINVAL);
    expect("accel N=0", nbody_accel(nullptr, 0, 1e-4f, nullptr, nullptr, nullptr), NBODY_OK);

    nbody_plan bad = {7, 0, 0, 0, 0, 0, 0};
    expect("plan bcast", nbody_accel_plan(A, 16, 1e-4f, B, nullptr, &bad, nullptr), NBODY_EINVAL);
    nbody_plan bad2 = {0, 8, 0, 0, 0, NBODY_MODE_PAIRS, 256};
    expect("plan band 256 tpl 8", nbody_accel_plan(A, 16, 1e-4f, B, nullptr, &bad2, nullptr),
           NBODY_EINVAL);

    expect("step nsteps<0", nbody_step(A, B, 16, 1e-3f, 1e-4f, -1, nullptr), NBODY_EINVAL);
    expect("step dt inf", nbody_step(A, B, 16, INFINITY, 1e-4f, 1, nullptr), NBODY_EINVAL);
    expect("step overlap", nbody_step(A, A, 16, 1e-3f, 1e-4f, 1, nullptr), NBODY_EINVAL);
    expect("step plan", nbody_step_plan(A, B, 16, 1e-3f, 1e-4f, 1, &bad, nullptr), NBODY_EINVAL);
    expect("step noalloc overlap", nbody_step_noalloc(A, A, 16, 1e-3f, 1e-4f, 1, nullptr),
           NBODY_EINVAL);
    expect("step noalloc eps2", nbody_step_noalloc(A, B, 16, 1e-3f, 0x1p-85f, 1, nullptr),
           NBODY_EINVAL);
    expect("step noalloc nsteps 0", nbody_step_noalloc(A, B, 16, 1e-3f, 1e-4f, 0, nullptr),
           NBODY_OK);
    expect("time_kernel one event", nbody_time_kernel((hipEvent_t)A, nullptr), NBODY_EINVAL);
    expect("time_kernel off", nbody_time_kernel(nullptr, nullptr), NBODY_OK);

    float *f = (float *)A;
    expect("soa x NULL", nbody_accel_soa(nullptr, f, f, f, 16, 1e-4f, C, C + 64, C + 128, nullptr,
                                         nullptr), NBODY_EINVAL);
    expect("soa step overlap", nbody_step_soa(f, f, f, f, f, f, f, 16, 1e-3f, 1e-4f, 1, nullptr),
           NBODY_EINVAL);

    expect("shard nshards 0", nbody_accel_shard(A, 16, 1e-4f, 0, 0, 1, nullptr, B, nullptr),
           NBODY_EINVAL);
    expect("shard index", nbody_accel_shard(A, 16, 1e-4f, 3, 3, 1, nullptr, B, nullptr),
           NBODY_EINVAL);
    expect("finish range", nbody_shard_finish(A, 16, 2, 9, 8, B, nullptr, nullptr), NBODY_EINVAL);

    int32_t *I = (int32_t *)C;
    expect("p2p ncell<0", nbody_p2p(A, 16, 1e-4f, I, -1, I, I, 4, B, nullptr, nullptr),
           NBODY_EINVAL);
    const float lo[3] = {0.0f, 0.0f, 0.0f};
    const int32_t dims0[3] = {0, 4, 4};
    expect("grid dims", nbody_near_grid(A, 16, 1e-4f, lo, 0.5f, dims0, B, nullptr, nullptr),
           NBODY_EINVAL);
    expect("tree leaf_size 0", nbody_near_tree(A, 16, 1e-4f, 0, B, nullptr, nullptr, nullptr),
           NBODY_EINVAL);
    nbody_tree_stats st = {7, 7, 7};
    expect("tree N=0", nbody_near_tree(nullptr, 0, 1e-4f, 1, nullptr, nullptr, &st, nullptr),
           NBODY_OK);
    if (st.leaves != 0 || st.list_entries != 0 || st.pair_terms != 0) {
        std::printf("FAIL tree N=0 stats not cleared\n");
        ++failures;
    }
    expect("diag N<0", nbody_diagnostics(A, B, nullptr, -1, 1e-4f, nullptr, nullptr),
           NBODY_EINVAL);
    expect("plan_for NULL", nbody_plan_for(16, 0, nullptr), NBODY_EINVAL);

    const char *v = nbody_version();
    if (!v || !std::strstr(v, "gfx950")) {
        std::printf("FAIL version\n");
        ++failures;
    }
    std::printf("%s: %d failures\n", failures ? "FAILED" : "ok", failures);
    return failures ? 1 : 0;
}
