// gfx950 (MI355X, CDNA4) kernels for direct all-pairs softened gravity.
//
// Per target i and source j (G = 1, every j including j = i):
//   d = x_j - x_i,  q = |d|^2 + eps2,  inv = q^(-1/2)
//   a_i += m_j inv^3 d,   p_i -= m_j inv
// (Degawa, "N 体問題", slides 4 and 12; Nakasato, "スライド 1", No.4; the pair
// routine of GPU Gems 3 ch. 31 as retold on the CSDN "Cuda Nbody笔记" page,
// whose 20-flop count per pair is the throughput convention.)
//
// Design (wave64, plain FP32 VALU; no MFMA because nothing here is a dense
// contraction):
//   * Each lane keeps T targets in VGPRs (register blocking: T interactions per
//     broadcast source, the idea behind the SoA 4x4 blocking of "スライド 1",
//     No.13-15).
//   * Sources reach all 64 lanes of a wave by one of three broadcasts:
//       LDS      - the workgroup stages WG-body float4 tiles in LDS with
//                  coalesced loads (double-buffered, one barrier per tile), and
//                  each wave reads a source with a uniform-address ds_read_b128;
//       SCALAR   - each wave reads sources with uniform scalar loads, so the
//                  VALU instructions take x_j, y_j, z_j, m_j straight from SGPRs;
//       READLANE - each lane loads one source and v_readlane hands it to SGPRs.
//   * The inner step costs 12 VALU instructions + 1 v_rsq_f32 per interaction
//     (13 + 1 with the potential): 3 sub, 3 FMA for q, rsq, 3 mul for m inv^3,
//     3 FMA into a, 1 FMA into p.
//   * Two-level accumulation: 256 sources go into fresh partial sums, which are
//     then added to the running totals (keeps the fp32 summation error of long
//     sums near the per-term rounding instead of growing with sqrt(N)).
//   * split-j: blockIdx.y selects a chunk of sources; with more than one chunk
//     the partial sums go to scratch and a second kernel adds them in ascending
//     chunk order (the multi-thread-per-row idea for small N of the GPU Gems 3
//     ch. 31 study page, section 4, made deterministic).
//   * Tails: target lanes past N compute on a clamped body and store nothing;
//     LDS/readlane source tails are padded with zero-mass bodies at the origin
//     (they add exact zeros); the scalar path runs its tail source by source.
#include "kernels.h"

namespace nbk {

namespace {

template <int T>
struct Targets {
    float x[T], y[T], z[T];
};

template <int T, bool POT>
struct Sums {
    float ax[T], ay[T], az[T], p[T];
};

template <int T, bool POT>
__device__ __forceinline__ void zero(Sums<T, POT> &s)
{
#pragma unroll
    for (int t = 0; t < T; ++t) {
        s.ax[t] = 0.0f;
        s.ay[t] = 0.0f;
        s.az[t] = 0.0f;
        if constexpr (POT) s.p[t] = 0.0f;
    }
}

template <int T, bool POT>
__device__ __forceinline__ void add_into(Sums<T, POT> &tot, const Sums<T, POT> &blk)
{
#pragma unroll
    for (int t = 0; t < T; ++t) {
        tot.ax[t] += blk.ax[t];
        tot.ay[t] += blk.ay[t];
        tot.az[t] += blk.az[t];
        if constexpr (POT) tot.p[t] += blk.p[t];
    }
}

// One source (sx, sy, sz, sm) against the lane's T targets. The operation
// order is fixed with explicit FMAs so that the acceleration bits do not
// depend on whether the potential is also computed.
template <int T, bool POT>
__device__ __forceinline__ void interact(float sx, float sy, float sz, float sm,
                                         const Targets<T> &tg, float eps2, Sums<T, POT> &acc)
{
#pragma unroll
    for (int t = 0; t < T; ++t) {
        const float dx = sx - tg.x[t];
        const float dy = sy - tg.y[t];
        const float dz = sz - tg.z[t];
        float q = __builtin_fmaf(dx, dx, eps2);
        q = __builtin_fmaf(dy, dy, q);
        q = __builtin_fmaf(dz, dz, q);
        const float inv = __builtin_amdgcn_rsqf(q);  // v_rsq_f32; q >= eps2 > 0 is normal
        const float mi = sm * inv;                   // m_j / sqrt(q)
        const float s = mi * (inv * inv);            // m_j / q^(3/2)
        acc.ax[t] = __builtin_fmaf(s, dx, acc.ax[t]);
        acc.ay[t] = __builtin_fmaf(s, dy, acc.ay[t]);
        acc.az[t] = __builtin_fmaf(s, dz, acc.az[t]);
        if constexpr (POT) acc.p[t] = __builtin_fmaf(sm, inv, acc.p[t]);
    }
}

template <int T, bool POT>
__device__ __forceinline__ void interact4(const float4 &b, const Targets<T> &tg, float eps2,
                                          Sums<T, POT> &acc)
{
    interact<T, POT>(b.x, b.y, b.z, b.w, tg, eps2, acc);
}

// Target t of this lane is body base + t*kWG + threadIdx.x: each t is one
// coalesced 4 KiB segment of the body array.
template <int T, int WG = kWG>
__device__ __forceinline__ Targets<T> load_targets(const float4 *__restrict__ pos, int n,
                                                   unsigned base)
{
    Targets<T> tg;
#pragma unroll
    for (int t = 0; t < T; ++t) {
        unsigned i = base + t * WG + threadIdx.x;
        const float4 b = pos[i < (unsigned)n ? i : (unsigned)(n - 1)];
        tg.x[t] = b.x;
        tg.y[t] = b.y;
        tg.z[t] = b.z;
    }
    return tg;
}

template <int T, bool POT, int WG = kWG>
__device__ __forceinline__ void store(const Sums<T, POT> &a, const AccelArgs &k, unsigned base)
{
#pragma unroll
    for (int t = 0; t < T; ++t) {
        const unsigned i = base + t * WG + threadIdx.x;
        if (i < (unsigned)k.n) {
            if (k.part) {
                const size_t o = (size_t)blockIdx.y * (size_t)k.n + i;
                k.part[o] = make_float4(a.ax[t], a.ay[t], a.az[t], POT ? a.p[t] : 0.0f);
            } else {
                k.acc_out[i] = make_float4(a.ax[t], a.ay[t], a.az[t], 0.0f);
                if constexpr (POT) k.pot_out[i] = -a.p[t];
            }
        }
    }
}

// Body j of the chunk [.., j1), or a zero-mass body at the origin past its end.
// The load index is clamped into the (never empty) chunk and the value is
// selected afterwards, so no out-of-range address is ever formed.
__device__ __forceinline__ float4 load_or_zero(const float4 *__restrict__ pos, int j, int j1)
{
    const bool in = j < j1;
    const float4 b = pos[in ? j : j1 - 1];
    return make_float4(in ? b.x : 0.0f, in ? b.y : 0.0f, in ? b.z : 0.0f, in ? b.w : 0.0f);
}

// A uniform value copied into a VGPR. On gfx950 a VALU instruction whose
// operands are all VGPRs issues about twice as fast as one that reads an SGPR,
// so loop-invariant scalars used in the inner step are kept in VGPRs.
__device__ __forceinline__ float in_vgpr(float s)
{
    float v;
    asm volatile("v_mov_b32 %0, %1" : "=v"(v) : "s"(s));
    return v;
}

// Keeps the compiler's scheduler from moving instructions across this point
// (used to keep prefetch loads ahead of the arithmetic that hides them).
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

__device__ __forceinline__ void chunk_range(const AccelArgs &k, int &j0, int &j1)
{
    const long long a = (long long)blockIdx.y * k.chunk;
    const long long b = a + k.chunk;
    j0 = (int)a;
    j1 = (int)(b < k.n ? b : k.n);
}

// ---------------------------------------------------------------- SCALAR
// Sources are read with uniform addresses, which the compiler turns into
// scalar loads (s_load_dwordx16 = 4 bodies); the VALU instructions read the
// source coordinates from SGPRs. Groups of U bodies are double-buffered so the
// loads of group g+1 are in flight while group g is computed.
template <int T, bool POT>
__global__ void __launch_bounds__(kWG) accel_scalar(AccelArgs k)
{
    constexpr int U = 8;
    constexpr int GPB = kFlush / U;  // groups per accumulation block (even)
    const unsigned base = blockIdx.x * (unsigned)(kWG * T);
    int j0, j1;
    chunk_range(k, j0, j1);
    const Targets<T> tg = load_targets<T>(k.pos, k.n, base);
    const float4 *__restrict__ src = k.pos;
    const float eps2 = k.eps2;

    Sums<T, POT> tot, blk;
    zero(tot);
    zero(blk);

    const int nfull = (j1 - j0) / kFlush;  // full accumulation blocks
    const int ngroups = nfull * GPB;
    if (ngroups > 0) {
        float4 a[U], b[U];
#pragma unroll
        for (int u = 0; u < U; ++u) a[u] = src[j0 + u];
        for (int g = 0; g < ngroups; g += 2) {
            const int jg = j0 + g * U;
#pragma unroll
            for (int u = 0; u < U; ++u) b[u] = src[jg + U + u];
            sched_fence();
#pragma unroll
            for (int u = 0; u < U; ++u) interact4<T, POT>(a[u], tg, eps2, blk);
            sched_fence();
            // next group pair; on the last pass reload the current one (in range, unused)
            const int jn = (g + 2 < ngroups) ? jg + 2 * U : jg;
#pragma unroll
            for (int u = 0; u < U; ++u) a[u] = src[jn + u];
            sched_fence();
#pragma unroll
            for (int u = 0; u < U; ++u) interact4<T, POT>(b[u], tg, eps2, blk);
            sched_fence();
            if ((g + 2) % GPB == 0) {
                add_into(tot, blk);
                zero(blk);
            }
        }
    }
    // tail: fewer than kFlush sources
    int j = j0 + ngroups * U;
    for (; j + U <= j1; j += U) {
        float4 a[U];
#pragma unroll
        for (int u = 0; u < U; ++u) a[u] = src[j + u];
#pragma unroll
        for (int u = 0; u < U; ++u) interact4<T, POT>(a[u], tg, eps2, blk);
    }
    for (; j < j1; ++j) interact4<T, POT>(src[j], tg, eps2, blk);
    add_into(tot, blk);
    store(tot, k, base);
}

// ---------------------------------------------------------------- LDS
// The workgroup stages WG bodies per tile in LDS (each thread loads one
// float4, coalesced). Two tile buffers: while tile t is read from one, the
// prefetched tile t+1 is written to the other, so one barrier per tile both
// publishes the new tile and guards the buffer about to be overwritten. The
// prefetch is issued at the top of the tile and only consumed (zero-padded and
// stored) at its end, so its latency hides behind the tile's arithmetic. Each
// wave reads sources with uniform-address ds_read_b128 (a broadcast) into
// VGPRs, in groups of U that are double-buffered across scheduling fences.
template <int T, bool POT, int WG>
__global__ void __launch_bounds__(WG) accel_lds(AccelArgs k)
{
    static_assert(WG % kFlush == 0, "accumulation blocks must tile the LDS tile");
    constexpr int U = T <= 2 ? 4 : 2;
    __shared__ float4 tile[2][WG];
    const unsigned base = blockIdx.x * (unsigned)(WG * T);
    int j0, j1;
    chunk_range(k, j0, j1);
    const Targets<T> tg = load_targets<T, WG>(k.pos, k.n, base);
    const float eps2 = in_vgpr(k.eps2);

    Sums<T, POT> tot, blk;
    zero(tot);
    zero(blk);

    const int ntiles = (j1 - j0 + WG - 1) / WG;
    int jl = j0 + threadIdx.x;
    tile[0][threadIdx.x] = load_or_zero(k.pos, jl, j1);
    __syncthreads();
    for (int it = 0; it < ntiles; ++it) {
        const int cur = it & 1;
        const bool more = it + 1 < ntiles;
        jl += WG;
        // raw prefetch of the next tile (index clamped into the chunk); the
        // zero-padding select happens at the store below
        float4 r = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        if (more) r = k.pos[jl < j1 ? jl : j1 - 1];
        const float4 *tl = tile[cur];
        float4 a[U], b[U];
#pragma unroll
        for (int u = 0; u < U; ++u) a[u] = tl[u];
        for (int u0 = 0; u0 < WG; u0 += 2 * U) {
#pragma unroll
            for (int u = 0; u < U; ++u) b[u] = tl[u0 + U + u];
            sched_fence();
#pragma unroll
            for (int u = 0; u < U; ++u) interact4<T, POT>(a[u], tg, eps2, blk);
            sched_fence();
            const int un = (u0 + 2 * U < WG) ? u0 + 2 * U : 0;
#pragma unroll
            for (int u = 0; u < U; ++u) a[u] = tl[un + u];
            sched_fence();
#pragma unroll
            for (int u = 0; u < U; ++u) interact4<T, POT>(b[u], tg, eps2, blk);
            sched_fence();
            if (((u0 + 2 * U) % kFlush) == 0) {
                add_into(tot, blk);
                zero(blk);
            }
        }
        if (more) {
            const bool in = jl < j1;
            tile[cur ^ 1][threadIdx.x] = make_float4(in ? r.x : 0.0f, in ? r.y : 0.0f,
                                                     in ? r.z : 0.0f, in ? r.w : 0.0f);
        }
        __syncthreads();
    }
    store<T, POT, WG>(tot, k, base);
}

// ---------------------------------------------------------------- READLANE
// Each lane loads one body of a 64-body group (coalesced; zero-mass padding
// past the chunk end) and v_readlane broadcasts body u to SGPRs. The next
// group's load is issued before the current group is consumed.
template <int T, bool POT>
__global__ void __launch_bounds__(kWG) accel_readlane(AccelArgs k)
{
    constexpr int U = 16;
    const unsigned base = blockIdx.x * (unsigned)(kWG * T);
    int j0, j1;
    chunk_range(k, j0, j1);
    const Targets<T> tg = load_targets<T>(k.pos, k.n, base);
    const float eps2 = k.eps2;
    const int lane = threadIdx.x & 63;

    Sums<T, POT> tot, blk;
    zero(tot);
    zero(blk);

    int jl = j0 + lane;
    float4 mine = load_or_zero(k.pos, jl, j1);
    for (int jb = j0; jb < j1; jb += 64) {
        jl += 64;
        const float4 nxt = load_or_zero(k.pos, jl, j1);
        const int mx = __builtin_bit_cast(int, mine.x), my = __builtin_bit_cast(int, mine.y);
        const int mz = __builtin_bit_cast(int, mine.z), mm = __builtin_bit_cast(int, mine.w);
        for (int u0 = 0; u0 < 64; u0 += U) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const float sx = __builtin_bit_cast(float, __builtin_amdgcn_readlane(mx, u0 + u));
                const float sy = __builtin_bit_cast(float, __builtin_amdgcn_readlane(my, u0 + u));
                const float sz = __builtin_bit_cast(float, __builtin_amdgcn_readlane(mz, u0 + u));
                const float sm = __builtin_bit_cast(float, __builtin_amdgcn_readlane(mm, u0 + u));
                interact<T, POT>(sx, sy, sz, sm, tg, eps2, blk);
            }
        }
        if (((jb - j0 + 64) % kFlush) == 0) {
            add_into(tot, blk);
            zero(blk);
        }
        mine = nxt;
    }
    add_into(tot, blk);
    store(tot, k, base);
}

// ---------------------------------------------------------------- combine / Euler
// Partial sums are added in ascending chunk order s = 0, 1, ..., S-1.
__device__ __forceinline__ float4 sum_parts(const float4 *__restrict__ part, int n, int splits,
                                            unsigned i)
{
    float4 a = part[i];
    for (int s = 1; s < splits; ++s) {
        const float4 b = part[(size_t)s * (size_t)n + i];
        a.x += b.x;
        a.y += b.y;
        a.z += b.z;
        a.w += b.w;
    }
    return a;
}

__global__ void __launch_bounds__(256) combine_kernel(const float4 *__restrict__ part, int n,
                                                      int splits, float4 *__restrict__ acc_out,
                                                      float *__restrict__ pot_out)
{
    const unsigned i = blockIdx.x * 256u + threadIdx.x;
    if (i >= (unsigned)n) return;
    const float4 a = sum_parts(part, n, splits, i);
    acc_out[i] = make_float4(a.x, a.y, a.z, 0.0f);
    if (pot_out) pot_out[i] = -a.w;
}

// Explicit Euler, position first with the old velocity (Degawa, "N 体問題",
// slides 5-6 and 15): x += dt v; v += dt a(x^n). Each update is one FMA; the
// mass (pos.w) and vel.w are carried through unchanged.
__global__ void __launch_bounds__(256) euler_kernel(const float4 *__restrict__ part, int n,
                                                    int splits, float4 *__restrict__ pos,
                                                    float4 *__restrict__ vel, float dt)
{
    const unsigned i = blockIdx.x * 256u + threadIdx.x;
    if (i >= (unsigned)n) return;
    const float4 a = sum_parts(part, n, splits, i);
    float4 x = pos[i];
    float4 v = vel[i];
    x.x = __builtin_fmaf(dt, v.x, x.x);
    x.y = __builtin_fmaf(dt, v.y, x.y);
    x.z = __builtin_fmaf(dt, v.z, x.z);
    v.x = __builtin_fmaf(dt, a.x, v.x);
    v.y = __builtin_fmaf(dt, a.y, v.y);
    v.z = __builtin_fmaf(dt, a.z, v.z);
    pos[i] = x;
    vel[i] = v;
}

template <int T, bool POT>
const void *accel_fn(int bcast, int wg)
{
    if (bcast == 1 && wg == 256) return (const void *)&accel_lds<T, POT, 256>;
    if (bcast == 1 && wg == 512) return (const void *)&accel_lds<T, POT, 512>;
    if (wg != kWG) return nullptr;
    if (bcast == 2) return (const void *)&accel_scalar<T, POT>;
    if (bcast == 3) return (const void *)&accel_readlane<T, POT>;
    return nullptr;
}

template <bool POT>
const void *accel_fn_t(int bcast, int tpl, int wg)
{
    switch (tpl) {
    case 1: return accel_fn<1, POT>(bcast, wg);
    case 2: return accel_fn<2, POT>(bcast, wg);
    case 4: return accel_fn<4, POT>(bcast, wg);
    case 8: return accel_fn<8, POT>(bcast, wg);
    default: return nullptr;
    }
}

}  // namespace

hipError_t launch_accel(int bcast, int tpl, int wg, bool pot, unsigned grid_x, unsigned splits,
                        const AccelArgs &args, hipStream_t stream)
{
    const void *fn = pot ? accel_fn_t<true>(bcast, tpl, wg) : accel_fn_t<false>(bcast, tpl, wg);
    if (!fn) return hipErrorInvalidValue;
    AccelArgs a = args;
    void *kargs[] = {&a};
    return hipLaunchKernel(fn, dim3(grid_x, splits, 1), dim3(wg, 1, 1), kargs, 0, stream);
}

hipError_t launch_combine(const float4 *part, int n, int splits, float4 *acc_out, float *pot_out,
                          hipStream_t stream)
{
    void *kargs[] = {&part, &n, &splits, &acc_out, &pot_out};
    const unsigned g = (unsigned)((n + 255) / 256);
    return hipLaunchKernel((const void *)&combine_kernel, dim3(g), dim3(256), kargs, 0, stream);
}

hipError_t launch_euler(const float4 *part, int n, int splits, float4 *pos, float4 *vel, float dt,
                        hipStream_t stream)
{
    void *kargs[] = {&part, &n, &splits, &pos, &vel, &dt};
    const unsigned g = (unsigned)((n + 255) / 256);
    return hipLaunchKernel((const void *)&euler_kernel, dim3(g), dim3(256), kargs, 0, stream);
}

}  // namespace nbk
