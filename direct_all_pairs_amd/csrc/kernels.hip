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
//   * Two-level accumulation: up to 256 sources (in pair mode, one band-pair
//     item) go into fresh partial sums, which are then added to compensated
//     running totals (TwoSum with a separate error sum), so the fp32 summation
//     error stays near the per-term rounding for any N.
//   * split-j: blockIdx.y selects a chunk of sources; with more than one chunk
//     the partial sums go to scratch and a second kernel adds them in ascending
//     chunk order (the multi-thread-per-row idea for small N of the GPU Gems 3
//     ch. 31 study page, section 4, made deterministic).
//   * Tails: target lanes past N compute on a clamped body and store nothing;
//     LDS/readlane source tails are padded with zero-mass bodies at the origin
//     (they add exact zeros); the scalar path runs its tail source by source.
// Sections below: the one-sided tile kernels (SCALAR, LDS, READLANE), the
// small-N kernel (SMALL: one kernel per evaluation or step), the
// pair-symmetric kernel (PAIRS: each unordered pair once, applied to both
// bodies), the ordered combine / Euler kernels, the shards of a split
// evaluation, diagnostics, the near field over cell lists and layout
// conversion.
#include "kernels.h"

#include <climits>
#include <cmath>
#include <cstdint>

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

// Running totals of the block sums, compensated: each addition is an exact
// TwoSum (Knuth: the rounded sum plus its exact rounding error), the errors go
// into a second sum e, and the total is s + e. The error of the totals then
// stays at the level of one block sum however many blocks a chunk holds (plain
// fp32 totals grow with the block count: measured err/B 1.6e-7 at N = 2^20 and
// 6.3e-7 at 2^22 with one chunk per 2^20 sources). Adding an exact zero leaves
// (s, e) unchanged, so zero-mass padding stays bit-neutral.
template <int T, bool POT>
struct Total {
    Sums<T, POT> s, e;
};

template <int T, bool POT>
__device__ __forceinline__ void zero(Total<T, POT> &tot)
{
    zero(tot.s);
    zero(tot.e);
}

__device__ __forceinline__ void two_sum_add(float &s, float &e, float x)
{
    const float t = s + x;
    const float xv = t - s;                  // the part of x that reached t
    const float err = (s - (t - xv)) + (x - xv);
    s = t;
    e += err;
}

template <int T, bool POT>
__device__ __forceinline__ void add_into(Total<T, POT> &tot, const Sums<T, POT> &blk)
{
#pragma unroll
    for (int t = 0; t < T; ++t) {
        two_sum_add(tot.s.ax[t], tot.e.ax[t], blk.ax[t]);
        two_sum_add(tot.s.ay[t], tot.e.ay[t], blk.ay[t]);
        two_sum_add(tot.s.az[t], tot.e.az[t], blk.az[t]);
        if constexpr (POT) two_sum_add(tot.s.p[t], tot.e.p[t], blk.p[t]);
    }
}

// s + e of a compensated total.
template <int T, bool POT>
__device__ __forceinline__ Sums<T, POT> result(const Total<T, POT> &tot)
{
    Sums<T, POT> r;
#pragma unroll
    for (int t = 0; t < T; ++t) {
        r.ax[t] = tot.s.ax[t] + tot.e.ax[t];
        r.ay[t] = tot.s.ay[t] + tot.e.ay[t];
        r.az[t] = tot.s.az[t] + tot.e.az[t];
        r.p[t] = POT ? tot.s.p[t] + tot.e.p[t] : 0.0f;
    }
    return r;
}

// One source (sx, sy, sz, sm) against the lane's T targets. The operation
// order is fixed with explicit FMAs so that the acceleration bits do not
// depend on whether the potential is also computed.
// FENCE: a scheduling fence after each term keeps every source's chain whole
// (the LDS tile kernel at one target per lane: 319.9 -> 314.6 ms at N = 2^20,
// the same bits).
template <int T, bool POT, bool FENCE = false>
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
        if constexpr (FENCE) __builtin_amdgcn_sched_barrier(0);
    }
}

template <int T, bool POT, bool FENCE = false>
__device__ __forceinline__ void interact4(const float4 &b, const Targets<T> &tg, float eps2,
                                          Sums<T, POT> &acc)
{
    interact<T, POT, FENCE>(b.x, b.y, b.z, b.w, tg, eps2, acc);
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

// Race probe, compiled in only for the test build of the library
// (-DNBK_RACE_PROBE): as soon as a barrier hands an LDS slot back for reuse,
// the thread that will refill it writes NaN there, so a reader that a missing
// or misplaced barrier left behind reads NaN (or the next data) and the
// outputs show it. Correct barriers leave every result bit unchanged.
#ifdef NBK_RACE_PROBE
constexpr bool kRaceProbe = true;
#else
constexpr bool kRaceProbe = false;
#endif

__device__ __forceinline__ void probe_poison(float4 &slot)
{
    if constexpr (kRaceProbe) {
        const float q = __builtin_nanf("");
        slot = make_float4(q, q, q, q);
        asm volatile("" ::: "memory");  // the store must stay although a refill follows
    }
}

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

    Total<T, POT> tot;
    Sums<T, POT> blk;
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
    store(result(tot), k, base);
}

// Partial sums are added in ascending chunk order s = 0, 1, ..., S-1, each
// addition a TwoSum whose error goes into a second sum (hundreds of slots in
// pair mode), loading eight slots ahead of the in-order additions.
__device__ __forceinline__ void two_sum_add4(float4 &a, float4 &e, const float4 &b)
{
    two_sum_add(a.x, e.x, b.x);
    two_sum_add(a.y, e.y, b.y);
    two_sum_add(a.z, e.z, b.z);
    two_sum_add(a.w, e.w, b.w);
}

__device__ __forceinline__ float4 sum_parts(const float4 *part, int n, int splits, unsigned i)
{
    float4 a = part[i];
    float4 e = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    int s = 1;
    for (; s + 8 <= splits; s += 8) {
        float4 b[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) b[u] = part[(size_t)(s + u) * (size_t)n + i];
#pragma unroll
        for (int u = 0; u < 8; ++u) two_sum_add4(a, e, b[u]);
    }
    for (; s < splits; ++s) two_sum_add4(a, e, part[(size_t)s * (size_t)n + i]);
    return make_float4(a.x + e.x, a.y + e.y, a.z + e.z, a.w + e.w);
}

// Explicit Euler, position first with the old velocity (Degawa, "N 体問題",
// slides 5-6 and 15): x' = x + dt v; v' = v + dt a(x). Each update is one FMA;
// the mass (x.w) and v.w are carried through unchanged.
__device__ __forceinline__ void euler_update(float4 &x, float4 &v, const float4 &a, float dt)
{
    x.x = __builtin_fmaf(dt, v.x, x.x);
    x.y = __builtin_fmaf(dt, v.y, x.y);
    x.z = __builtin_fmaf(dt, v.z, x.z);
    v.x = __builtin_fmaf(dt, a.x, v.x);
    v.y = __builtin_fmaf(dt, a.y, v.y);
    v.z = __builtin_fmaf(dt, a.z, v.z);
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
    // accumulation block: kFlush sources, or the whole tile when it is smaller
    constexpr int FL = WG < kFlush ? WG : kFlush;
    static_assert(WG % FL == 0, "accumulation blocks must tile the LDS tile");
    constexpr int U = T <= 2 ? 4 : 2;
    __shared__ float4 tile[2][WG];
    const unsigned base = blockIdx.x * (unsigned)(WG * T);
    int j0, j1;
    chunk_range(k, j0, j1);
    const Targets<T> tg = load_targets<T, WG>(k.pos, k.n, base);
    const float eps2 = in_vgpr(k.eps2);

    Total<T, POT> tot;
    Sums<T, POT> blk;
    zero(tot);
    zero(blk);

    const int ntiles = (j1 - j0 + WG - 1) / WG;
    int jl = j0 + threadIdx.x;
    tile[0][threadIdx.x] = load_or_zero(k.pos, jl, j1);
    __syncthreads();
    for (int it = 0; it < ntiles; ++it) {
        const int cur = it & 1;
        const bool more = it + 1 < ntiles;
        if (more) probe_poison(tile[cur ^ 1][threadIdx.x]);
        jl += WG;
        // raw prefetch of the next tile (index clamped into the chunk); the
        // zero-padding select happens at the store below
        float4 r = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        if (more) r = k.pos[jl < j1 ? jl : j1 - 1];
        const float4 *tl = tile[cur];
        float4 a[U], b[U];
#pragma unroll
        for (int u = 0; u < U; ++u) a[u] = tl[u];
#pragma unroll 1
        for (int u0 = 0; u0 < WG; u0 += 2 * U) {
#pragma unroll
            for (int u = 0; u < U; ++u) b[u] = tl[u0 + U + u];
            sched_fence();
#pragma unroll
            for (int u = 0; u < U; ++u) interact4<T, POT, T == 1>(a[u], tg, eps2, blk);
            sched_fence();
            const int un = (u0 + 2 * U < WG) ? u0 + 2 * U : 0;
#pragma unroll
            for (int u = 0; u < U; ++u) a[u] = tl[un + u];
            sched_fence();
#pragma unroll
            for (int u = 0; u < U; ++u) interact4<T, POT, T == 1>(b[u], tg, eps2, blk);
            sched_fence();
            if (((u0 + 2 * U) % FL) == 0) {
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
    store<T, POT, WG>(result(tot), k, base);
}

// ---------------------------------------------------------------- SMALL
// Small N: each 256-thread workgroup owns TW targets and sums over every
// source, so an evaluation (or an Euler step) is one kernel with no partial
// sums in memory. Thread (t, g) = (tid mod TW, tid / TW) takes target t and
// the sources g, g + G, g + 2G, ... (G = 256 / TW groups) of every LDS tile.
// Tiles of 1024 bodies are double-buffered (the next one is loaded into
// registers while the current one is evaluated; one barrier per tile). Lanes
// of one group read the same LDS address (a broadcast) and a wave's groups are
// consecutive bodies, so the reads are conflict-free.
// The G group sums of a target are added in two fixed stages: inside each
// wave by an xor butterfly over its 64 / TW groups (every lane of a target
// ends with the same bits), then the four wave sums in ascending wave order
// (23 % faster than adding the G group sums through LDS at TW = 4, N = 1024).
template <int TW, bool POT, bool STEP>
__global__ void __launch_bounds__(256) accel_small(SmallArgs k)
{
    constexpr int WG = 256;
    constexpr int G = WG / TW;     // source groups
    constexpr int TS = 1024;       // bodies per tile
    constexpr int L = TS / WG;     // tile loads per thread
    constexpr int PER = TS / G;    // sources per thread per tile
    constexpr int NW = WG / 64;    // waves
    static_assert(TW <= 32 && TS % WG == 0 && TS % G == 0, "small-kernel shape");
    __shared__ float4 tile[2][TS];
    __shared__ float4 red[NW][TW];
    const int t = threadIdx.x % TW, g = threadIdx.x / TW;
    const int i = blockIdx.x * TW + t;
    const float4 me = k.pos[i < k.n ? i : k.n - 1];
    Targets<1> tg;
    tg.x[0] = me.x;
    tg.y[0] = me.y;
    tg.z[0] = me.z;
    const float eps2 = in_vgpr(k.eps2);
    Total<1, POT> tot;
    Sums<1, POT> blk;
    zero(tot);

    const int ntiles = (k.n + TS - 1) / TS;
#pragma unroll
    for (int l = 0; l < L; ++l) tile[0][l * WG + threadIdx.x] = load_or_zero(k.pos, l * WG + threadIdx.x, k.n);
    __syncthreads();
    for (int it = 0; it < ntiles; ++it) {
        const bool more = it + 1 < ntiles;
        const int nb = (it + 1) * TS + threadIdx.x;  // this thread's first body of the next tile
        if (kRaceProbe && more) {
            for (int l = 0; l < L; ++l) probe_poison(tile[(it + 1) & 1][l * WG + threadIdx.x]);
        }
        float4 r[L];
#pragma unroll
        for (int l = 0; l < L; ++l) {
            const int j = nb + l * WG;
            r[l] = more ? k.pos[j < k.n ? j : k.n - 1] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        }
        const float4 *tl = tile[it & 1];
        zero(blk);
#pragma unroll 8
        for (int u = 0; u < PER; ++u) interact4<1, POT>(tl[g + u * G], tg, eps2, blk);
        add_into(tot, blk);
        if (more) {
#pragma unroll
            for (int l = 0; l < L; ++l) {
                const bool in = nb + l * WG < k.n;
                tile[(it + 1) & 1][l * WG + threadIdx.x] =
                    make_float4(in ? r[l].x : 0.0f, in ? r[l].y : 0.0f, in ? r[l].z : 0.0f,
                                in ? r[l].w : 0.0f);
            }
        }
        __syncthreads();
    }
    const Sums<1, POT> r = result(tot);
    float ax = r.ax[0], ay = r.ay[0], az = r.az[0], ap = POT ? r.p[0] : 0.0f;
    // lanes l and l ^ m (m a multiple of TW) hold the same target t
#pragma unroll
    for (int m = TW; m < 64; m <<= 1) {
        ax += __shfl_xor(ax, m);
        ay += __shfl_xor(ay, m);
        az += __shfl_xor(az, m);
        if constexpr (POT) ap += __shfl_xor(ap, m);
    }
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    if (lane < TW) red[w][lane] = make_float4(ax, ay, az, ap);
    __syncthreads();
    if (threadIdx.x >= TW || i >= k.n) return;
    float4 a = red[0][t];
    for (int ww = 1; ww < NW; ++ww) {
        const float4 b = red[ww][t];
        a.x += b.x;
        a.y += b.y;
        a.z += b.z;
        a.w += b.w;
    }
    if constexpr (STEP) {
        float4 x = me;
        float4 v = k.vel[i];
        euler_update(x, v, a, k.dt);
        k.pos_next[i] = x;
        k.vel[i] = v;
    } else {
        k.acc_out[i] = make_float4(a.x, a.y, a.z, 0.0f);
        if constexpr (POT) k.pot_out[i] = -a.w;
    }
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

    Total<T, POT> tot;
    Sums<T, POT> blk;
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
    store(result(tot), k, base);
}

// ---------------------------------------------------------------- PAIRS
// Pair-symmetric evaluation. r_ji = -r_ij and |r_ji| = |r_ij|, so one pair's
// q = |r|^2 + eps2, inv = q^(-1/2) and inv^3 serve both bodies:
//   a_i += m_j inv^3 r_ij,   a_j -= m_i inv^3 r_ij,   p_i -= m_j inv,   p_j -= m_i inv
// (19 VALU instructions and one v_rsq_f32 per pair instead of 2 x 13 and two).
//
// Work split: bodies are cut into nb bands of BD. Work item (A, d), d in
// [1, nb/2], is the unordered band pair {A, B = (A + d) mod nb}; for even nb
// the opposite band d = nb/2 belongs only to the lower-numbered A. Item
// (A, 0) is the diagonal band, evaluated one-sided (every i of A against every
// j of A, self pairs included). Item (A, d) writes its A-side sums to partial
// slot d and its B-side sums to slot nb - d; the diagonal writes slot 0. Each
// body therefore receives exactly one partial in every slot 0..nb-1, written
// once, and the combine adds the slots in ascending order (deterministic).
//
// Inside an item the 4 waves share one i-set of 64*T bodies of band A (T per
// lane) and take the 64-body j-blocks of band B round-robin. A j-block pass is
// 64 steps: at step s lane l pairs its T targets with j-body (l - s) mod 64 of
// the wave's own LDS copy of the block, and adds that body's sums into its LDS
// slot (same index), which lane l - 1 wrote the step before. After 64 steps
// every j-body has met every lane's targets once. A j-block's sums are added
// into the item's LDS accumulator of band B only by the wave that owns the
// block, in i-set order. After each i-set the waves' A-side sums are added in
// wave order through LDS.

// Body b (64-bit index) or a zero-mass body at the origin for b >= n.
__device__ __forceinline__ float4 body_or_zero(const float4 *__restrict__ pos, int n, long long b)
{
    const bool in = b < n;
    const float4 v = pos[in ? b : n - 1];
    return make_float4(in ? v.x : 0.0f, in ? v.y : 0.0f, in ? v.z : 0.0f, in ? v.w : 0.0f);
}

// Large i-sets or bands sum an i-set across waves sequentially through the
// block and slot rows (keeps 2048-body bands at 40 KiB of LDS, four workgroups
// per CU); small ones, whose occupancy is set by registers, use a one-pass
// buffer with two barriers.
template <int T, int BD>
constexpr bool kSeqReduce = BD >= 2048 || T >= 8;

// Entries per wave row of the j-block and slot arrays: one 64-body block
// (1 KiB, so a row base ORs onto a block offset). The sequential i-set sum
// uses both arrays as one buffer of 8 blocks, enough for 64*T sums at T <= 8.
constexpr int kRowLen = 64;
constexpr int kBlkBytes = 64 * (int)sizeof(float4);

// With 8 targets per lane the targets' sums run over the wave's whole share of
// the i-set's j-blocks (no per-j-block partials): 32 fewer registers, which
// brings the kernel to 128 and four waves per SIMD. The slot combine is
// compensated, so the longer fp32 sums stay far inside the error bound.
template <int T>
constexpr bool kFlatSums = T >= 8;

// Bands above 2048 bodies keep an item's B-side sums in the item's own B-side
// slot in global memory instead of LDS (64 KiB would not fit four workgroups per
// CU): the thread that owns a j-body reads, updates and writes its slot entry
// once per i-set, in i-set order, so the sums and their bits are those of the
// LDS accumulator and no other thread touches the entry.
template <int BD>
constexpr bool kGlobalJacc = BD > 2048;

template <int T, int BD, bool SEQ = kSeqReduce<T, BD>, bool GJ = kGlobalJacc<BD>>
struct PairsShared {
    float4 jacc[BD];          // B-side sums of the item, one per body of band B
    float4 jblk[4][kRowLen];  // each wave's copy of its current j-block
    float4 jsum[4][kRowLen];  // each wave's B-side sums of that block, by block index
    float4 ired[4][64 * T];   // per-wave A-side sums of the current i-set
};

template <int T, int BD>
struct PairsShared<T, BD, true, true> {
    float4 jblk[4][kRowLen];  // as below, without the LDS accumulator of band B
    float4 jsum[4][kRowLen];
};

template <int T, int BD>
struct PairsShared<T, BD, true, false> {
    float4 jacc[BD];          // B-side sums of the item, one per body of band B
    float4 jblk[4][kRowLen];  // each wave's copy of its current j-block; between
                              // i-sets, with jsum, the running cross-wave sum of
                              // the i-set's A-side sums
    float4 jsum[4][kRowLen];  // each wave's B-side sums of its block, by block index
};

// One step: partner (jx, jy, jz, jm) against the lane's T targets. b* gather
// the targets' sums; with SYM, g* gather the partner's.
template <int T, bool POT, bool SYM>
__device__ __forceinline__ void pair_step(float jx, float jy, float jz, float jm,
                                          const float (&tx)[T], const float (&ty)[T],
                                          const float (&tz)[T], const float (&tm)[T],
                                          float eps2, float (&bx)[T], float (&by)[T],
                                          float (&bz)[T], float (&bp)[T], float &gx, float &gy,
                                          float &gz, float &gp)
{
#pragma unroll
    for (int t = 0; t < T; ++t) {
        const float dx = jx - tx[t], dy = jy - ty[t], dz = jz - tz[t];
        float q = __builtin_fmaf(dx, dx, eps2);
        q = __builtin_fmaf(dy, dy, q);
        q = __builtin_fmaf(dz, dz, q);
        const float inv = __builtin_amdgcn_rsqf(q);
        // with the potential also a fence between the rsq and its products (1-2 %
        // faster with 8 targets per lane; 1.5 % slower without the potential)
        if constexpr (T >= 8 && POT) __builtin_amdgcn_sched_barrier(0);
        const float inv3 = (inv * inv) * inv;  // shared by both sides
        // m_i / r^3 is formed before m_j / r^3: with this order the register
        // allocator places the step's temporaries so that far fewer instructions
        // read three VGPRs of one bank (register number mod 4), which issue at
        // half rate on gfx950 (same arithmetic, same bits)
        const float si = SYM ? tm[t] * inv3 : 0.0f;  // m_i / r^3
        const float sj = jm * inv3;                  // m_j / r^3
        bx[t] = __builtin_fmaf(sj, dx, bx[t]);
        by[t] = __builtin_fmaf(sj, dy, by[t]);
        bz[t] = __builtin_fmaf(sj, dz, bz[t]);
        if constexpr (POT) bp[t] = __builtin_fmaf(jm, inv, bp[t]);
        if constexpr (SYM) {
            // the partner's sums are kept with the sign of r_ij (a_j = -sum): plain
            // multiplies and FMAs, no negated operand; the sign is applied once per
            // j-block when the sums go into the band accumulator (bit-identical,
            // since fma(-a, b, c) = -fma(a, b, -c) in round-to-nearest)
            gx = __builtin_fmaf(si, dx, gx);
            gy = __builtin_fmaf(si, dy, gy);
            gz = __builtin_fmaf(si, dz, gz);
            if constexpr (POT) gp = __builtin_fmaf(tm[t], inv, gp);
        }
        // With 8 targets per lane each target's chain stays together: the scheduler
        // may not pull the next target's differences or rsq in among these FMAs.
        // Measured on gfx950, that strictly sequential stream pairs the VALU
        // instructions of two waves more often and takes 56.4 instead of 59.5 SIMD
        // cycles per wave-pair (1.3-5 % faster, box to box), while a software-
        // pipelined one (the next rsq placed ahead of these FMAs) is 11 % slower;
        // with 4 targets per lane the compiler's own order measured 2-4 % faster,
        // so it is left free there.
        if constexpr (T >= 8) __builtin_amdgcn_sched_barrier(0);
    }
}

template <typename V>
__device__ __forceinline__ V &at_byte(void *base, int off)
{
    return *reinterpret_cast<V *>(static_cast<char *>(base) + off);
}

// One j-block pass of 64 steps: at step s lane l pairs its T targets with body
// (l - s) mod 64 of the wave's block copy (byte row `row` of blk; jbody is the
// lane's own body, the partner of step 0), and with SYM adds that body's sums
// into its entry of the wave's sum row, which lane l - 1 wrote the step before.
// U steps per loop trip.
template <int T, bool POT, bool SYM, int U>
__device__ __forceinline__ void block_pass(void *blk, void *sum, int row, int lane, float4 jbody,
                                           const float (&tx)[T], const float (&ty)[T],
                                           const float (&tz)[T], const float (&tm)[T],
                                           float eps2, float (&bx)[T], float (&by)[T],
                                           float (&bz)[T], float (&bp)[T])
{
    float jx = jbody.x, jy = jbody.y, jz = jbody.z, jm = jbody.w;
    int cur = row | (lane * (int)sizeof(float4));  // byte offset of entry (lane - step) mod 64
#pragma unroll U
    for (int step = 0; step < 64; ++step) {
        const int nxt = ((cur - (int)sizeof(float4)) & (kBlkBytes - 1)) | row;
        // the partner's sums first, then the partner of the next step (read
        // ahead of this step's arithmetic): LDS reads return in order, so the
        // first FMA into the sums waits only for the first read
        float gx = 0.0f, gy = 0.0f, gz = 0.0f, gp = 0.0f;
        if constexpr (SYM) {
            const float4 g = at_byte<const float4>(sum, cur);
            gx = g.x;
            gy = g.y;
            gz = g.z;
            gp = g.w;
        }
        const float4 nb4 = at_byte<const float4>(blk, nxt);
        pair_step<T, POT, SYM>(jx, jy, jz, jm, tx, ty, tz, tm, eps2, bx, by, bz, bp, gx, gy, gz,
                               gp);
        if constexpr (SYM) {
            at_byte<float4>(sum, cur) = make_float4(gx, gy, gz, gp);
            __builtin_amdgcn_wave_barrier();
        }
        jx = nb4.x;
        jy = nb4.y;
        jz = nb4.z;
        jm = nb4.w;
        cur = nxt;
    }
}

// Item {A, B}: band A's targets held in registers (their sums written to
// outA[body - offA] after each i-set), band B walked in j-blocks. With SYM the
// B side is added into the LDS accumulator jacc (kept across the items of a
// run; the caller zeroes and stores it), or with a global accumulator into
// outB[body - offB], which the first item of a run starts afresh.
template <int T, int BD, bool POT, bool SYM>
__device__ __forceinline__ void pairs_item(const PairsArgs &k, int A, int B, float4 *outA,
                                           long long offA, float4 *outB, long long offB,
                                           bool first_of_run, float eps2, PairsShared<T, BD> &sh)
{
    constexpr int W = 4;
    constexpr int NIS = BD / (64 * T);  // i-sets per band
    constexpr int NJB = BD / 64;        // j-blocks per band
    static_assert(NIS >= 1 && NJB % W == 0, "band must hold whole i-sets and j-blocks");
    static_assert(sizeof(sh.jblk[0]) == kBlkBytes && sizeof(sh.jsum[0]) == kBlkBytes,
                  "rows must be one block each");
    static_assert(!kSeqReduce<T, BD> || 64 * T <= 2 * W * kRowLen,
                  "the sequential i-set sum must fit the block and slot rows");
    constexpr bool FLAT = kFlatSums<T>;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int row = w * (int)sizeof(sh.jblk[0]);  // byte offset of the wave's row
    for (int is = 0; is < NIS; ++is) {
        float tx[T], ty[T], tz[T], tm[T];
        // i-set sums (a*) and, unless FLAT, the current j-block's partials (b*)
        float ax[T], ay[T], az[T], ap[T];
        float bx[T], by[T], bz[T], bp[T];
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const float4 b = body_or_zero(k.pos, k.n, (long long)A * BD + is * 64 * T + t * 64 + lane);
            tx[t] = b.x;
            ty[t] = b.y;
            tz[t] = b.z;
            tm[t] = b.w;
            ax[t] = ay[t] = az[t] = ap[t] = 0.0f;
            bx[t] = by[t] = bz[t] = bp[t] = 0.0f;
        }
        float4 jnext = body_or_zero(k.pos, k.n, (long long)B * BD + w * 64 + lane);
        for (int jb = w; jb < NJB; jb += W) {
            const float4 jbody = jnext;
            // the wave's next j-block, loaded while this one is evaluated
            if (jb + W < NJB) jnext = body_or_zero(k.pos, k.n, (long long)B * BD + (jb + W) * 64 + lane);
            // The block copy and the slots are written and read only by this
            // wave, whose LDS accesses execute in program order; the wave
            // barriers keep the compiler from moving accesses across.
            __builtin_amdgcn_wave_barrier();
            sh.jblk[w][lane] = jbody;
            if constexpr (SYM) sh.jsum[w][lane] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            __builtin_amdgcn_wave_barrier();
            if constexpr (!FLAT) {
#pragma unroll
                for (int t = 0; t < T; ++t) bx[t] = by[t] = bz[t] = bp[t] = 0.0f;
            }
            // two steps per trip (no register copies of the partner) except where
            // measured slower: 4 targets per lane in 2048-body bands
            constexpr int U = (T == 4 && BD >= 2048) ? 1 : 2;
            block_pass<T, POT, SYM, U>(&sh.jblk[0][0], &sh.jsum[0][0], row, lane, jbody, tx, ty,
                                       tz, tm, eps2, bx, by, bz, bp);
            if constexpr (!FLAT) {
#pragma unroll
                for (int t = 0; t < T; ++t) {
                    ax[t] += bx[t];
                    ay[t] += by[t];
                    az[t] += bz[t];
                    ap[t] += bp[t];
                }
            }
            if constexpr (SYM && kGlobalJacc<BD>) {
                const float4 g = sh.jsum[w][lane];
                const long long body = (long long)B * BD + jb * 64 + lane;
                if (body < k.n) {
                    float4 *dst = outB + (body - offB);
                    float4 o = (is == 0 && first_of_run) ? make_float4(0.0f, 0.0f, 0.0f, 0.0f) : *dst;
                    o.x -= g.x;
                    o.y -= g.y;
                    o.z -= g.z;
                    o.w += g.w;
                    *dst = o;
                }
            } else if constexpr (SYM) {
                const float4 g = sh.jsum[w][lane];
                float4 o = sh.jacc[jb * 64 + lane];
                o.x -= g.x;
                o.y -= g.y;
                o.z -= g.z;
                o.w += g.w;
                sh.jacc[jb * 64 + lane] = o;
            }
        }
        if constexpr (FLAT) {
#pragma unroll
            for (int t = 0; t < T; ++t) {
                ax[t] = bx[t];
                ay[t] = by[t];
                az[t] = bz[t];
                ap[t] = bp[t];
            }
        }
        // Cross-wave sum of the i-set, in wave order ((w0 + w1) + w2) + w3 either way.
        if constexpr (!kSeqReduce<T, BD>) {
#pragma unroll
            for (int t = 0; t < T; ++t)
                sh.ired[w][t * 64 + lane] = make_float4(ax[t], ay[t], az[t], ap[t]);
            __syncthreads();
            for (int idx = threadIdx.x; idx < 64 * T; idx += 64 * W) {
                float4 s = sh.ired[0][idx];
#pragma unroll
                for (int ww = 1; ww < W; ++ww) {
                    const float4 v = sh.ired[ww][idx];
                    s = make_float4(s.x + v.x, s.y + v.y, s.z + v.z, s.w + v.w);
                }
                const long long body = (long long)A * BD + is * 64 * T + idx;
                if (body < k.n) outA[body - offA] = s;
            }
            __syncthreads();
            if constexpr (kRaceProbe) {
                for (int t = 0; t < T; ++t) probe_poison(sh.ired[w][t * 64 + lane]);
            }
            continue;
        }
        // Sequential form through the block and slot rows (all waves are past
        // their j-blocks at the barrier); wave W-1 stores the total.
        float4 *red = &sh.jblk[0][0];
        __syncthreads();
        for (int ww = 0; ww < W; ++ww) {
            if (w == ww) {
#pragma unroll
                for (int t = 0; t < T; ++t) {
                    const int idx = t * 64 + lane;
                    float4 v = make_float4(ax[t], ay[t], az[t], ap[t]);
                    if (ww > 0) {
                        const float4 s = red[idx];
                        v = make_float4(s.x + v.x, s.y + v.y, s.z + v.z, s.w + v.w);
                    }
                    if (ww < W - 1) {
                        red[idx] = v;
                    } else {
                        const long long body = (long long)A * BD + is * 64 * T + idx;
                        if (body < k.n) outA[body - offA] = v;
                    }
                }
            }
            __syncthreads();
        }
        probe_poison(sh.jblk[w][lane]);
        probe_poison(sh.jsum[w][lane]);
    }
}

// Whether item (x, d) exists: the diagonal, d below nb/2, and for even nb the
// opposite pair d = nb/2 from the lower half only.
__device__ __forceinline__ bool item_exists(int x, int d, int nb)
{
    if (d == 0) return true;
    if (nb == 1 || 2 * d > nb) return false;
    return 2 * d < nb || x < nb / 2;
}

// grid (band1 - band0, 1 + R), 256 threads. Row 0: the diagonal item of
// owner X = band0 + blockIdx.x. Row 1 + r: run r of X, the items (X, d) for d
// in [1 + r K, min((r + 1) K, nb/2)] in ascending d; band X is the walked band
// of each, so its sums stay in the LDS accumulator for the whole run and are
// stored once, into own slot 1 + r, and each partner band Y = X + d holds its
// targets in registers and writes them to partner slot d. A run whose first
// item does not exist (only d = nb/2 for X >= nb/2, even nb) returns at once,
// uniformly, before any barrier.
template <int T, int BD, bool POT>
__global__ void __launch_bounds__(256) accel_pairs(PairsArgs k)
{
    __shared__ PairsShared<T, BD> sh;
    const int nb = k.nbands;
    const int X = k.band0 + (int)blockIdx.x;
    const float eps2 = in_vgpr(k.eps2);
    if (blockIdx.y == 0) {
        pairs_item<T, BD, POT, false>(k, X, X, k.own, k.own0, nullptr, 0, true, eps2, sh);
        return;
    }
    const int r = (int)blockIdx.y - 1;
    const int d0 = 1 + run_start(r, nb, k.run);
    const int d1 = run_start(r + 1, nb, k.run);
    if (!item_exists(X, d0, nb)) return;
    float4 *runslot = k.own + (size_t)(1 + r) * (size_t)k.own_stride;
    if constexpr (!kGlobalJacc<BD>) {
        for (int i = threadIdx.x; i < BD; i += 256) sh.jacc[i] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        __syncthreads();
    }
    for (int d = d0; d <= d1; ++d) {
        if (!item_exists(X, d, nb)) break;  // only d = nb/2 can be missing: the run's last
        const int Y = X + d < nb ? X + d : X + d - nb;
        const int p = k.partner_by_owner ? X - k.band0 : d - 1;
        float4 *tgt = k.partner + (size_t)p * (size_t)k.partner_stride;
        pairs_item<T, BD, POT, true>(k, Y, X, tgt, 0, runslot, k.own0, d == d0, eps2, sh);
    }
    if constexpr (!kGlobalJacc<BD>) {
        // entry i was accumulated by this same thread (block i / 64 belongs to
        // wave (i / 64) mod 4), so no barrier is needed before the store
        for (int i = threadIdx.x; i < BD; i += 256) {
            const long long body = (long long)X * BD + i;
            if (body < k.n) runslot[body - k.own0] = sh.jacc[i];
        }
    }
}

// ---------------------------------------------------------------- combine / Euler
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

// The ordered sum and Euler step of euler_update, in place.
__global__ void __launch_bounds__(256) euler_kernel(const float4 *__restrict__ part, int n,
                                                    int splits, float4 *__restrict__ pos,
                                                    float4 *__restrict__ vel, float dt)
{
    const unsigned i = blockIdx.x * 256u + threadIdx.x;
    if (i >= (unsigned)n) return;
    const float4 a = sum_parts(part, n, splits, i);
    float4 x = pos[i];
    float4 v = vel[i];
    euler_update(x, v, a, dt);
    pos[i] = x;
    vel[i] = v;
}

// ---------------------------------------------------------------- pair finish
// Adds base[s * stride], s = 0 .. count-1, in order into the compensated sum
// (a, e); a body's first addend starts the sum (as in sum_parts). Loads run
// eight slots ahead of the in-order additions.
__device__ __forceinline__ void add_slots(float4 &a, float4 &e, bool &started,
                                          const float4 *base, size_t stride, int count)
{
    int s = 0;
    if (!started && count > 0) {
        a = base[0];
        started = true;
        s = 1;
    }
    for (; s + 8 <= count; s += 8) {
        float4 b[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) b[u] = base[(size_t)(s + u) * stride];
#pragma unroll
        for (int u = 0; u < 8; ++u) two_sum_add4(a, e, b[u]);
    }
    for (; s < count; ++s) two_sum_add4(a, e, base[(size_t)s * stride]);
}

__device__ __forceinline__ void add_one(float4 &a, float4 &e, bool &started, const float4 &v)
{
    if (started) {
        two_sum_add4(a, e, v);
    } else {
        a = v;
        started = true;
    }
}

// Own slots that band x's bodies hold: the diagonal and every run whose first
// item exists (only the last run, when it is d = nb/2 alone for x >= nb/2,
// can be empty).
__device__ __forceinline__ int own_slots(int x, int nb, int run, int nruns)
{
    return 1 + nruns - ((nruns > 0 && !item_exists(x, 1 + run_start(nruns - 1, nb, run), nb)) ? 1 : 0);
}

// Partner slots d = 1 .. that band x's bodies hold: all D = nb/2 except, for
// even nb, d = nb/2 when its owner x - nb/2 (mod nb) is in the upper half.
__device__ __forceinline__ int partner_slots(int x, int nb)
{
    const int D = nb / 2;
    if (D == 0) return 0;
    const int o = x >= D ? x - D : x - D + nb;
    return item_exists(o, D, nb) ? D : D - 1;
}

__global__ void __launch_bounds__(256) pairs_finish_kernel(PairsFinishArgs k)
{
    const unsigned i = blockIdx.x * 256u + threadIdx.x;
    if (i >= (unsigned)k.n) return;
    const int x = (int)(i / (unsigned)k.band), nb = k.nbands;
    const int nruns = pair_runs(nb, k.run);
    const size_t n = (size_t)k.n;
    float4 a = make_float4(0.0f, 0.0f, 0.0f, 0.0f), e = a;
    bool started = false;
    add_slots(a, e, started, k.part + i, n, own_slots(x, nb, k.run, nruns));
    add_slots(a, e, started, k.part + (size_t)(1 + nruns) * n + i, n, partner_slots(x, nb));
    const float4 r = make_float4(a.x + e.x, a.y + e.y, a.z + e.z, a.w + e.w);
    if (k.pos) {
        float4 xp = k.pos[i];
        float4 v = k.vel[i];
        euler_update(xp, v, r, k.dt);
        k.pos[i] = xp;
        k.vel[i] = v;
        return;
    }
    k.acc_out[i] = make_float4(r.x, r.y, r.z, 0.0f);
    if (k.pot_out) k.pot_out[i] = -r.w;
}

// ---------------------------------------------------------------- shards
// A shard owns the items of the owner bands [band0, band1): the own slots of
// its bands' bodies and the partner slot d of a body of band x when x - d
// (mod nb) is one of them. Added in the finish's order, so one shard of one is
// the one-pass finish bit for bit.
__global__ void __launch_bounds__(256) shard_combine_kernel(const float4 *__restrict__ part, int n,
                                                            int band, int nb, int run, int band0,
                                                            int band1, float4 *__restrict__ out)
{
    const unsigned i = blockIdx.x * 256u + threadIdx.x;
    if (i >= (unsigned)n) return;
    const int x = (int)(i / (unsigned)band);
    const int nruns = pair_runs(nb, run);
    float4 a = make_float4(0.0f, 0.0f, 0.0f, 0.0f), e = a;
    bool started = false;
    if (x >= band0 && x < band1) add_slots(a, e, started, part + i, (size_t)n, own_slots(x, nb, run, nruns));
    const int np = partner_slots(x, nb);
    const float4 *pb = part + (size_t)(1 + nruns) * (size_t)n + i;
    for (int d = 1; d <= np; ++d) {
        const int o = x >= d ? x - d : x - d + nb;
        if (o >= band0 && o < band1) add_one(a, e, started, pb[(size_t)(d - 1) * (size_t)n]);
    }
    out[i] = make_float4(a.x + e.x, a.y + e.y, a.z + e.z, a.w + e.w);
}

__global__ void __launch_bounds__(256) shard_finish_kernel(const float4 *__restrict__ partials,
                                                           int n, int nshards, int t0, int t1,
                                                           float4 *__restrict__ acc_out,
                                                           float *__restrict__ pot_out)
{
    const unsigned i = (unsigned)t0 + blockIdx.x * 256u + threadIdx.x;
    if (i >= (unsigned)t1) return;
    const float4 a = sum_parts(partials, n, nshards, i);
    acc_out[i - t0] = make_float4(a.x, a.y, a.z, 0.0f);
    if (pot_out) pot_out[i - t0] = -a.w;
}

// ---------------------------------------------------------------- passes
__global__ void __launch_bounds__(256) pass_combine_kernel(PassArgs k)
{
    const unsigned i = blockIdx.x * 256u + threadIdx.x;
    if (i >= (unsigned)k.n) return;
    const int x = (int)(i / (unsigned)k.band), nb = k.nbands;
    float4 a = make_float4(0.0f, 0.0f, 0.0f, 0.0f), e = a;
    bool started = !k.first;
    if (started) {
        a = k.tot_s[i];
        e = k.tot_e[i];
    }
    // this body's own slots (its band is one of the pass's owners)
    if (x >= k.band0 && x < k.band1)
        add_slots(a, e, started, k.own + ((int)i - k.own0), (size_t)k.own_count,
                  own_slots(x, nb, k.run, pair_runs(nb, k.run)));
    // its partner sides from the pass's owners, ascending owner
    for (int o = k.band0; o < k.band1; ++o) {
        int d = x - o;
        if (d < 0) d += nb;
        if (d >= 1 && item_exists(o, d, nb))
            add_one(a, e, started, k.partner[(size_t)(o - k.band0) * (size_t)k.n + i]);
    }
    if (!k.last) {
        k.tot_s[i] = a;
        k.tot_e[i] = e;
        return;
    }
    const float4 r = make_float4(a.x + e.x, a.y + e.y, a.z + e.z, a.w + e.w);
    if (k.pot_out) {
        k.acc_out[i] = make_float4(r.x, r.y, r.z, 0.0f);
        k.pot_out[i] = -r.w;
    } else {
        k.acc_out[i] = r;
    }
}

// ---------------------------------------------------------------- diagnostics
// Conserved quantities of a state, in fp64 (the inputs are fp32, so products
// and squares are nearly exact): per body
//   K += m |v|^2 / 2,  W += m (p + m / eps) / 2,  P += m v,  L += m x × v,
//   M += m,  MX += m x
// (the pair energy from the method's potential with its softened self term
// removed; Nakasato, "スライド 1", No.4 for p). Thread t of workgroup b takes
// bodies b*256 + t + k*(B*256); workgroup sums use a fixed tree, the final sum
// adds the B workgroup sums in order. Deterministic for a given N.
constexpr int kDiagMaxBlocks = 1024;

__device__ __forceinline__ void diag_tree(double (&v)[kDiagSums], double (*red)[256])
{
#pragma unroll
    for (int q = 0; q < kDiagSums; ++q) red[q][threadIdx.x] = v[q];
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
        if ((int)threadIdx.x < s) {
#pragma unroll
            for (int q = 0; q < kDiagSums; ++q) red[q][threadIdx.x] += red[q][threadIdx.x + s];
        }
        __syncthreads();
    }
}

__global__ void __launch_bounds__(256) diag_partial_kernel(const float4 *__restrict__ pos,
                                                           const float4 *__restrict__ vel,
                                                           const float *__restrict__ pot, int n,
                                                           double inv_eps, double *part)
{
    __shared__ double red[kDiagSums][256];
    double v[kDiagSums];
#pragma unroll
    for (int q = 0; q < kDiagSums; ++q) v[q] = 0.0;
    for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n;
         i += (long long)gridDim.x * 256) {
        const float4 b = pos[i], u = vel[i];
        const double m = b.w, x = b.x, y = b.y, z = b.z;
        const double vx = u.x, vy = u.y, vz = u.z;
        v[0] += 0.5 * m * (vx * vx + vy * vy + vz * vz);
        v[1] += 0.5 * m * ((double)pot[i] + m * inv_eps);
        v[2] += m * vx;
        v[3] += m * vy;
        v[4] += m * vz;
        v[5] += m * (y * vz - z * vy);
        v[6] += m * (z * vx - x * vz);
        v[7] += m * (x * vy - y * vx);
        v[8] += m;
        v[9] += m * x;
        v[10] += m * y;
        v[11] += m * z;
    }
    diag_tree(v, red);
    if (threadIdx.x < kDiagSums) part[blockIdx.x * kDiagSums + threadIdx.x] = red[threadIdx.x][0];
}

__global__ void __launch_bounds__(256) diag_final_kernel(const double *__restrict__ part,
                                                         int nblocks, double *__restrict__ out)
{
    __shared__ double red[kDiagSums][256];
    double v[kDiagSums];
#pragma unroll
    for (int q = 0; q < kDiagSums; ++q) v[q] = 0.0;
    for (int b = threadIdx.x; b < nblocks; b += 256) {
#pragma unroll
        for (int q = 0; q < kDiagSums; ++q) v[q] += part[b * kDiagSums + q];
    }
    diag_tree(v, red);
    if (threadIdx.x != 0) return;
    const double k = red[0][0], w = red[1][0], m = red[8][0];
    out[0] = k;
    out[1] = w;
    out[2] = k + w;
    for (int c = 0; c < 3; ++c) {
        out[3 + c] = red[2 + c][0];
        out[6 + c] = red[5 + c][0];
        out[10 + c] = m != 0.0 ? red[9 + c][0] / m : 0.0;
    }
    out[9] = m;
}

// ---------------------------------------------------------------- near field
// All-pairs as the near part of a hierarchical method (GPU Gems 3 ch. 31 study
// page, section 6; Nakasato, "スライド 1", No.34): each target cell's bodies
// sum over the bodies of the cells in its interaction list. Two waves (64
// threads each) per target cell, taking alternate chunks of the cell's bodies,
// 64 at a time, one per lane (or 256, four per lane); each
// listed source cell is staged through the wave's own 64-body LDS row and read
// back with LDS reads (a broadcast within each source group). Every source
// tile is one block of the compensated two-level accumulation. Ranges and list entries are
// checked before use (memory safety for any input): a target cell with an
// invalid range is skipped, an invalid list range is empty, an out-of-range
// list entry or a source cell with an invalid range adds nothing.
// A list hands out source runs: entry e of [lo, hi) is a range of bodies
// [sb, sn), or nothing (`source` returns false for an invalid or empty entry).
// CSR lists are walked as one sequence of bodies cut into 64-body tiles (the
// listed cells one after another, so small cells share tiles instead of each
// filling part of one), kPackEntries entries at a time: for each such segment
// wave 0 reads the entries' body ranges and writes their exclusive prefix pre[]
// and offsets off[] (position p of the segment, pre[e] <= p < pre[e + 1], is
// body p + off[e]) to LDS between two workgroup barriers.
constexpr int kPackEntries = 64;
constexpr int kPackLds = 2 * kPackEntries + 1;  // ints: pre[0 .. 64], off[0 .. 63]

struct PackedLists {
    const int *off;
    const int *list;
    long long nlist;
    int ncell;
    int *tab;         // kPackLds LDS ints (set by the kernel)
    int bound_seg;    // segment in tab (-1: none), uniform
    __device__ void bind(const P2PArgs &, int) { bound_seg = -1; }
    __device__ int cell(int b) const { return b; }  // workgroups in cell order
    __device__ void range(int c, int &lo, int &hi) const
    {
        long long a = off[c], b = off[c + 1];
        if (a < 0 || b < a || b > nlist) a = b = 0;
        lo = (int)a;
        hi = (int)b;
    }
    // entry e: the bodies of listed cell list[e]
    __device__ bool source(const P2PArgs &k, int e, int &sb, int &sn) const
    {
        const int s = list[e];
        if (s < 0 || s >= ncell) return false;
        sb = k.cell_start[s];
        sn = k.cell_start[s + 1];
        return sb >= 0 && sn > sb && sn <= k.n;
    }
    __device__ int segments(int lo, int hi) const
    {
        return hi > lo ? (hi - lo + kPackEntries - 1) / kPackEntries : 0;
    }
    // wave 0: entries [lo + sg * 64, ...) of the list into tab
    __device__ void load_segment(const P2PArgs &k, int lo, int hi, int sg, int lane)
    {
        const int e = lo + sg * kPackEntries + lane;
        int sb = 0, sn = 0;
        const bool ok = e < hi && source(k, e, sb, sn);
        const int size = ok ? sn - sb : 0;
        int incl = size;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(incl, o);
            if (lane >= o) incl += y;
        }
        const int excl = incl - size;
        tab[lane] = excl;
        tab[kPackEntries + 1 + lane] = sb - excl;
        if (lane == 63) tab[kPackEntries] = incl;
    }
};

// The 27 neighbours of the target cell as 9 runs of consecutive cells: for
// each (y, z) offset (entry 3 (z + 1) + (y + 1)) the cells x - 1 .. x + 1 that
// lie in the grid are consecutive in the x-fastest cell order, so their bodies
// are one contiguous range of the sorted array (the same bodies in the same
// order as the three cells one after another, in a third of the runs, which
// leaves fewer part-filled source tiles). Lanes 0..8 read the runs' body ranges
// from cell_start into LDS once per workgroup, so that the tile walk of every
// wave finds them there instead of waiting on global loads at each run.
// The chunk kernel walks the 9 runs as one sequence of bodies (run 0, then run 1,
// ...) cut into 64-body tiles, so that only the last tile of the neighbourhood is
// part-filled rather than the last tile of every run: position p of the sequence
// lies in run e with pre[e] <= p < pre[e + 1] and is body p + off[e].
constexpr int kGridRuns = 9;
constexpr int kGridLds = 2 * kGridRuns + (kGridRuns + 1) + kGridRuns;  // ints

struct GridLists {
    int dx, dy, dz;
    // kGridLds LDS ints: the body range [sb, sn) of each run ((-1, -1) outside the grid),
    // then pre[10] and off[9] of the run sequence
    int *nbr;
    int heavy_first;  // launch order of cells: see cell()
    // The cell of launch index b. With heavy_first, heaviest neighbourhoods first: the
    // interior cells (27 neighbours), then the six faces (18), the twelve edges (12)
    // and the eight corners (8), each in natural order. Workgroups start roughly in
    // launch order, so the cheapest cells are the ones left for the end of the launch,
    // where they fill the CUs that free up (at 256 bodies per cell and N = 2^20, 4096
    // cells run as about four rounds of workgroups: 4.3 % faster, same bits). A
    // bijection of [0, dx*dy*dz); the identity without heavy_first or when a dimension
    // is below 3.
    __device__ int at(int x, int y, int z) const { return (z * dy + y) * dx + x; }
    __device__ int cell(int b) const
    {
        const int ix = dx - 2, iy = dy - 2, iz = dz - 2;
        if (!heavy_first || ix < 1 || iy < 1 || iz < 1) return b;
        const int ni = ix * iy * iz;
        if (b < ni) return at(1 + b % ix, 1 + (b / ix) % iy, 1 + b / (ix * iy));
        b -= ni;
#pragma unroll 1
        for (int f = 0; f < 6; ++f) {  // z faces, y faces, x faces; low side first
            const int axis = f >> 1, hi = f & 1;
            const int a = axis == 2 ? iy : ix, sz = (axis == 0 ? iy : iz) * a;
            if (b < sz) {
                const int u = 1 + b % a, v = 1 + b / a;
                if (axis == 0) return at(u, v, hi ? dz - 1 : 0);
                if (axis == 1) return at(u, hi ? dy - 1 : 0, v);
                return at(hi ? dx - 1 : 0, u, v);
            }
            b -= sz;
        }
#pragma unroll 1
        for (int e = 0; e < 12; ++e) {  // four edges along x, four along y, four along z
            const int axis = e >> 2, p = e & 1, q = (e >> 1) & 1;
            const int len = axis == 0 ? ix : (axis == 1 ? iy : iz);
            if (b < len) {
                const int t = 1 + b;
                if (axis == 0) return at(t, p ? dy - 1 : 0, q ? dz - 1 : 0);
                if (axis == 1) return at(p ? dx - 1 : 0, t, q ? dz - 1 : 0);
                return at(p ? dx - 1 : 0, q ? dy - 1 : 0, t);
            }
            b -= len;
        }
        return at(b & 1 ? dx - 1 : 0, b & 2 ? dy - 1 : 0, b & 4 ? dz - 1 : 0);
    }
    __device__ const int *pre() const { return nbr + 2 * kGridRuns; }
    __device__ const int *off() const { return nbr + 3 * kGridRuns + 1; }
    __device__ void bind(const P2PArgs &k, int c)
    {
        const int lane = threadIdx.x;
        if (lane < kGridRuns) {
            const int cx = c % dx, cy = (c / dx) % dy, cz = c / (dx * dy);
            const int y = cy + lane % 3 - 1, z = cz + lane / 3 - 1;
            const bool in = y >= 0 && y < dy && z >= 0 && z < dz;
            const int row = (z * dy + y) * dx;
            const int first = row + (cx > 0 ? cx - 1 : 0);
            const int last = row + (cx + 1 < dx ? cx + 1 : dx - 1);
            nbr[2 * lane] = in ? k.cell_start[first] : -1;
            nbr[2 * lane + 1] = in ? k.cell_start[last + 1] : -1;
        }
        __syncthreads();
        if (lane == 0) {
            int *pr = nbr + 2 * kGridRuns, *of = nbr + 3 * kGridRuns + 1;
            int at = 0;
            for (int e = 0; e < kGridRuns; ++e) {
                const int sb = nbr[2 * e], sn = nbr[2 * e + 1];
                const bool ok = sb >= 0 && sn > sb && sn <= k.n;
                pr[e] = at;
                of[e] = ok ? sb - at : 0;
                at += ok ? sn - sb : 0;
            }
            pr[kGridRuns] = at;
        }
        __syncthreads();
    }
    __device__ void range(int, int &lo, int &hi) const
    {
        lo = 0;
        hi = 9;
    }
    __device__ bool source(const P2PArgs &k, int e, int &sb, int &sn) const
    {
        sb = __builtin_amdgcn_readfirstlane(nbr[2 * e]);
        sn = __builtin_amdgcn_readfirstlane(nbr[2 * e + 1]);
        return sb >= 0 && sn > sb && sn <= k.n;
    }
};

// Walk over the source tiles of a target cell's list: tile = bodies
// [j0, min(j0 + 64, se)) of list entry e. Starting from (e, j0, se), moves to
// the next tile (the rest of the same run, then the next valid non-empty
// entry); false when the list is exhausted. Uniform across the wave.
template <typename Lists>
__device__ __forceinline__ bool next_tile(const P2PArgs &k, const Lists &lists, int hi, int &e,
                                          int &j0, int &se)
{
    if (j0 + 64 < se) {
        j0 += 64;
        return true;
    }
#pragma unroll 1
    for (++e; e < hi; ++e) {
        int sb, sn;
        if (!lists.source(k, e, sb, sn)) continue;  // invalid or empty: no tiles
        j0 = sb;
        se = sn;
        return true;
    }
    return false;
}

// The chunk that starts where rem targets of a cell are left: one target per lane
// on 2^lg lanes per source group: 64 when more than 48 remain, 32 when 33-48 remain
// (the rest, at most 16, then takes a chunk of its own with four or more source
// groups, instead of leaving up to half of a 64-lane chunk idle: a chunk costs a
// walk over the neighbourhood, so a rest of 17 or more keeps the 64-lane chunk),
// else the next power of two >= rem. Returns the targets the chunk takes. (Four
// targets per lane in 256-target chunks, each staged source serving four terms,
// needed 124 VGPRs and four waves per SIMD; at eight waves the one-target chunks
// measured 4-5 % faster on 16^3 and 15^3 grids of N = 2^20 and on octree leaves of
// ~256 bodies, the only places the automatic choice had used them.)
__device__ __forceinline__ int chunk_span(int rem, int &lg)
{
    const int want = rem > 48 ? 64 : (rem > 32 ? 32 : rem);
    int tw = 1;
    lg = 0;
    while (tw < want) {
        tw <<= 1;
        ++lg;
    }
    return tw;
}

// Whether a cell of r bodies has a chunk q >= 1 (the chunk sequence of chunk_span);
// the launches ask for q < 4 (at most four chunk workgroups per cell).
__device__ __forceinline__ bool cell_has_chunk(int r, int q)
{
    int n = 0;
    while (r > 0 && n <= q) {
        int lg;
        r -= chunk_span(r, lg);
        ++n;
    }
    return n > q;
}

// Waves per workgroup of the near-field chunk kernel: W waves work on the same
// target chunk, wave w taking the source tiles w, w + W, w + 2W, ... of the
// chunk's neighbourhood walk, and their sums are added in wave order at the
// end. With four waves a cell's work is spread over waves that finish
// together, instead of one long wave per chunk whose remainder chunk ran after
// the others (256 bodies per cell at N = 2^20: 2.40 -> 2.11 ms); small cells,
// whose neighbourhoods are a few tiles, keep one wave (9.5 bodies per cell:
// 0.23 ms with one wave, 0.49 with four). Four from kP2PWavesMinBodies bodies
// per cell on average.
constexpr int kP2PWaves = 4;
constexpr int kP2PWavesMinBodies = 64;

// Moves the walk `count` tiles on; false if the list ends first.
template <typename Lists>
__device__ __forceinline__ bool skip_tiles(const P2PArgs &k, const Lists &lists, int hi, int &e,
                                           int &j0, int &se, int count)
{
    for (int s = 0; s < count; ++s)
        if (!next_tile(k, lists, hi, e, j0, se)) return false;
    return true;
}

// A wave's walk over the source tiles of a target cell's list: start() puts it on
// tile w, next() moves it `step` tiles on, count() is the number of bodies in the
// current tile (at most 64) and load() lane's body of it (an index clamped into
// the tile; the stage pads the lanes past count() with zero masses). All uniform
// across the wave.
//   PackedListCursor: the current segment of a CSR list (PackedLists, in LDS) as
//   one sequence of bodies in 64-body tiles; lane's body of tile t is found by a
//   binary search of its position in the segment's prefix pre[].
struct PackedListCursor {
    int total, t;
    const int *tab;  // LDS: pre[0 .. 64], off[0 .. 63]
    bool have;
    __device__ void start(const P2PArgs &, const PackedLists &l, int, int, int w)
    {
        tab = l.tab;
        total = __builtin_amdgcn_readfirstlane(tab[kPackEntries]);
        t = w;
        have = t * 64 < total;
    }
    __device__ void next(const P2PArgs &, const PackedLists &, int step)
    {
        t += step;
        have = t * 64 < total;
    }
    __device__ int count() const { return total - t * 64 < 64 ? total - t * 64 : 64; }
    __device__ float4 load(const P2PArgs &k, int lane) const
    {
        int p = t * 64 + lane;
        p = p < total ? p : total - 1;
        int a = 1, b = kPackEntries;  // the last e with pre[e] <= p (pre[0] = 0)
        while (a < b) {
            const int m = (a + b) >> 1;
            if (tab[m] <= p) a = m + 1;
            else b = m;
        }
        return k.pos[p + tab[kPackEntries + 1 + a - 1]];
    }
};

//   PackedCursor: the 9 grid runs as one sequence of bodies in 64-body tiles
//   (GridLists), so only the sequence's last tile is part-filled.
struct PackedCursor {
    int total, t;
    int pre[kGridRuns];  // pre[1 .. 8] of the run sequence (uniform)
    const int *off;      // LDS
    bool have;
    __device__ void start(const P2PArgs &, const GridLists &l, int, int, int w)
    {
        const int *p = l.pre();
#pragma unroll
        for (int e = 1; e < kGridRuns; ++e) pre[e] = __builtin_amdgcn_readfirstlane(p[e]);
        total = __builtin_amdgcn_readfirstlane(p[kGridRuns]);
        off = l.off();
        t = w;
        have = t * 64 < total;
    }
    __device__ void next(const P2PArgs &, const GridLists &, int step)
    {
        t += step;
        have = t * 64 < total;
    }
    __device__ int count() const { return total - t * 64 < 64 ? total - t * 64 : 64; }
    __device__ float4 load(const P2PArgs &k, int lane) const
    {
        int p = t * 64 + lane;
        p = p < total ? p : total - 1;
        int e = 0;
#pragma unroll
        for (int q = 1; q < kGridRuns; ++q) e += p >= pre[q] ? 1 : 0;
        return k.pos[p + off[e]];
    }
};

template <typename Lists>
struct CursorOf;
template <>
struct CursorOf<PackedLists> {
    using type = PackedListCursor;
};
template <>
struct CursorOf<GridLists> {
    using type = PackedCursor;
};



// Stages the tile [j0, j0 + cnt) (loaded into cur) in the wave's LDS row, zero-mass
// padded: the row is written and read by this wave only (LDS accesses of one wave
// execute in order), the wave barriers keep the compiler from moving them across.
__device__ __forceinline__ void stage_row(float4 *row, int lane, int cnt, const float4 &cur)
{
    const bool in = lane < cnt;
    __builtin_amdgcn_wave_barrier();
    row[lane] = make_float4(in ? cur.x : 0.0f, in ? cur.y : 0.0f, in ? cur.z : 0.0f,
                            in ? cur.w : 0.0f);
    __builtin_amdgcn_wave_barrier();
}

// Runs eval(cnt) for every source tile of the target cell's walk that falls to wave w
// of W (tiles w, w + W, ...), with the tile's cnt bodies staged in the wave's LDS row
// (zero-mass padded). Each wave issues the global load of its next tile before it
// evaluates the current one. CSR lists are walked segment by segment: every wave of
// the workgroup passes the same barriers (segment count and bound segment are
// uniform), so wave 0 may rewrite the segment table; a one-segment list stays bound
// for the cell's later chunks.
template <int W, typename Lists, typename F>
__device__ __forceinline__ void walk_tiles(const P2PArgs &k, Lists &lists, int lo, int hi, int w,
                                           int lane, float4 *row, F &&eval)
{
    using Cursor = typename CursorOf<Lists>::type;
    int nseg = 1;
    if constexpr (__is_same(Lists, PackedLists)) nseg = lists.segments(lo, hi);
    for (int sg = 0; sg < nseg; ++sg) {
        if constexpr (__is_same(Lists, PackedLists)) {
            if (lists.bound_seg != sg) {
                __syncthreads();  // every wave is done with the previous table
                if (kRaceProbe && w == 0) {
                    // race probe: an empty table first (in-bounds for any reader: every
                    // position maps to itself, and a reader of the total sees no tiles)
                    for (int i = lane; i < kPackLds; i += 64) lists.tab[i] = 0;
                    __builtin_amdgcn_wave_barrier();
                }
                if (w == 0) lists.load_segment(k, lo, hi, sg, lane);
                __syncthreads();
                lists.bound_seg = sg;
            }
        }
        Cursor cs;
        cs.start(k, lists, lo, hi, w);
        float4 cur = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        if (cs.have) cur = cs.load(k, lane);
        while (cs.have) {
            const int cnt = cs.count();
            stage_row(row, lane, cnt, cur);
            Cursor nx = cs;
            nx.next(k, lists, W);
            if (nx.have) cur = nx.load(k, lane);
            eval(cnt);
            cs = nx;
        }
    }
}

// One lane's share of a full 64-body tile in one-target chunks of G source groups: the
// sources r[0], r[G], r[2G], ... (r = the row plus the lane's group), 64 / G of them; a
// compile-time G puts every LDS read at an immediate offset.
template <int G, bool POT>
__device__ __forceinline__ void full_tile_sources(const float4 *r, const Targets<1> &tg,
                                                  float eps2, Sums<1, POT> &blk)
{
#pragma unroll 16
    for (int u = 0; u < 64 / G; ++u) interact4<1, POT>(r[u * G], tg, eps2, blk);
}

// Targets per chunk (chunk_span): a cell's bodies go 64 at a time; a chunk of tw < 64 targets
// has tw lanes per source group and G = 64 / tw groups, lane (t, g) = (lane mod tw,
// lane / tw) summing every G-th source of each of its tiles for target t; the G
// group sums of a target are added in ascending g. So a 20-body cell keeps 64 lanes
// busy instead of 20. A lane's terms go into an fp32 partial of at most kFlush
// sources, then into the compensated totals (after every tile this cost a 4-body
// cell's lanes more than their four terms per tile). Each wave issues the global
// load of its next source tile before it evaluates the current one.
// Occupancy: the one-target kernels ask for eight waves per SIMD (at most 64 VGPRs).
// Left alone, the compiler gave the CSR-list variants 116-122 VGPRs (four waves per
// SIMD), loading a whole 16-source unroll of LDS reads ahead of the arithmetic; capped
// they take 59-64 and no scratch (octree leaves of 32 bodies: 0.31 -> 0.24 ms).
template <bool POT, typename Lists, int W>
__global__ void __launch_bounds__(64 * W, 8) p2p_kernel(P2PArgs k, Lists lists)
{
    __shared__ float4 rows[W][64];
    __shared__ float4 red[W][64];  // each wave's per-(target, group) sums of the chunk
    __shared__ int nbr[kGridLds > kPackLds ? kGridLds : kPackLds];  // the lists' LDS table
    const int c = lists.cell((int)blockIdx.x), lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int tb = k.cell_start[c], te = k.cell_start[c + 1];
    if (tb < 0 || te < tb || te > k.n) return;
    // workgroup blockIdx.y of the cell's gridDim.y takes its chunks q with
    // q mod gridDim.y == blockIdx.y; it exits at once when it has none
    const int ny = (int)gridDim.y, y = (int)blockIdx.y;
    if (y > 0 && !cell_has_chunk(te - tb, y)) return;
    if constexpr (__is_same(Lists, GridLists)) lists.nbr = nbr;
    if constexpr (__is_same(Lists, PackedLists)) lists.tab = nbr;
    lists.bind(k, c);
    int lo, hi;
    lists.range(c, lo, hi);
    const float eps2 = in_vgpr(k.eps2);
    float4 *row = rows[w];
    for (int t0 = tb, q = 0; t0 < te; ++q) {
        const int rem = te - t0;
        const bool mine = q % ny == y;
        int lg;
        const int span = chunk_span(rem, lg);
        if (!mine) {
            t0 += span;
            continue;
        }
        const int tw = span;
        const int groups = 64 >> lg;
        const int t = lane & (tw - 1), g = lane >> lg;
        const int i = t0 + t;
        const float4 me = k.pos[i < te ? i : te - 1];
        Targets<1> tg;
        tg.x[0] = me.x;
        tg.y[0] = me.y;
        tg.z[0] = me.z;
        Total<1, POT> tot;
        zero(tot);
        // a lane's sources go into blk, at most kFlush of them, then into tot: a tile
        // gives a lane cnt / groups of them
        Sums<1, POT> blk;
        zero(blk);
        int held = 0;
        const int per_tile = tw;  // at most 64 / groups = tw sources per tile
        walk_tiles<W>(k, lists, lo, hi, w, lane, row, [&](int cnt) {
            if (cnt == 64) {
                // full tile: the lane's sources at constant offsets from row + g
                switch (groups) {
                case 1: full_tile_sources<1, POT>(row, tg, eps2, blk); break;
                case 2: full_tile_sources<2, POT>(row + g, tg, eps2, blk); break;
                case 4: full_tile_sources<4, POT>(row + g, tg, eps2, blk); break;
                case 8: full_tile_sources<8, POT>(row + g, tg, eps2, blk); break;
                case 16: full_tile_sources<16, POT>(row + g, tg, eps2, blk); break;
                case 32: full_tile_sources<32, POT>(row + g, tg, eps2, blk); break;
                default: full_tile_sources<64, POT>(row + g, tg, eps2, blk); break;
                }
            } else {
#pragma unroll 4
                for (int u0 = 0; u0 < cnt; u0 += groups)
                    interact4<1, POT>(row[u0 + g], tg, eps2, blk);
            }
            held += per_tile;
            if (held > kFlush - per_tile) {
                add_into(tot, blk);
                zero(blk);
                held = 0;
            }
        });
        add_into(tot, blk);
        const Sums<1, POT> r = result(tot);
        float4 a = make_float4(r.ax[0], r.ay[0], r.az[0], POT ? r.p[0] : 0.0f);
        if constexpr (W > 1) {
            red[w][lane] = a;
            __syncthreads();
            // the W wave sums of each (target, group) in wave order
            a = red[0][lane];
#pragma unroll
            for (int ww = 1; ww < W; ++ww) {
                const float4 v = red[ww][lane];
                a = make_float4(a.x + v.x, a.y + v.y, a.z + v.z, a.w + v.w);
            }
        }
        if (w == 0) {
            // the groups of each target in ascending g, through wave 0's own row
            __builtin_amdgcn_wave_barrier();
            row[lane] = a;
            __builtin_amdgcn_wave_barrier();
            if (g == 0 && i < te) {
                float4 s = row[t];
                for (int gg = 1; gg < groups; ++gg) {
                    const float4 v = row[t + gg * tw];
                    s = make_float4(s.x + v.x, s.y + v.y, s.z + v.z, s.w + v.w);
                }
                const int o = k.out_index ? k.out_index[i] : i;
                k.acc_out[o] = make_float4(s.x, s.y, s.z, 0.0f);
                if constexpr (POT) k.pot_out[o] = -s.w;
            }
        }
        if constexpr (W > 1) {
            __syncthreads();  // red is refilled by the next chunk
            probe_poison(red[w][lane]);
        }
        t0 += tw;
    }
}

__device__ __forceinline__ int grid_axis(float x, float lo, float inv_h, int dim)
{
    float f = floorf((x - lo) * inv_h);
    if (!(f >= 0.0f)) f = 0.0f;
    if (f > (float)(dim - 1)) f = (float)(dim - 1);
    return (int)f;
}

// ---------------------------------------------------------------- near grid, pair-symmetric
// Each unordered pair of neighbouring cells {c, c + dir} is evaluated once, by the
// cell with the lower linear index (its owner), and applied to both cells'
// bodies, as the band pairs of the all-pairs kernel are; a cell's own pairs are
// evaluated one-sided. The 13 forward directions (dx, dy, dz), those with dz > 0,
// or dz = 0 and dy > 0, or dz = dy = 0 and dx > 0, are numbered
//   k = 0: (+1, 0, 0);  k = 1..3: (k - 2, +1, 0);  k = 4..12: ((k-4) % 3 - 1, (k-4) / 3 - 1, +1)
// and form five runs of consecutive cells (x fastest in the linear index): run 0
// = direction 0, run 1 = directions 1..3, run 2 + r = directions 4 + 3r .. 6 + 3r,
// each clipped to the grid. A body of cell c holds 14 partial sums: slot 0 from
// its own cell's workgroup (its cell one-sided and its side of the cell's forward
// pairs), slot 1 + k from the workgroup of the cell c - dir_k (its side of that
// pair), written once each; the finish adds the slots that exist in that order.
constexpr int kSymRuns = 5;
constexpr int kSymDirs = 13;

__host__ __device__ constexpr int sym_dir_dx(int k) { return k == 0 ? 1 : (k < 4 ? k - 2 : (k - 4) % 3 - 1); }
__host__ __device__ constexpr int sym_dir_dy(int k) { return k == 0 ? 0 : (k < 4 ? 1 : (k - 4) / 3 - 1); }
__host__ __device__ constexpr int sym_dir_dz(int k) { return k < 4 ? 0 : 1; }

// Launch index b -> owner cell: with heavy, first the cells whose forward
// neighbourhood is whole (1 <= x <= dx-2, 1 <= y <= dy-2, z <= dz-2: 13
// neighbour cells), then the others in natural order, so that the smaller
// neighbourhoods fill the CUs at the end of the launch. A bijection of
// [0, dx*dy*dz); the identity without heavy or below 3 x 3 x 2 cells.
__host__ __device__ inline int sym_cell(int b, int dx, int dy, int dz, bool heavy)
{
    const int ix = dx - 2, iy = dy - 2, iz = dz - 1;
    if (!heavy || ix < 1 || iy < 1 || iz < 1) return b;
    const int ni = ix * iy * iz;
    if (b < ni) return ((b / (ix * iy)) * dy + 1 + (b / ix) % iy) * dx + 1 + b % ix;
    int k = b - ni;
    const int per = 2 * dx + 2 * iy;  // other cells of a plane z <= dz-2: rows y = 0, dy-1, ends x = 0, dx-1
    if (k < per * iz) {
        const int z = k / per;
        int r = k % per, y, x;
        if (r < dx) {
            y = 0;
            x = r;
        } else if ((r -= dx) < 2 * iy) {
            y = 1 + r / 2;
            x = (r & 1) ? dx - 1 : 0;
        } else {
            y = dy - 1;
            x = r - 2 * iy;
        }
        return (z * dy + y) * dx + x;
    }
    k -= per * iz;  // the last plane, whole
    return ((dz - 1) * dy + k / dx) * dx + k % dx;
}

// Run t (0..4) of owner cell (cx, cy, cz) on a dx x dy x dz grid: the row (y, z)
// of its cells, their x range [xf, xl] and the direction k0 of cell xf; false when
// the run holds no cell of the grid.
__host__ __device__ inline bool sym_run(int t, int cx, int cy, int cz, int dx, int dy, int dz,
                                        int &y, int &z, int &xf, int &xl, int &k0)
{
    y = cy;
    z = cz;
    xf = cx + 1;
    xl = cx + 1;
    k0 = 0;
    if (t == 1) {
        y = cy + 1;
        xf = cx - 1;
        k0 = 1;
    } else if (t >= 2) {
        y = cy + (t - 2) - 1;
        z = cz + 1;
        xf = cx - 1;
        k0 = 4 + 3 * (t - 2);
    }
    if (xf < 0) {
        k0 -= xf;
        xf = 0;
    }
    if (xl > dx - 1) xl = dx - 1;
    return y >= 0 && y < dy && z < dz && xf <= xl;
}

struct SymShared {
    float4 jblk[4][kRowLen];  // each wave's copy of its current block; with jsum,
                              // between i-sets, the running cross-wave sum
    float4 jsum[4][kRowLen];  // each wave's partner sums of that block
    int sb[kSymRuns];         // body range [sb, sb + len) of each run (len 0 outside the grid)
    int pre[kSymRuns + 1];    // prefix of the run lengths
    int b1[kSymRuns], b2[kSymRuns];  // first body of the run's second and third cell (INT_MAX: none)
    int k0[kSymRuns];         // direction of the run's first cell
};

static_assert(kSymSlots == 1 + kSymDirs, "one own slot and one per forward direction");

struct SymArgs {
    const float4 *pos;      // N bodies grouped by cell (cell order)
    int n;
    float eps2;
    const int *cell_start;  // ncell + 1 entries
    int dims[3];
    int heavy_first;
    float4 *part;           // 14 slots of N records: part[slot * N + i]
};

// One i-set of R rows of 64 owner targets [i0, i0 + 64 R) (past o1: zero mass):
// the owner cell one-sided, then the forward sequence in pairs; the targets'
// sums go to own slot 0, the forward bodies' sums to their direction slots
// (stored on the first i-set, added to on later ones by the same thread).
template <int R, bool POT>
__device__ __forceinline__ void sym_iset(const SymArgs &k, SymShared &sh, int i0, int o0, int o1,
                                         bool first, float eps2)
{
    constexpr int W = 4;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int row = w * (int)sizeof(sh.jblk[0]);
    float tx[R], ty[R], tz[R], tm[R], ax[R], ay[R], az[R], ap[R];
#pragma unroll
    for (int t = 0; t < R; ++t) {
        const int b = i0 + t * 64 + lane;
        const float4 v = k.pos[b < o1 ? b : o1 - 1];
        const bool in = b < o1;
        tx[t] = in ? v.x : 0.0f;
        ty[t] = in ? v.y : 0.0f;
        tz[t] = in ? v.z : 0.0f;
        tm[t] = in ? v.w : 0.0f;
        ax[t] = ay[t] = az[t] = ap[t] = 0.0f;
    }
    // the owner cell against itself, one-sided (self pairs included)
    const int no = o1 - o0;
    for (int jb = w; jb * 64 < no; jb += W) {
        const int b = o0 + jb * 64 + lane;
        const float4 v = k.pos[b < o1 ? b : o1 - 1];
        const float4 jbody = b < o1 ? v : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        __builtin_amdgcn_wave_barrier();
        sh.jblk[w][lane] = jbody;
        __builtin_amdgcn_wave_barrier();
        block_pass<R, POT, false, 2>(&sh.jblk[0][0], &sh.jsum[0][0], row, lane, jbody, tx, ty, tz,
                                     tm, eps2, ax, ay, az, ap);
    }
    // the forward sequence, pair-symmetric
    const int total = sh.pre[kSymRuns];
    for (int jb = w; jb * 64 < total; jb += W) {
        const int p = jb * 64 + lane;
        int e = 0;
#pragma unroll
        for (int r = 1; r < kSymRuns; ++r) e += p >= sh.pre[r] ? 1 : 0;
        const int b = sh.sb[e] + (p - sh.pre[e]);
        const bool in = p < total;
        const float4 v = k.pos[in ? b : 0];
        const float4 jbody = in ? v : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        __builtin_amdgcn_wave_barrier();
        sh.jblk[w][lane] = jbody;
        sh.jsum[w][lane] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        __builtin_amdgcn_wave_barrier();
        block_pass<R, POT, true, 2>(&sh.jblk[0][0], &sh.jsum[0][0], row, lane, jbody, tx, ty, tz,
                                    tm, eps2, ax, ay, az, ap);
        const float4 g = sh.jsum[w][lane];
        if (in) {
            const int dir = sh.k0[e] + (b >= sh.b1[e] ? 1 : 0) + (b >= sh.b2[e] ? 1 : 0);
            float4 *dst = k.part + (size_t)(1 + dir) * (size_t)k.n + b;
            float4 o = first ? make_float4(0.0f, 0.0f, 0.0f, 0.0f) : *dst;
            o.x -= g.x;
            o.y -= g.y;
            o.z -= g.z;
            o.w += g.w;
            *dst = o;
        }
    }
    // the targets' sums across the waves, in wave order, through the block and sum rows
    float4 *red = &sh.jblk[0][0];
    __syncthreads();
    for (int ww = 0; ww < W; ++ww) {
        if (w == ww) {
#pragma unroll
            for (int t = 0; t < R; ++t) {
                const int idx = t * 64 + lane;
                float4 v = make_float4(ax[t], ay[t], az[t], ap[t]);
                if (ww > 0) {
                    const float4 q = red[idx];
                    v = make_float4(q.x + v.x, q.y + v.y, q.z + v.z, q.w + v.w);
                }
                if (ww < W - 1) {
                    red[idx] = v;
                } else if (i0 + idx < o1) {
                    k.part[i0 + idx] = v;
                }
            }
        }
        __syncthreads();
    }
    probe_poison(sh.jblk[w][lane]);
    probe_poison(sh.jsum[w][lane]);
}

// One workgroup per owner cell (launch order: sym_cell), 256 threads.
template <bool POT>
__global__ void __launch_bounds__(256) p2p_sym_kernel(SymArgs k)
{
    __shared__ SymShared sh;
    const int dx = k.dims[0], dy = k.dims[1], dz = k.dims[2];
    const int c = sym_cell((int)blockIdx.x, dx, dy, dz, k.heavy_first != 0);
    const int o0 = k.cell_start[c], o1 = k.cell_start[c + 1];
    if (o1 <= o0) return;  // an empty cell owns no pairs (uniform, before any barrier)
    const int cx = c % dx, cy = (c / dx) % dy, cz = c / (dx * dy);
    const int t = threadIdx.x;
    if (t < kSymRuns) {
        int y, z, xf, xl, k0;
        const bool in = sym_run(t, cx, cy, cz, dx, dy, dz, y, z, xf, xl, k0);
        const int rowc = (z * dy + y) * dx;
        const int sb = in ? k.cell_start[rowc + xf] : 0;
        const int se = in ? k.cell_start[rowc + xl + 1] : 0;
        sh.sb[t] = sb;
        sh.pre[t + 1] = se - sb;  // lengths; prefix below
        sh.b1[t] = in && xf + 1 <= xl ? k.cell_start[rowc + xf + 1] : INT_MAX;
        sh.b2[t] = in && xf + 2 <= xl ? k.cell_start[rowc + xf + 2] : INT_MAX;
        sh.k0[t] = k0;
    }
    __syncthreads();
    if (t == 0) {
        sh.pre[0] = 0;
        for (int r = 0; r < kSymRuns; ++r) sh.pre[r + 1] += sh.pre[r];
    }
    __syncthreads();
    const float eps2 = in_vgpr(k.eps2);
    for (int i0 = o0; i0 < o1; i0 += 512) {
        const int rows = min(8, (o1 - i0 + 63) / 64);
        const bool first = i0 == o0;
        switch (rows) {
        case 1: sym_iset<1, POT>(k, sh, i0, o0, o1, first, eps2); break;
        case 2: sym_iset<2, POT>(k, sh, i0, o0, o1, first, eps2); break;
        case 3: sym_iset<3, POT>(k, sh, i0, o0, o1, first, eps2); break;
        case 4: sym_iset<4, POT>(k, sh, i0, o0, o1, first, eps2); break;
        case 5: sym_iset<5, POT>(k, sh, i0, o0, o1, first, eps2); break;
        case 6: sym_iset<6, POT>(k, sh, i0, o0, o1, first, eps2); break;
        case 7: sym_iset<7, POT>(k, sh, i0, o0, o1, first, eps2); break;
        default: sym_iset<8, POT>(k, sh, i0, o0, o1, first, eps2); break;
        }
    }
}

// Body i (cell order, cell from its sorted key): slot 0, then slot 1 + k for each
// direction k whose owner cell (its cell - dir_k) lies in the grid and holds
// bodies, in compensated sums; the results go to row out_index[i].
__global__ void __launch_bounds__(256) sym_finish_kernel(const float4 *__restrict__ part, int n,
                                                         const unsigned *__restrict__ cell_of,
                                                         const int *__restrict__ cell_start,
                                                         int dx, int dy, int dz,
                                                         const int *__restrict__ out_index,
                                                         float4 *__restrict__ acc_out,
                                                         float *__restrict__ pot_out)
{
    const unsigned i = blockIdx.x * 256u + threadIdx.x;
    if (i >= (unsigned)n) return;
    const int c = (int)cell_of[i];
    const int cx = c % dx, cy = (c / dx) % dy, cz = c / (dx * dy);
    // which slots exist, then all their loads, then the additions in slot order
    bool has[kSymDirs];
#pragma unroll
    for (int q = 0; q < kSymDirs; ++q) {
        const int ox = cx - sym_dir_dx(q), oy = cy - sym_dir_dy(q), oz = cz - sym_dir_dz(q);
        const bool in = ox >= 0 && ox < dx && oy >= 0 && oy < dy && oz >= 0;
        const int o = in ? (oz * dy + oy) * dx + ox : 0;
        has[q] = in && cell_start[o + 1] > cell_start[o];
    }
    float4 v[kSymDirs];
#pragma unroll
    for (int q = 0; q < kSymDirs; ++q)
        v[q] = has[q] ? part[(size_t)(1 + q) * (size_t)n + i] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    float4 a = part[i], e = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
    for (int q = 0; q < kSymDirs; ++q)
        if (has[q]) two_sum_add4(a, e, v[q]);
    const int r = out_index ? out_index[i] : (int)i;
    acc_out[r] = make_float4(a.x + e.x, a.y + e.y, a.z + e.z, 0.0f);
    if (pot_out) pot_out[r] = -(a.w + e.w);
}

__global__ void __launch_bounds__(256) grid_keys_kernel(const float4 *__restrict__ pos, int n,
                                                        GridSpec g, unsigned *__restrict__ keys,
                                                        int *__restrict__ idx)
{
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    const float4 b = pos[i];
    const int x = grid_axis(b.x, g.lo[0], g.inv_h, g.dims[0]);
    const int y = grid_axis(b.y, g.lo[1], g.inv_h, g.dims[1]);
    const int z = grid_axis(b.z, g.lo[2], g.inv_h, g.dims[2]);
    keys[i] = (unsigned)((z * g.dims[1] + y) * g.dims[0] + x);
    idx[i] = i;
}

__global__ void __launch_bounds__(256) gather_kernel(const float4 *__restrict__ pos,
                                                     const int *__restrict__ perm, int n,
                                                     float4 *__restrict__ out)
{
    const int k = blockIdx.x * 256 + threadIdx.x;
    if (k < n) out[k] = pos[perm[k]];
}

__global__ void __launch_bounds__(256) cell_starts_kernel(const unsigned *__restrict__ keys, int n,
                                                          int ncell, int *__restrict__ start)
{
    const int c = blockIdx.x * 256 + threadIdx.x;
    if (c > ncell) return;
    int a = 0, b = n;  // first k in [a, b) with keys[k] >= c
    while (a < b) {
        const int m = a + (b - a) / 2;
        if (keys[m] < (unsigned)c) a = m + 1;
        else b = m;
    }
    start[c] = a;
}

// ---------------------------------------------------------------- binning sort
// Stable LSD radix sort of (key, body index) pairs (the cell keys of nbody_near_grid,
// the Morton keys of nbody_near_tree), 8 key bits per pass, three steps per pass:
//   hist    - workgroup b counts the digits of its contiguous key range
//             [b per, (b + 1) per) into counts[digit][b] (LDS counters: the
//             counts do not depend on the order of the additions);
//   scan    - counts become exclusive offsets in digit-major order (digit,
//             then workgroup), so equal digits keep the order of the
//             workgroups, i.e. of the input (two kernels: tile sums, then each
//             tile scanned from the sum of the tiles before it);
//   scatter - workgroup b ranks its range in input order, restages each chunk
//             in LDS in digit order and writes each digit's run from its offset
//             (below).
// Every step is integer and in a fixed order: the result is the stable sort,
// the same bits every time, so a cell keeps its bodies in input order.
constexpr int kSortBits = 8;
constexpr int kSortDigits = 1 << kSortBits;  // 256: one counter per thread
constexpr int kSortMaxBlocks = 2048;         // counts <= 2^19 entries: <= 128 scan tiles
constexpr int kSortScanThreads = 1024;
constexpr int kSortScanTile = 4 * kSortScanThreads;  // counts per scan workgroup
constexpr int kSortKeysPerBlock = 4096;      // most keys per workgroup (up to N = 2^23)
constexpr int kSortMinKeysPerBlock = 1024;   // fewest keys per workgroup
constexpr int kSortTargetBlocks = 512;

struct SortShape {
    int nblocks;  // workgroups per pass
    int per;      // keys per workgroup (a multiple of 256; the last range may be shorter)
};

SortShape sort_shape(int n)
{
    // about kSortTargetBlocks workgroups of 1024 to 4096 keys (measured: 1024 keys per
    // workgroup at N = 2^16 and 300,007 bodies, 2048 at 2^20)
    long long want = (long long)n / kSortTargetBlocks;
    want = want < kSortMinKeysPerBlock ? kSortMinKeysPerBlock
                                       : (want > kSortKeysPerBlock ? kSortKeysPerBlock : want);
    int nb = (int)(((long long)n + want - 1) / want);
    if (nb > kSortMaxBlocks) nb = kSortMaxBlocks;
    if (nb < 1) nb = 1;
    long long per = ((long long)n + nb - 1) / nb;
    per = (per + 255) / 256 * 256;
    nb = (int)(((long long)n + per - 1) / per);
    return {nb < 1 ? 1 : nb, (int)per};
}

__device__ __forceinline__ void sort_range(int n, int per, int &b0, int &e)
{
    const long long a = (long long)blockIdx.x * per;
    const long long z = a + per;
    b0 = (int)a;
    e = (int)(z < n ? z : n);
}

template <typename K>
__global__ void __launch_bounds__(256) sort_hist_kernel(const K *__restrict__ keys, int n,
                                                        int per, int shift, int nblocks,
                                                        int *__restrict__ counts)
{
    __shared__ int h[kSortDigits];
    h[threadIdx.x] = 0;
    __syncthreads();
    int b0, e;
    sort_range(n, per, b0, e);
    for (int i = b0 + (int)threadIdx.x; i < e; i += 256)
        atomicAdd(&h[(unsigned)(keys[i] >> shift) & (kSortDigits - 1)], 1);
    __syncthreads();
    counts[threadIdx.x * nblocks + blockIdx.x] = h[threadIdx.x];
}

// Exclusive prefix sum of counts[0 .. total) in place, in tiles of 4096 entries, one
// workgroup per tile: sort_tile_sums_kernel adds up each tile, then sort_scan_kernel
// scans its tile from the sum of the tiles before it (a coalesced load of the tile
// into LDS, each thread the sum of four consecutive entries, an inclusive scan of
// those over the wave by shuffles, the 16 wave totals added in wave order, the four
// exclusive prefixes written back through LDS). Integer sums: the result is exact.
// Sum over the workgroup of v (one value per thread), in a fixed order; every thread
// gets it. red holds kSortScanThreads / 64 ints.
__device__ __forceinline__ int sort_block_sum(int v, int *red)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    if (lane == 0) red[w] = v;
    __syncthreads();
    int s = 0;
    for (int q = 0; q < kSortScanThreads / 64; ++q) s += red[q];
    return s;
}

__global__ void __launch_bounds__(kSortScanThreads)
    sort_tile_sums_kernel(const int *__restrict__ counts, int total, int *__restrict__ tile_sums)
{
    __shared__ int red[kSortScanThreads / 64];
    const int base = blockIdx.x * kSortScanTile, t = threadIdx.x;
    int v = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int i = base + k * kSortScanThreads + t;
        v += i < total ? counts[i] : 0;
    }
    const int s = sort_block_sum(v, red);
    if (t == 0) tile_sums[blockIdx.x] = s;
}

__global__ void __launch_bounds__(kSortScanThreads)
    sort_scan_kernel(int *__restrict__ counts, int total, const int *__restrict__ tile_sums)
{
    __shared__ int4 buf[kSortScanThreads];  // the tile's kSortScanTile entries
    __shared__ int wsum[kSortScanThreads / 64];
    __shared__ int red[kSortScanThreads / 64];
    int *flat = reinterpret_cast<int *>(buf);
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int base = blockIdx.x * kSortScanTile;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int i = base + k * kSortScanThreads + t;
        flat[k * kSortScanThreads + t] = i < total ? counts[i] : 0;
    }
    // the tiles before this one (at most kSortScanThreads of them)
    const int carry = sort_block_sum(t < (int)blockIdx.x ? tile_sums[t] : 0, red);
    const int4 v = buf[t];  // entries 4t .. 4t + 3 of the tile (published by the barrier above)
    const int sum = v.x + v.y + v.z + v.w;
    int incl = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o);
        if (lane >= o) incl += y;
    }
    if (lane == 63) wsum[w] = incl;
    __syncthreads();
    int before = carry;
    for (int q = 0; q < w; ++q) before += wsum[q];
    const int e = before + incl - sum;
    buf[t] = make_int4(e, e + v.x, e + v.x + v.y, e + v.x + v.y + v.z);
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int i = base + k * kSortScanThreads + t;
        if (i < total) counts[i] = flat[k * kSortScanThreads + t];
    }
}

// Scatter: workgroup b places its range chunk by chunk (kSortChunk keys, 256 per
// round). A round ranks its keys in input order (the eight digit-bit ballots give a
// lane's place among the wave's keys of its digit, the per-wave counts in LDS the
// place among earlier waves', the running count the place among earlier rounds'),
// and the chunk is restaged in LDS in digit order; then consecutive threads write
// consecutive entries of each digit's run, so the global writes come in runs of
// about chunk / 256 keys instead of one key per address. Stable, integer, fixed
// order: the same bits every time.
constexpr int kSortChunk = 2048;
constexpr int kSortRounds = kSortChunk / 256;

template <typename K>
__global__ void __launch_bounds__(256) sort_scatter_kernel(const K *__restrict__ kin,
                                                           const int *__restrict__ vin, int n,
                                                           int per, int shift, int nblocks,
                                                           const int *__restrict__ offsets,
                                                           K *__restrict__ kout,
                                                           int *__restrict__ vout)
{
    __shared__ int base[kSortDigits];     // global position of each digit's next key
    __shared__ int run[kSortDigits];      // keys of each digit in the chunk so far
    __shared__ int lstart[kSortDigits];   // each digit's first slot in the restaged chunk
    __shared__ int wcnt[4][kSortDigits];  // per wave: keys of each digit in the round
    __shared__ int wsum[4];
    __shared__ K skey[kSortChunk];
    __shared__ int sval[kSortChunk];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    base[tid] = offsets[tid * nblocks + blockIdx.x];
#pragma unroll
    for (int q = 0; q < 4; ++q) wcnt[q][tid] = 0;
    int b0, e;
    sort_range(n, per, b0, e);
    for (int c0 = b0; c0 < e; c0 += kSortChunk) {
        const int cnt = e - c0 < kSortChunk ? e - c0 : kSortChunk;
        run[tid] = 0;
        K key[kSortRounds];
        int val[kSortRounds], rank[kSortRounds];
        unsigned dig[kSortRounds];
#pragma unroll
        for (int r = 0; r < kSortRounds; ++r) {  // all loads first
            const int i = c0 + r * 256 + tid;
            const bool valid = r * 256 + tid < cnt;
            key[r] = valid ? kin[i] : K(0);
            val[r] = valid ? vin[i] : 0;
        }
        __syncthreads();
#pragma unroll
        for (int r = 0; r < kSortRounds; ++r) {
            if (r * 256 >= cnt) break;  // uniform
            const bool valid = r * 256 + tid < cnt;
            const unsigned d = (unsigned)(key[r] >> shift) & (kSortDigits - 1);
            dig[r] = d;
            unsigned long long same = __ballot(valid);
#pragma unroll
            for (int bit = 0; bit < kSortBits; ++bit) {
                const bool set = (d >> bit) & 1u;
                const unsigned long long on = __ballot(set);
                same &= set ? on : ~on;
            }
            const unsigned long long below = same & ((1ull << lane) - 1ull);
            if (valid && below == 0) wcnt[w][d] = __popcll(same);  // the digit's first lane
            __syncthreads();
            int at = run[d] + __popcll(below);
            for (int q = 0; q < w; ++q) at += wcnt[q][d];
            rank[r] = at;
            __syncthreads();
            run[tid] += wcnt[0][tid] + wcnt[1][tid] + wcnt[2][tid] + wcnt[3][tid];
#pragma unroll
            for (int q = 0; q < 4; ++q) wcnt[q][tid] = 0;
            __syncthreads();
        }
        // each digit's first slot in the chunk: exclusive scan of run over the digits
        const int mine = run[tid];
        int incl = mine;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(incl, o);
            if (lane >= o) incl += y;
        }
        if (lane == 63) wsum[w] = incl;
        __syncthreads();
        int before = 0;
        for (int q = 0; q < w; ++q) before += wsum[q];
        lstart[tid] = before + incl - mine;
        __syncthreads();
#pragma unroll
        for (int r = 0; r < kSortRounds; ++r) {
            if (r * 256 >= cnt) break;
            if (r * 256 + tid < cnt) {
                const int slot = lstart[dig[r]] + rank[r];
                if (slot < cnt) {
                    skey[slot] = key[r];
                    sval[slot] = val[r];
                }
            }
        }
        __syncthreads();
        for (int sl = tid; sl < cnt; sl += 256) {
            const K k = skey[sl];
            const unsigned d = (unsigned)(k >> shift) & (kSortDigits - 1);
            const int g = base[d] + sl - lstart[d];
            if (g >= 0 && g < n) {
                kout[g] = k;
                vout[g] = sval[sl];
            }
        }
        __syncthreads();  // base, run and the staging area are rewritten by the next chunk
        base[tid] += mine;
    }
}

// ---------------------------------------------------------------- prefix sums
// Exclusive prefix sum of any int array in place, tile by tile (4096 entries per
// workgroup, the layout of sort_scan_kernel), each tile starting from an offset
// given by the exclusive sums of the tile totals (scanned the same way, so any
// length below 2^31 works). The last thread of the last tile writes the total.
__global__ void __launch_bounds__(kSortScanThreads)
    scan_tiles_kernel(int *__restrict__ data, int total, const int *__restrict__ offsets,
                      int *__restrict__ total_out)
{
    __shared__ int4 buf[kSortScanThreads];
    __shared__ int wsum[kSortScanThreads / 64];
    int *flat = reinterpret_cast<int *>(buf);
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int base = blockIdx.x * kSortScanTile;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int i = base + k * kSortScanThreads + t;
        flat[k * kSortScanThreads + t] = i < total ? data[i] : 0;
    }
    __syncthreads();
    const int carry = offsets ? offsets[blockIdx.x] : 0;
    const int4 v = buf[t];
    const int sum = v.x + v.y + v.z + v.w;
    int incl = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o);
        if (lane >= o) incl += y;
    }
    if (lane == 63) wsum[w] = incl;
    __syncthreads();
    int before = carry;
    for (int q = 0; q < w; ++q) before += wsum[q];
    const int e = before + incl - sum;
    buf[t] = make_int4(e, e + v.x, e + v.x + v.y, e + v.x + v.y + v.z);
    if (total_out && t == kSortScanThreads - 1 && blockIdx.x == gridDim.x - 1)
        *total_out = e + sum;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int i = base + k * kSortScanThreads + t;
        if (i < total) data[i] = flat[k * kSortScanThreads + t];
    }
}

// ---------------------------------------------------------------- octree leaves
// nbody_near_tree builds the leaves of an octree over the bodies and their
// interaction lists, then runs the near-field kernel over them. The tree is
// implicit in the Morton order: node (L, p) is the run of sorted keys whose top
// 3L bits (of 63) are p. Steps (each a kernel, every decision in float32 or
// integers):
//   bounds  - smallest and largest coordinate per axis (exact: min and max);
//   keys    - the 63-bit key of each body in the root cube, then the stable sort;
//   levels  - each sorted body's leaf level by bisection over L, with the size of
//             its node at level L found by two binary searches confined to the
//             leaf_size bodies on either side of it (a node reaching past them
//             holds more than leaf_size);
//   leaves  - the bodies where a leaf begins, scanned into leaf numbers; each
//             leaf's key, level and cube;
//   table   - for the cells of one coarse level, the first leaf at or after each,
//             so that a search for a key starts inside one cell's leaves;
//   lists   - one thread per (leaf A, cell q of the 27 of A's level around it): the
//             leaf that holds the whole cell q (listed once, from the first such
//             cell), or else the deeper leaves inside q whose cubes meet A's, found
//             by walking q's leaves in key order and skipping, past a leaf that
//             misses A, the largest subtree around it that misses A. Every leaf
//             meeting A's closed cube lies in or over one of the 27 cells. A count
//             pass and a fill pass run the same enumeration; leaf A's list is the
//             concatenation of its 27 parts in q order.
constexpr int kTreeBits = 21;  // levels below the root
constexpr int kTreeBoundsBlocks = 512;
using u64 = unsigned long long;

__device__ __forceinline__ u64 tree_spread(unsigned c)  // bit b of c -> bit 3b
{
    u64 r = 0;
#pragma unroll
    for (int b = 0; b < kTreeBits; ++b) r |= (u64)((c >> b) & 1u) << (3 * b);
    return r;
}

__device__ __forceinline__ int tree_gather(u64 k, int bits)  // bit 3b of k -> bit b
{
    unsigned r = 0;
    for (int b = 0; b < bits; ++b) r |= (unsigned)((k >> (3 * b)) & 1u) << b;
    return (int)r;
}

__device__ __forceinline__ unsigned tree_cell(float x, float lo, float inv)
{
    constexpr float top = (float)((1 << kTreeBits) - 1);
    float f = floorf((x - lo) * inv);
    if (!(f >= 0.0f)) f = 0.0f;
    if (f > top) f = top;
    return (unsigned)f;
}

__device__ __forceinline__ int tree_shift(int level) { return 3 * (kTreeBits - level); }

__device__ __forceinline__ u64 tree_key(int x, int y, int z, int level)  // cell start key
{
    return (tree_spread((unsigned)x) | (tree_spread((unsigned)y) << 1) |
            (tree_spread((unsigned)z) << 2)) << tree_shift(level);
}

__global__ void __launch_bounds__(256) tree_bounds_kernel(const float4 *__restrict__ pos, int n,
                                                          float *__restrict__ part)
{
    __shared__ float red[4][6];
    float v[6] = {INFINITY, INFINITY, INFINITY, -INFINITY, -INFINITY, -INFINITY};
    for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n;
         i += (long long)gridDim.x * 256) {
        const float4 b = pos[i];
        v[0] = fminf(v[0], b.x);
        v[1] = fminf(v[1], b.y);
        v[2] = fminf(v[2], b.z);
        v[3] = fmaxf(v[3], b.x);
        v[4] = fmaxf(v[4], b.y);
        v[5] = fmaxf(v[5], b.z);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
#pragma unroll
        for (int d = 0; d < 3; ++d) {
            v[d] = fminf(v[d], __shfl_xor(v[d], o));
            v[3 + d] = fmaxf(v[3 + d], __shfl_xor(v[3 + d], o));
        }
    }
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    if (lane == 0)
        for (int d = 0; d < 6; ++d) red[w][d] = v[d];
    __syncthreads();
    if (threadIdx.x < 6) {
        const int d = threadIdx.x;
        float r = red[0][d];
        for (int q = 1; q < 4; ++q) r = d < 3 ? fminf(r, red[q][d]) : fmaxf(r, red[q][d]);
        part[blockIdx.x * 6 + d] = r;
    }
}

__global__ void __launch_bounds__(64) tree_frame_kernel(const float *__restrict__ part, int nparts,
                                                        float4 *__restrict__ frame,
                                                        int *__restrict__ counters)
{
    float v[6] = {INFINITY, INFINITY, INFINITY, -INFINITY, -INFINITY, -INFINITY};
    for (int b = threadIdx.x; b < nparts; b += 64)
        for (int d = 0; d < 6; ++d)
            v[d] = d < 3 ? fminf(v[d], part[b * 6 + d]) : fmaxf(v[d], part[b * 6 + d]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
#pragma unroll
        for (int d = 0; d < 3; ++d) {
            v[d] = fminf(v[d], __shfl_xor(v[d], o));
            v[3 + d] = fmaxf(v[3 + d], __shfl_xor(v[3 + d], o));
        }
    }
    if (threadIdx.x < kTreeCounters) counters[threadIdx.x] = 0;
    if (threadIdx.x == 0) {
        float side = 0.0f;
        for (int d = 0; d < 3; ++d) {
            const float ext = v[3 + d] - v[d];
            if (ext > side) side = ext;
        }
        if (!(side > 0.0f)) side = 1.0f;
        frame[0] = make_float4(v[0], v[1], v[2], (float)(1 << kTreeBits) / side);
    }
}

__global__ void __launch_bounds__(256) tree_keys_kernel(const float4 *__restrict__ pos, int n,
                                                        const float4 *__restrict__ frame,
                                                        u64 *__restrict__ keys,
                                                        int *__restrict__ idx)
{
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    const float4 f = frame[0];
    const float4 b = pos[i];
    keys[i] = tree_spread(tree_cell(b.x, f.x, f.w)) | (tree_spread(tree_cell(b.y, f.y, f.w)) << 1) |
              (tree_spread(tree_cell(b.z, f.z, f.w)) << 2);
    idx[i] = i;
}

// Does the node at level L holding sorted body k have at most S bodies? Its first
// and last bodies are searched for among the S bodies before and after k only: a
// node reaching past them holds at least S + 1. key_at(m) reads sorted key m.
template <typename KeyAt>
__device__ __forceinline__ bool tree_node_fits(KeyAt key_at, int n, int k, u64 key, int L, int S)
{
    const int s = tree_shift(L);
    const u64 p = key >> s;
    int a = k - S > 0 ? k - S : 0, b = k;  // first index in [a, k] with prefix p
    while (a < b) {
        const int m = a + (b - a) / 2;
        if ((key_at(m) >> s) < p) a = m + 1;
        else b = m;
    }
    const long long hi = (long long)k + S + 1;
    int c = k + 1, d = hi < n ? (int)hi : n;  // first index in (k, k + S + 1) past the node
    while (c < d) {
        const int m = c + (d - c) / 2;
        if ((key_at(m) >> s) <= p) c = m + 1;
        else d = m;
    }
    return c - a <= S;
}

// Sorted body k begins its leaf (of level L) when the body before it lies in another
// node of that level.
__device__ __forceinline__ bool tree_leaf_begins(const u64 *__restrict__ keys, int k, int L)
{
    const int s = tree_shift(L);
    return k == 0 || (keys[k - 1] >> s) != (keys[k] >> s);
}

// Each sorted body's leaf level by bisection over L (node sizes shrink with L: the first
// L that fits). With WIN (leaf_size <= kTreeWinS) the workgroup first copies the keys its
// searches can reach, [k0 - S, k0 + 256 + S), into LDS, so that the ~2 x 5 x log2(S)
// dependent reads of each body come from LDS instead of the caches.
constexpr int kTreeWinS = 1024;

template <bool WIN>
__global__ void __launch_bounds__(256) tree_levels_kernel(const u64 *__restrict__ keys, int n,
                                                          int S, int *__restrict__ level,
                                                          int *__restrict__ start)
{
    __shared__ u64 win[WIN ? 256 + 2 * kTreeWinS : 1];
    const int k0 = blockIdx.x * 256, k = k0 + threadIdx.x;
    const int w0 = k0 - S > 0 ? k0 - S : 0;
    if constexpr (WIN) {
        const long long e = (long long)k0 + 256 + S;
        const int w1 = e < n ? (int)e : n;
        for (int i = w0 + threadIdx.x; i < w1; i += 256) win[i - w0] = keys[i];
        __syncthreads();
    }
    if (k >= n) return;
    auto key_at = [&](int m) -> u64 {
        if constexpr (WIN) return win[m - w0];
        else return keys[m];
    };
    const u64 key = key_at(k);
    int lo = 0, hi = kTreeBits;
    while (lo < hi) {
        const int L = (lo + hi) >> 1;
        if (tree_node_fits(key_at, n, k, key, L, S)) hi = L;
        else lo = L + 1;
    }
    level[k] = lo;
    const int s = tree_shift(lo);
    start[k] = k == 0 || (key_at(k - 1) >> s) != (key >> s) ? 1 : 0;  // as tree_leaf_begins
}

// Leaf A: cell_start[A] = its first sorted body, key (cleared below its level),
// box = (corner x, y, z in level-21 units, level).
__global__ void __launch_bounds__(256) tree_leaves_kernel(const u64 *__restrict__ keys,
                                                          const int *__restrict__ level,
                                                          const int *__restrict__ ids, int n,
                                                          int *__restrict__ cell_start,
                                                          u64 *__restrict__ leaf_key,
                                                          int4 *__restrict__ leaf_box)
{
    const int k = blockIdx.x * 256 + threadIdx.x;
    if (k >= n) return;
    const int L = level[k], s = tree_shift(L);
    const bool first = tree_leaf_begins(keys, k, L);
    const int a = ids[k];
    if (first) {
        const u64 p = keys[k] >> s;
        cell_start[a] = k;
        leaf_key[a] = p << s;
        const int sh = kTreeBits - L;
        leaf_box[a] = make_int4(tree_gather(p, L) << sh, tree_gather(p >> 1, L) << sh,
                                tree_gather(p >> 2, L) << sh, L);
    }
    if (k == n - 1) cell_start[a + (first ? 1 : 0)] = n;
}

// Coarse table: table[c] = first leaf whose key is at least the start of cell c of
// level lt, for c = 0 .. 8^lt (the last: nleaf).
__global__ void __launch_bounds__(256) tree_table_kernel(const u64 *__restrict__ leaf_key,
                                                         const int *__restrict__ counters,
                                                         int lt, int *__restrict__ table)
{
    const long long c = (long long)blockIdx.x * 256 + threadIdx.x;
    const long long cells = 1ll << (3 * lt);
    if (c > cells) return;
    const int nleaf = counters[0];
    if (c == cells) {
        table[c] = nleaf;
        return;
    }
    const u64 x = (u64)c << tree_shift(lt);
    int a = 0, b = nleaf;
    while (a < b) {
        const int m = a + (b - a) / 2;
        if (leaf_key[m] < x) a = m + 1;
        else b = m;
    }
    table[c] = a;
}

struct TreeIndex {
    const u64 *key;      // leaf keys, ascending
    const int4 *box;     // leaf cubes
    const int *table;    // coarse table over level lt
    int nleaf, lt;
    // first leaf in [a, b) with key >= x; b if none
    __device__ int lower_in(int a, int b, u64 x) const
    {
        while (a < b) {
            const int m = a + (b - a) / 2;
            if (key[m] < x) a = m + 1;
            else b = m;
        }
        return a;
    }
    // lower_in(a, b, x) found from a outwards: a, then a + 1, a + 2, a + 4, ... until a key
    // at or past x, then a binary search inside that step. A skipped subtree mostly ends
    // at the next leaf (94 % of the skips of a 65,536-body Plummer sphere at leaf size 64),
    // which this finds with one load instead of a search over the cell's whole key range
    // (the walk's chains of dependent loads were up to ~600 long there).
    __device__ int gallop(int a, int b, u64 x) const
    {
        if (a >= b || key[a] >= x) return a;
        int lo = a + 1, step = 1;
        while (lo < b && key[lo] < x) {
            a = lo;
            step <<= 1;
            lo = a + step < b ? a + step : b;
        }
        return lower_in(a + 1, lo, x);
    }
    // The first leaf with key > x (u) and the first with key >= y (l), as two interleaved
    // binary searches whose loads overlap; the leaves with keys in x's coarse cell c are
    // [table[c], table[c + 1]), so each search starts inside one cell.
    __device__ void upper_lower(u64 x, u64 y, int &u, int &l) const
    {
        const u64 cx = x >> tree_shift(lt), cy = y >> tree_shift(lt);
        int a0 = table[cx], b0 = table[cx + 1];
        int a1 = nleaf, b1 = nleaf;  // y = 2^63: past every key
        if (cy < (1ull << (3 * lt))) {
            a1 = table[cy];
            b1 = table[cy + 1];
        }
        while (a0 < b0 || a1 < b1) {
            const int m0 = a0 + (b0 - a0) / 2, m1 = a1 + (b1 - a1) / 2;
            const u64 k0 = a0 < b0 ? key[m0] : 0, k1 = a1 < b1 ? key[m1] : 0;
            if (a0 < b0) {
                if (k0 <= x) a0 = m0 + 1;
                else b0 = m0;
            }
            if (a1 < b1) {
                if (k1 < y) a1 = m1 + 1;
                else b1 = m1;
            }
        }
        u = a0;
        l = a1;
    }
};

// Do the closed cubes (o, level l) and A's (oa, size sa) meet? Coordinates in level-21 units.
__device__ __forceinline__ bool tree_meet(int ox, int oy, int oz, int l, const int (&oa)[3],
                                          int sa)
{
    const int sb = 1 << (kTreeBits - l);
    return ox <= oa[0] + sa && oa[0] <= ox + sb && oy <= oa[1] + sa && oa[1] <= oy + sb &&
           oz <= oa[2] + sa && oa[2] <= oz + sb;
}

// The count pass also keeps each part's first keep_cap entries in keep[t * keep_cap ..];
// the fill pass copies a part that fits from there and walks again only for longer ones.
template <bool FILL>
__global__ void __launch_bounds__(256) tree_lists_kernel(TreeIndex ix,
                                                         const int *__restrict__ cell_start,
                                                         longlong2 *__restrict__ part,
                                                         int *__restrict__ cnt,
                                                         const int *__restrict__ off,
                                                         int *__restrict__ list, int list_cap,
                                                         int *__restrict__ list_off,
                                                         int *__restrict__ keep, int keep_cap)
{
    const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
    const int nleaf = ix.nleaf;
    const bool live = t < 27ll * nleaf;
    if (!FILL && t == 27ll * nleaf) cnt[t] = 0;  // the entry past the last part
    int w = 0;
    long long terms = 0;
    if (live) {
        const int A = (int)(t / 27), q = (int)(t % 27);
        const int4 ba = ix.box[A];
        const int L = ba.w, s = tree_shift(L), lim = 1 << L, sh = kTreeBits - L;
        const int oa[3] = {ba.x, ba.y, ba.z};
        const int sa = 1 << sh;
        const int ca[3] = {ba.x >> sh, ba.y >> sh, ba.z >> sh};
        long long at = 0, end = 0;
        if (FILL) {
            at = off[t];
            end = off[t + 1] < list_cap ? off[t + 1] : list_cap;  // never past the buffer
            if (q == 0) list_off[A] = (int)at;
            if (A == nleaf - 1 && q == 26) list_off[nleaf] = (int)end;
        }
        auto emit = [&](int B) {
            if (FILL) {
                if (at + w < end) list[at + w] = B;
            } else {
                terms += cell_start[B + 1] - cell_start[B];
                if (w < keep_cap) keep[(size_t)t * keep_cap + w] = B;
            }
            ++w;
        };
        bool kept = false;
        if (FILL && keep_cap > 0) {
            const long long c = off[t + 1] - off[t];
            if (c <= keep_cap) {  // the count pass kept the whole part
                for (int i = 0; i < (int)c; ++i)
                    if (at + i < end) list[at + i] = keep[(size_t)t * keep_cap + i];
                kept = true;
            }
        }
        const int cq[3] = {ca[0] + q % 3 - 1, ca[1] + (q / 3) % 3 - 1, ca[2] + q / 9 - 1};
        if (!kept && cq[0] >= 0 && cq[1] >= 0 && cq[2] >= 0 && cq[0] < lim && cq[1] < lim &&
            cq[2] < lim) {
            const u64 qk = tree_key(cq[0], cq[1], cq[2], L);
            const u64 qe = qk + (1ull << s);
            int ub, E;
            ix.upper_lower(qk, qe, ub, E);
            const int b = ub - 1;
            const int4 bb = b >= 0 ? ix.box[b] : make_int4(0, 0, 0, kTreeBits + 1);
            if (bb.w <= L && qk < ix.key[b] + (1ull << tree_shift(bb.w))) {
                // leaf b holds the whole cell: listed from the first in-range cell inside it
                const int u = L - bb.w;
                bool seen = false;
                for (int r = 0; r < q && !seen; ++r) {
                    const int cr[3] = {ca[0] + r % 3 - 1, ca[1] + (r / 3) % 3 - 1,
                                       ca[2] + r / 9 - 1};
                    if (cr[0] < 0 || cr[1] < 0 || cr[2] < 0 || cr[0] >= lim || cr[1] >= lim ||
                        cr[2] >= lim)
                        continue;
                    seen = (cr[0] >> u) == (cq[0] >> u) && (cr[1] >> u) == (cq[1] >> u) &&
                           (cr[2] >> u) == (cq[2] >> u);
                }
                if (!seen) emit(b);
            } else {
                // the deeper leaves inside the cell, in key order: from the first key at
                // or after the cell's start (b itself when it starts there)
                int B = b >= 0 && ix.key[b] == qk ? b : b + 1;
                while (B < E) {
                    const int4 bx = ix.box[B];
                    if (tree_meet(bx.x, bx.y, bx.z, bx.w, oa, sa)) {
                        emit(B);
                        ++B;
                        continue;
                    }
                    // the coarsest ancestor of B below the cell that misses A: every leaf
                    // in it misses A too
                    int l = L + 1;
                    for (; l < bx.w; ++l) {
                        const int m = ~((1 << (kTreeBits - l)) - 1);
                        if (!tree_meet(bx.x & m, bx.y & m, bx.z & m, l, oa, sa)) break;
                    }
                    const int sl = tree_shift(l);
                    const u64 past = ((ix.key[B] >> sl) + 1) << sl;
                    B = ix.gallop(B + 1, E, past);
                }
            }
        }
        if (!FILL) cnt[t] = w;
    }
    if (!FILL) {
        // the workgroup's list entries and pair terms, added later in workgroup order
        // (integers: exact); one record per workgroup, no contended atomics
        __shared__ long long red[2][4];
        long long tw = w, tt = live ? terms * (long long)(cell_start[t / 27 + 1] -
                                                          cell_start[t / 27]) : 0;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            tw += __shfl_xor(tw, o);
            tt += __shfl_xor(tt, o);
        }
        if ((threadIdx.x & 63) == 0) {
            red[0][threadIdx.x >> 6] = tw;
            red[1][threadIdx.x >> 6] = tt;
        }
        __syncthreads();
        if (threadIdx.x == 0)
            part[blockIdx.x] = make_longlong2(red[0][0] + red[0][1] + red[0][2] + red[0][3],
                                              red[1][0] + red[1][1] + red[1][2] + red[1][3]);
    }
}

// Sums of the per-workgroup records: workgroup b adds part[b * per .. (b + 1) * per)
// (integers, fixed order) into out[b]; with counters set (one workgroup), the sums go
// to counters[2..3] (list entries) and counters[4..5] (pair terms) as 64-bit integers.
__global__ void __launch_bounds__(256) tree_totals_kernel(const longlong2 *__restrict__ part,
                                                          int nparts, int per,
                                                          longlong2 *__restrict__ out,
                                                          int *__restrict__ counters)
{
    __shared__ long long red[2][4];
    long long a = 0, b = 0;
    const long long i0 = (long long)blockIdx.x * per;
    const long long i1 = i0 + per < nparts ? i0 + per : nparts;
    for (long long i = i0 + threadIdx.x; i < i1; i += 256) {
        a += part[i].x;
        b += part[i].y;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        a += __shfl_xor(a, o);
        b += __shfl_xor(b, o);
    }
    if ((threadIdx.x & 63) == 0) {
        red[0][threadIdx.x >> 6] = a;
        red[1][threadIdx.x >> 6] = b;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        const long long sa = red[0][0] + red[0][1] + red[0][2] + red[0][3];
        const long long sb = red[1][0] + red[1][1] + red[1][2] + red[1][3];
        if (counters) {
            *reinterpret_cast<u64 *>(counters + 2) = (u64)sa;
            *reinterpret_cast<u64 *>(counters + 4) = (u64)sb;
        } else {
            out[blockIdx.x] = make_longlong2(sa, sb);
        }
    }
}

// ---------------------------------------------------------------- SoA layout
// Separate x, y, z, m arrays (the host layout of the lecture's CPU program,
// Degawa slide 15) in and out of the 16-byte records the kernels read.
__global__ void __launch_bounds__(256) pack_kernel(const float *__restrict__ a,
                                                   const float *__restrict__ b,
                                                   const float *__restrict__ c,
                                                   const float *__restrict__ d, int n,
                                                   float4 *__restrict__ out)
{
    const unsigned i = blockIdx.x * 256u + threadIdx.x;
    if (i >= (unsigned)n) return;
    out[i] = make_float4(a[i], b[i], c[i], d ? d[i] : 0.0f);
}

__global__ void __launch_bounds__(256) unpack_kernel(const float4 *__restrict__ in, int n,
                                                     float *__restrict__ a,
                                                     float *__restrict__ b,
                                                     float *__restrict__ c)
{
    const unsigned i = blockIdx.x * 256u + threadIdx.x;
    if (i >= (unsigned)n) return;
    const float4 v = in[i];
    a[i] = v.x;
    b[i] = v.y;
    c[i] = v.z;
}

template <int T, bool POT>
const void *accel_fn(int bcast, int wg)
{
    if (bcast == 1 && wg == 64) return (const void *)&accel_lds<T, POT, 64>;
    if (bcast == 1 && wg == 128) return (const void *)&accel_lds<T, POT, 128>;
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

template <int TW>
const void *small_fn(bool pot, bool step)
{
    if (step) return (const void *)&accel_small<TW, false, true>;
    return pot ? (const void *)&accel_small<TW, true, false>
               : (const void *)&accel_small<TW, false, false>;
}

template <int T, int BD>
const void *pairs_fn(bool pot)
{
    return pot ? (const void *)&accel_pairs<T, BD, true> : (const void *)&accel_pairs<T, BD, false>;
}

hipError_t launch_pairs(int band, int tpl, bool pot, const PairsArgs &args, hipStream_t stream)
{
    const void *fn = nullptr;
    if (tpl == 4) {
        if (band == 256) fn = pairs_fn<4, 256>(pot);
        if (band == 512) fn = pairs_fn<4, 512>(pot);
        if (band == 1024) fn = pairs_fn<4, 1024>(pot);
        if (band == 2048) fn = pairs_fn<4, 2048>(pot);
    } else if (tpl == 8) {
        if (band == 512) fn = pairs_fn<8, 512>(pot);
        if (band == 1024) fn = pairs_fn<8, 1024>(pot);
        if (band == 2048) fn = pairs_fn<8, 2048>(pot);
        if (band == 4096) fn = pairs_fn<8, 4096>(pot);
    }
    const PairsArgs &a = args;
    if (!fn || a.n < 1 || a.nbands != (a.n + band - 1) / band || a.band0 < 0 ||
        a.band1 > a.nbands || a.band0 >= a.band1 || a.run < 1 ||
        a.nruns != pair_runs(a.nbands, a.run) || !a.own || !a.partner || a.own0 < 0 ||
        1 + a.nruns > 65535)
        return hipErrorInvalidValue;
    PairsArgs c = a;
    void *kargs[] = {&c};
    return hipLaunchKernel(fn, dim3((unsigned)(a.band1 - a.band0), (unsigned)(1 + a.nruns), 1),
                           dim3(256, 1, 1), kargs, 0, stream);
}

hipError_t launch_pairs_finish(const PairsFinishArgs &args, hipStream_t stream)
{
    const PairsFinishArgs &a = args;
    if (a.n < 1 || a.band < 1 || a.nbands != (a.n + a.band - 1) / a.band || a.run < 1 ||
        !a.part || (a.pos == nullptr) != (a.vel == nullptr) || (!a.pos && !a.acc_out))
        return hipErrorInvalidValue;
    PairsFinishArgs c = a;
    void *kargs[] = {&c};
    const unsigned g = (unsigned)((a.n + 255) / 256);
    return hipLaunchKernel((const void *)&pairs_finish_kernel, dim3(g), dim3(256), kargs, 0,
                           stream);
}

hipError_t launch_pass_combine(const PassArgs &args, hipStream_t stream)
{
    const PassArgs &a = args;
    if (a.n < 1 || a.band < 1 || a.nbands != (a.n + a.band - 1) / a.band || a.band0 < 0 ||
        a.band1 > a.nbands || a.band0 >= a.band1 || a.own0 != a.band0 * a.band ||
        a.own_count < 1 || a.own0 + a.own_count > a.n || !a.acc_out || a.run < 1 ||
        !a.own || !a.partner ||
        (!(a.first && a.last) && (!a.tot_s || !a.tot_e)))
        return hipErrorInvalidValue;
    PassArgs p = a;
    void *kargs[] = {&p};
    const unsigned g = (unsigned)((a.n + 255) / 256);
    return hipLaunchKernel((const void *)&pass_combine_kernel, dim3(g), dim3(256), kargs, 0, stream);
}

hipError_t launch_shard_combine(const float4 *part, int n, int band, int nbands, int run,
                                int band0, int band1, float4 *out, hipStream_t stream)
{
    if (n < 1 || band < 1 || nbands != (n + band - 1) / band || band0 < 0 || band1 > nbands ||
        band0 >= band1 || run < 1 || !part || !out)
        return hipErrorInvalidValue;
    void *kargs[] = {&part, &n, &band, &nbands, &run, &band0, &band1, &out};
    const unsigned g = (unsigned)((n + 255) / 256);
    return hipLaunchKernel((const void *)&shard_combine_kernel, dim3(g), dim3(256), kargs, 0,
                           stream);
}

hipError_t launch_shard_finish(const float4 *partials, int n, int nshards, int t0, int t1,
                               float4 *acc_out, float *pot_out, hipStream_t stream)
{
    if (n < 1 || nshards < 1 || t0 < 0 || t1 > n || t0 >= t1) return hipErrorInvalidValue;
    void *kargs[] = {&partials, &n, &nshards, &t0, &t1, &acc_out, &pot_out};
    const unsigned g = (unsigned)((t1 - t0 + 255) / 256);
    return hipLaunchKernel((const void *)&shard_finish_kernel, dim3(g), dim3(256), kargs, 0,
                           stream);
}

hipError_t launch_small(int tw, bool pot, bool step, const SmallArgs &args, hipStream_t stream)
{
    const void *fn = nullptr;
    if (tw == 4) fn = small_fn<4>(pot, step);
    if (tw == 8) fn = small_fn<8>(pot, step);
    if (tw == 16) fn = small_fn<16>(pot, step);
    if (tw == 32) fn = small_fn<32>(pot, step);
    if (!fn || args.n < 1) return hipErrorInvalidValue;
    if (step && (!args.pos_next || !args.vel || args.pos_next == args.pos))
        return hipErrorInvalidValue;
    if (!step && !args.acc_out) return hipErrorInvalidValue;
    SmallArgs a = args;
    void *kargs[] = {&a};
    return hipLaunchKernel(fn, dim3((unsigned)((a.n + tw - 1) / tw)), dim3(256), kargs, 0, stream);
}

template <typename Lists>
hipError_t launch_p2p_any(bool pot, const P2PArgs &args, Lists l, hipStream_t stream)
{
    P2PArgs a = args;
    void *k[] = {&a, &l};
    const void *fn;
    const bool four = (long long)a.n >= (long long)kP2PWavesMinBodies * a.ncell;
    const int waves = four ? kP2PWaves : 1;
    if (four)
        fn = pot ? (const void *)&p2p_kernel<true, Lists, kP2PWaves>
                 : (const void *)&p2p_kernel<false, Lists, kP2PWaves>;
    else
        fn = pot ? (const void *)&p2p_kernel<true, Lists, 1>
                 : (const void *)&p2p_kernel<false, Lists, 1>;
    // ny workgroups per cell, workgroup y taking the target chunks q = y, y + ny, ...:
    // one below 64 bodies per cell on average (most cells are one chunk: a second
    // workgroup would only exit; N = 2^20 on a 64^3 grid 0.268 -> 0.220 ms, leaves of
    // ~4 bodies 0.375 -> 0.326 ms), two from 64, four from 192 (against two: 16^3 and
    // 15^3 grids of N = 2^20 0.9 and 2.2 % faster, octree leaves of ~256 bodies 4 %),
    // and from 384 about one per 64-target chunk of a cell a little larger than the
    // mean, ceil((m + 3 sqrt(m)) / 64) for mean cell size m, at most 1024 (so that a
    // few very large cells still fill the GPU). This replaced a kernel of 256-thread
    // workgroups sharing 256-body source tiles for large cells: against it, N = 2^20
    // on grids of 14^3 to 4^3 cells (382 to 16384 bodies each) 3.58 -> 2.80, 5.31 ->
    // 4.47, 8.73 -> 7.51, 15.6 -> 14.7, 33.0 -> 31.1 and 162 -> 99 ms; octree leaves of
    // ~1000 bodies 14.6 -> 9.2 ms.
    unsigned ny = (long long)a.n >= 192ll * a.ncell ? 4u : ((long long)a.n >= 64ll * a.ncell ? 2u : 1u);
    if ((long long)a.n >= 384ll * a.ncell) {
        const double m = (double)a.n / (double)a.ncell;
        const double want = std::ceil((m + 3.0 * std::sqrt(m)) / 64.0);
        ny = want >= 1024.0 ? 1024u : (unsigned)want;
    }
    return hipLaunchKernel(fn, dim3((unsigned)a.ncell, ny), dim3(64 * waves), k, 0, stream);
}

hipError_t launch_p2p(bool pot, const P2PArgs &args, hipStream_t stream)
{
    if (args.ncell < 1) return args.ncell == 0 ? hipSuccess : hipErrorInvalidValue;
    return launch_p2p_any(pot, args,
                          PackedLists{args.list_off, args.list, args.nlist, args.ncell, nullptr, -1},
                          stream);
}

hipError_t launch_p2p_grid(bool pot, const P2PArgs &args, const GridSpec &g, hipStream_t stream)
{
    if (args.ncell < 1 || args.ncell != g.dims[0] * g.dims[1] * g.dims[2])
        return hipErrorInvalidValue;
    // heavy cells first from 16 bodies per cell on average (measured: 0.9 % faster at
    // 16, 2.4 % slower at 9.5 and 11 % at 4 bodies per cell, where the launch has many
    // rounds and the natural order reads neighbouring cells together)
    const int heavy_first = (long long)args.n >= 16ll * args.ncell ? 1 : 0;
    return launch_p2p_any(pot, args, GridLists{g.dims[0], g.dims[1], g.dims[2], nullptr, heavy_first},
                          stream);
}

hipError_t launch_p2p_sym(bool pot, const float4 *pos, int n, float eps2, const int *cell_start,
                          const GridSpec &g, float4 *part, hipStream_t stream)
{
    const long long ncell = (long long)g.dims[0] * g.dims[1] * g.dims[2];
    if (n < 1 || !pos || !cell_start || !part || g.dims[0] < 1 || g.dims[1] < 1 ||
        g.dims[2] < 1 || ncell > INT_MAX)
        return hipErrorInvalidValue;
    SymArgs a{pos, n, eps2, cell_start, {g.dims[0], g.dims[1], g.dims[2]}, 1, part};
    void *kargs[] = {&a};
    const void *fn = pot ? (const void *)&p2p_sym_kernel<true> : (const void *)&p2p_sym_kernel<false>;
    return hipLaunchKernel(fn, dim3((unsigned)ncell), dim3(256), kargs, 0, stream);
}

hipError_t launch_sym_finish(const float4 *part, int n, const unsigned *cell_of,
                             const int *cell_start, const GridSpec &g, const int *out_index,
                             float4 *acc_out, float *pot_out, hipStream_t stream)
{
    if (n < 1 || !part || !cell_of || !cell_start || !acc_out) return hipErrorInvalidValue;
    int dx = g.dims[0], dy = g.dims[1], dz = g.dims[2];
    void *kargs[] = {&part, &n, &cell_of, &cell_start, &dx, &dy, &dz, &out_index, &acc_out, &pot_out};
    return hipLaunchKernel((const void *)&sym_finish_kernel, dim3((unsigned)((n + 255) / 256)),
                           dim3(256), kargs, 0, stream);
}

hipError_t launch_grid_keys(const float4 *pos, int n, const GridSpec &g, unsigned *keys, int *idx,
                            hipStream_t stream)
{
    if (n <= 0) return n == 0 ? hipSuccess : hipErrorInvalidValue;
    GridSpec gg = g;
    void *k[] = {&pos, &n, &gg, &keys, &idx};
    return hipLaunchKernel((const void *)&grid_keys_kernel, dim3((unsigned)((n + 255) / 256)),
                           dim3(256), k, 0, stream);
}

hipError_t launch_gather(const float4 *pos, const int *perm, int n, float4 *out,
                         hipStream_t stream)
{
    if (n <= 0) return n == 0 ? hipSuccess : hipErrorInvalidValue;
    void *k[] = {&pos, &perm, &n, &out};
    return hipLaunchKernel((const void *)&gather_kernel, dim3((unsigned)((n + 255) / 256)),
                           dim3(256), k, 0, stream);
}

hipError_t launch_cell_starts(const unsigned *sorted_keys, int n, int ncell, int *cell_start,
                              hipStream_t stream)
{
    if (ncell < 0 || n < 0) return hipErrorInvalidValue;
    void *k[] = {&sorted_keys, &n, &ncell, &cell_start};
    return hipLaunchKernel((const void *)&cell_starts_kernel,
                           dim3((unsigned)((ncell + 1 + 255) / 256)), dim3(256), k, 0, stream);
}

size_t sort_temp_bytes(int n, int key_bytes)
{
    const SortShape sh = sort_shape(n < 1 ? 1 : n);
    const size_t keys = ((size_t)(n < 1 ? 1 : n) * (size_t)key_bytes + 255) / 256 * 256;
    const size_t vals = ((size_t)(n < 1 ? 1 : n) * 4 + 255) / 256 * 256;
    const size_t counts = ((size_t)kSortDigits * (size_t)sh.nblocks * sizeof(int) + 255) / 256 * 256;
    return keys + vals + counts + (size_t)kSortScanThreads * sizeof(int);
}

template <typename K>
hipError_t sort_pairs_t(void *temp, const K *keys_in, K *keys_out, const int *vals_in,
                        int *vals_out, int n, int end_bit, hipStream_t stream)
{
    if (n < 1 || end_bit < 1 || end_bit > (int)(8 * sizeof(K)) || !temp)
        return hipErrorInvalidValue;
    const SortShape sh = sort_shape(n);
    const size_t keys = ((size_t)n * sizeof(K) + 255) / 256 * 256;
    const size_t vals = ((size_t)n * 4 + 255) / 256 * 256;
    K *k_alt = (K *)temp;
    int *v_alt = (int *)((char *)temp + keys);
    int *counts = (int *)((char *)temp + keys + vals);
    int total = kSortDigits * sh.nblocks;
    int *tile_sums = (int *)((char *)counts +
                             ((size_t)total * sizeof(int) + 255) / 256 * 256);
    const unsigned ntiles = (unsigned)((total + kSortScanTile - 1) / kSortScanTile);
    static_assert(kSortDigits * kSortMaxBlocks <= kSortScanTile * kSortScanThreads,
                  "one scan workgroup adds at most kSortScanThreads tile sums");
    const int passes = (end_bit + kSortBits - 1) / kSortBits;
    const K *ks = keys_in;
    const int *vs = vals_in;
    int nn = n, per = sh.per, nbl = sh.nblocks;
    for (int p = 0; p < passes; ++p) {
        // the last pass writes the outputs; before it, the two buffers alternate so that
        // no pass reads the array it writes
        const bool to_out = (passes - 1 - p) % 2 == 0;
        K *kd = to_out ? keys_out : k_alt;
        int *vd = to_out ? vals_out : v_alt;
        int shift = p * kSortBits;
        void *a1[] = {&ks, &nn, &per, &shift, &nbl, &counts};
        hipError_t e = hipLaunchKernel((const void *)&sort_hist_kernel<K>, dim3(nbl), dim3(256),
                                       a1, 0, stream);
        if (e != hipSuccess) return e;
        void *a2[] = {&counts, &total, &tile_sums};
        e = hipLaunchKernel((const void *)&sort_tile_sums_kernel, dim3(ntiles),
                            dim3(kSortScanThreads), a2, 0, stream);
        if (e != hipSuccess) return e;
        e = hipLaunchKernel((const void *)&sort_scan_kernel, dim3(ntiles), dim3(kSortScanThreads),
                            a2, 0, stream);
        if (e != hipSuccess) return e;
        void *a3[] = {&ks, &vs, &nn, &per, &shift, &nbl, &counts, &kd, &vd};
        e = hipLaunchKernel((const void *)&sort_scatter_kernel<K>, dim3(nbl), dim3(256), a3, 0,
                            stream);
        if (e != hipSuccess) return e;
        ks = kd;
        vs = vd;
    }
    return hipSuccess;
}

hipError_t sort_pairs(void *temp, const unsigned *keys_in, unsigned *keys_out, const int *vals_in,
                      int *vals_out, int n, int end_bit, hipStream_t stream)
{
    return sort_pairs_t<unsigned>(temp, keys_in, keys_out, vals_in, vals_out, n, end_bit, stream);
}

hipError_t sort_pairs64(void *temp, const unsigned long long *keys_in,
                        unsigned long long *keys_out, const int *vals_in, int *vals_out, int n,
                        int end_bit, hipStream_t stream)
{
    return sort_pairs_t<unsigned long long>(temp, keys_in, keys_out, vals_in, vals_out, n,
                                            end_bit, stream);
}

size_t scan_temp_bytes(long long total)
{
    size_t bytes = 256;
    for (long long t = total; t > kSortScanTile;) {
        t = (t + kSortScanTile - 1) / kSortScanTile;
        bytes += ((size_t)t * sizeof(int) + 255) / 256 * 256;
    }
    return bytes;
}

hipError_t scan_exclusive(int *data, long long total, int *total_out, void *temp,
                          hipStream_t stream)
{
    if (total < 0 || total > INT32_MAX || (total > 0 && !data)) return hipErrorInvalidValue;
    int tot = (int)total;
    const unsigned ntiles = tot > 0 ? (unsigned)((tot + kSortScanTile - 1) / kSortScanTile) : 1u;
    int *offsets = nullptr;
    if (ntiles > 1) {
        if (!temp) return hipErrorInvalidValue;
        offsets = (int *)temp;
        void *a[] = {&data, &tot, &offsets};
        hipError_t e = hipLaunchKernel((const void *)&sort_tile_sums_kernel, dim3(ntiles),
                                       dim3(kSortScanThreads), a, 0, stream);
        if (e != hipSuccess) return e;
        void *rest = (char *)temp + ((size_t)ntiles * sizeof(int) + 255) / 256 * 256;
        e = scan_exclusive(offsets, ntiles, nullptr, rest, stream);
        if (e != hipSuccess) return e;
    }
    const int *offs = offsets;
    void *a[] = {&data, &tot, &offs, &total_out};
    return hipLaunchKernel((const void *)&scan_tiles_kernel, dim3(ntiles), dim3(kSortScanThreads),
                           a, 0, stream);
}

size_t tree_frame_temp_bytes(int) { return (size_t)kTreeBoundsBlocks * 6 * sizeof(float); }

hipError_t launch_tree_frame(const float4 *pos, int n, float *temp, float4 *frame, int *counters,
                             hipStream_t stream)
{
    if (n < 0) return hipErrorInvalidValue;
    long long nb = ((long long)n + 255) / 256;
    int nparts = (int)(nb < 1 ? 1 : (nb > kTreeBoundsBlocks ? kTreeBoundsBlocks : nb));
    void *a[] = {&pos, &n, &temp};
    hipError_t e = hipLaunchKernel((const void *)&tree_bounds_kernel, dim3(nparts), dim3(256), a, 0,
                                   stream);
    if (e != hipSuccess) return e;
    void *b[] = {&temp, &nparts, &frame, &counters};
    return hipLaunchKernel((const void *)&tree_frame_kernel, dim3(1), dim3(64), b, 0, stream);
}

hipError_t launch_tree_keys(const float4 *pos, int n, const float4 *frame,
                            unsigned long long *keys, int *idx, hipStream_t stream)
{
    if (n <= 0) return n == 0 ? hipSuccess : hipErrorInvalidValue;
    void *a[] = {&pos, &n, &frame, &keys, &idx};
    return hipLaunchKernel((const void *)&tree_keys_kernel, dim3((unsigned)((n + 255) / 256)),
                           dim3(256), a, 0, stream);
}

hipError_t launch_tree_levels(const unsigned long long *skeys, int n, int leaf_size, int *level,
                              int *start, hipStream_t stream)
{
    if (n <= 0) return n == 0 ? hipSuccess : hipErrorInvalidValue;
    if (leaf_size < 1) return hipErrorInvalidValue;
    void *a[] = {&skeys, &n, &leaf_size, &level, &start};
    const void *fn = leaf_size <= kTreeWinS ? (const void *)&tree_levels_kernel<true>
                                            : (const void *)&tree_levels_kernel<false>;
    return hipLaunchKernel(fn, dim3((unsigned)((n + 255) / 256)), dim3(256), a, 0, stream);
}

hipError_t launch_tree_leaves(const unsigned long long *skeys, const int *level, const int *ids,
                              int n, int *cell_start, unsigned long long *leaf_key, int4 *leaf_box,
                              hipStream_t stream)
{
    if (n <= 0) return n == 0 ? hipSuccess : hipErrorInvalidValue;
    void *a[] = {&skeys, &level, &ids, &n, &cell_start, &leaf_key, &leaf_box};
    return hipLaunchKernel((const void *)&tree_leaves_kernel, dim3((unsigned)((n + 255) / 256)),
                           dim3(256), a, 0, stream);
}

int tree_table_level(int nleaf)
{
    int lt = 1;
    while (lt < kTreeTableMaxLevel && (1ll << (3 * lt)) < (long long)nleaf) ++lt;
    return lt;
}

hipError_t launch_tree_table(const unsigned long long *leaf_key, const int *counters, int lt,
                             int *table, hipStream_t stream)
{
    if (lt < 1 || lt > kTreeTableMaxLevel) return hipErrorInvalidValue;
    const long long entries = (1ll << (3 * lt)) + 1;
    void *a[] = {&leaf_key, &counters, &lt, &table};
    return hipLaunchKernel((const void *)&tree_table_kernel,
                           dim3((unsigned)((entries + 255) / 256)), dim3(256), a, 0, stream);
}

constexpr int kTreeTotalsPer = 1024;  // records per workgroup of the first totals pass

size_t tree_parts_bytes(int nleaf)
{
    const long long nb = (27ll * nleaf + 1 + 255) / 256;
    return (size_t)(nb + (nb + kTreeTotalsPer - 1) / kTreeTotalsPer) * sizeof(longlong2);
}

hipError_t launch_tree_lists(const TreeLeaves &lv, int *counters, void *parts, int *cnt,
                             const int *off, int *list, int list_cap, int *list_off, int *keep,
                             int keep_cap, hipStream_t stream)
{
    if (lv.nleaf <= 0 || lv.nleaf > kTreeMaxLeaves) return hipErrorInvalidValue;
    const bool fill = list != nullptr;
    if (fill ? (!off || !list_off) : (!cnt || !parts || !counters)) return hipErrorInvalidValue;
    if (keep_cap < 0 || (keep_cap > 0 && !keep)) return hipErrorInvalidValue;
    TreeIndex ix{lv.leaf_key, lv.leaf_box, lv.table, lv.nleaf, lv.lt};
    const int *cs = lv.cell_start;
    longlong2 *pt = (longlong2 *)parts;
    void *a[] = {&ix, &cs, &pt, &cnt, &off, &list, &list_cap, &list_off, &keep, &keep_cap};
    const void *fn = fill ? (const void *)&tree_lists_kernel<true>
                          : (const void *)&tree_lists_kernel<false>;
    const long long threads = 27ll * lv.nleaf + 1;
    int nblocks = (int)((threads + 255) / 256);
    hipError_t e = hipLaunchKernel(fn, dim3((unsigned)nblocks), dim3(256), a, 0, stream);
    if (e != hipSuccess || fill) return e;
    // the workgroup records in two passes: kTreeTotalsPer per workgroup, then one
    int per = kTreeTotalsPer, ng = (nblocks + per - 1) / per;
    longlong2 *mid = pt + nblocks;
    int *none = nullptr;
    void *b1[] = {&pt, &nblocks, &per, &mid, &none};
    e = hipLaunchKernel((const void *)&tree_totals_kernel, dim3((unsigned)ng), dim3(256), b1, 0,
                        stream);
    if (e != hipSuccess) return e;
    void *b2[] = {&mid, &ng, &ng, &mid, &counters};
    return hipLaunchKernel((const void *)&tree_totals_kernel, dim3(1), dim3(256), b2, 0, stream);
}

hipError_t launch_pack(const float *a, const float *b, const float *c, const float *d, int n,
                       float4 *out, hipStream_t stream)
{
    if (n <= 0) return n == 0 ? hipSuccess : hipErrorInvalidValue;
    void *k[] = {&a, &b, &c, &d, &n, &out};
    return hipLaunchKernel((const void *)&pack_kernel, dim3((unsigned)((n + 255) / 256)),
                           dim3(256), k, 0, stream);
}

hipError_t launch_unpack(const float4 *in, int n, float *a, float *b, float *c, hipStream_t stream)
{
    if (n <= 0) return n == 0 ? hipSuccess : hipErrorInvalidValue;
    void *k[] = {&in, &n, &a, &b, &c};
    return hipLaunchKernel((const void *)&unpack_kernel, dim3((unsigned)((n + 255) / 256)),
                           dim3(256), k, 0, stream);
}

int diag_blocks(int n)
{
    const int b = (n + 255) / 256;
    return b < 1 ? 1 : (b > kDiagMaxBlocks ? kDiagMaxBlocks : b);
}

hipError_t launch_diagnostics(const float4 *pos, const float4 *vel, const float *pot, int n,
                              double inv_eps, double *part, double *out, hipStream_t stream)
{
    if (n < 0 || !part || !out || (n > 0 && (!pos || !vel || !pot))) return hipErrorInvalidValue;
    const int nb = diag_blocks(n);
    void *k1[] = {&pos, &vel, &pot, &n, &inv_eps, &part};
    hipError_t e = hipLaunchKernel((const void *)&diag_partial_kernel, dim3(nb), dim3(256), k1, 0,
                                   stream);
    if (e != hipSuccess) return e;
    int nbl = nb;
    void *k2[] = {&part, &nbl, &out};
    return hipLaunchKernel((const void *)&diag_final_kernel, dim3(1), dim3(256), k2, 0, stream);
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
