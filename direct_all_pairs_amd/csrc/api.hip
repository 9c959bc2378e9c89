// C ABI of the library (declared in include/nbody.h): argument checks, launch
// planning, the cached split-j scratch area and the step loop.
#include <hip/hip_runtime.h>

#include <array>
#include <cmath>
#include <cfloat>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <tuple>
#include <tuple>
#include <utility>

// The library is built with hidden symbol visibility; only the C ABI declared
// in nbody.h is exported.
#pragma GCC visibility push(default)
#include "../../include/nbody.h"
#pragma GCC visibility pop
#include "kernels.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

int ok()
{
    g_err.clear();
    return NBODY_OK;
}

int hip_fail(hipError_t e, const char *what)
{
    return fail(NBODY_EHIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

bool overlap(const void *a, size_t na, const void *b, size_t nb)
{
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + nb && b0 < a0 + na;
}

// eps2 must be finite and at least 2^-84: the softening is what makes the
// j = i term finite (Degawa, "N 体問題", slide 12), and the largest 1/r^3 a
// pair term forms, eps2^(-3/2) (the self pair), must be finite in fp32. Below
// 2^-84 it exceeds 2^126 and overflows once cubed from the rsq (the pair kernel
// forms (inv * inv) * inv), turning the self term into inf * 0 = NaN.
constexpr float kEps2Min = 0x1p-84f;
bool eps2_ok(float e) { return std::isfinite(e) && e >= kEps2Min; }
int eps2_fail(float e)
{
    return fail(NBODY_EINVAL, "eps2=%g must be a finite float >= 2^-84 (%g), so that "
                              "eps2^(-3/2) is finite in fp32", (double)e, (double)kEps2Min);
}

// ------------------------------------------------------------ device facts

std::mutex g_mu;
struct DeviceFacts {
    int cus = 1;            // compute units
    size_t mem_bytes = 0;   // device memory
};
std::map<int, DeviceFacts> g_dev;

int device_facts(int dev, DeviceFacts *out)
{
    std::lock_guard<std::mutex> lk(g_mu);
    auto it = g_dev.find(dev);
    if (it != g_dev.end()) {
        *out = it->second;
        return NBODY_OK;
    }
    DeviceFacts f;
    int v = 0;
    hipError_t e = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute(multiprocessor count)");
    f.cus = v > 0 ? v : 1;
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
    f.mem_bytes = prop.totalGlobalMem;
    g_dev[dev] = f;
    *out = f;
    return NBODY_OK;
}

// ------------------------------------------------------------ scratch cache

struct Scratch {
    void *ptr = nullptr;
    size_t bytes = 0;
};
// Keyed by (device, stream, slot); slots 1 and 2 hold the list counts and the
// interaction lists of nbody_near_tree, whose sizes are known only part-way
// through its build.
std::map<std::tuple<int, hipStream_t, int>, Scratch> g_scratch;

// Held by every entry point that uses scratch, from taking the block until its
// last launch is enqueued, and by nbody_release_workspace: no host thread can
// grow (free) a block another thread has taken but not yet launched work on.
// Enqueueing takes microseconds; the GPU work itself runs after the lock.
std::mutex g_enqueue;
using EnqueueLock = std::lock_guard<std::mutex>;

// ------------------------------------------------------------ static scratch
// nbody_step_noalloc takes its scratch from this array instead of hipMalloc:
// every GPU the library runs on holds its own copy (in the library's code
// object) until the process ends, and every such call on that GPU shares it.
// In host code `scratch` names only a host-side stand-in: the kernels get the
// device address that hipGetSymbolAddress returns for the current device.
constexpr size_t kStaticScratchBytes = size_t(1) << 27;  // 128 MiB
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

std::map<int, void *> g_static_scratch;  // device -> its copy of `scratch` (under g_mu)

// The device address of `scratch` on device dev, which must be current; looked
// up once per device.
int static_scratch(int dev, void **out)
{
    std::lock_guard<std::mutex> lk(g_mu);
    auto it = g_static_scratch.find(dev);
    if (it != g_static_scratch.end()) {
        *out = it->second;
        return NBODY_OK;
    }
    void *p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (p == nullptr || !aligned(p, 256))
        return fail(NBODY_EHIP, "hipGetSymbolAddress(scratch) returned %p", p);
    g_static_scratch[dev] = p;
    *out = p;
    return NBODY_OK;
}

// ------------------------------------------------------------ near-tree graphs
// A near-tree call launches about fifty kernels of a few microseconds each, so past
// the first sort passes the GPU waits on the host's launches (~160 us of a 950 us
// call at N = 2^20). The kernels and arguments of its build up to the leaf-count wait
// are fixed by (N, node size, positions, scratch block), those of the list passes
// after it by (leaf count, table level, kept entries, list capacity, scratch blocks).
// The second call with the same key captures that sequence into a graph on a library
// stream and later ones replay it on the caller's stream; a first call launches the
// kernels directly, so one-off calls pay no capture and the replays can be checked
// against it. Under g_enqueue. Every entry's last replay has finished when the next
// call takes the lock for the build phase (the call waits for it); list-phase
// entries may still run, so replacing any entry first waits for the device.
struct TreeGraphKey {
    int dev, phase;
    hipStream_t stream;
    std::array<int64_t, 6> v;
    std::array<const void *, 6> p;
    bool operator<(const TreeGraphKey &o) const
    {
        return std::tie(dev, phase, stream, v, p) < std::tie(o.dev, o.phase, o.stream, o.v, o.p);
    }
};
struct TreeGraph {
    int seen = 0;
    hipGraphExec_t exec = nullptr;
};
std::map<TreeGraphKey, TreeGraph> g_tree_graphs;
std::map<int, hipStream_t> g_capture_stream;  // per device, default priority
constexpr size_t kTreeGraphMax = 16;

// Waits for every device that holds a cached graph (a replay may still run there), then
// destroys them all; the caller's current device is restored.
int drop_tree_graphs()
{
    if (g_tree_graphs.empty()) return NBODY_OK;
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    int last = -1;
    for (auto &kv : g_tree_graphs) {  // ordered by device first
        if (kv.first.dev == last) continue;
        last = kv.first.dev;
        hipError_t x = hipSetDevice(last);
        if (x == hipSuccess) x = hipDeviceSynchronize();
        if (e == hipSuccess) e = x;
    }
    const hipError_t r = hipSetDevice(cur);
    if (e == hipSuccess) e = r;
    for (auto &kv : g_tree_graphs)
        if (kv.second.exec) hipGraphExecDestroy(kv.second.exec);
    g_tree_graphs.clear();
    return e == hipSuccess ? NBODY_OK : hip_fail(e, "hipDeviceSynchronize (tree graphs)");
}

template <typename F>
hipError_t run_graphed(const TreeGraphKey &key, hipStream_t stream, F &&enqueue)
{
    if (g_tree_graphs.size() >= kTreeGraphMax && g_tree_graphs.find(key) == g_tree_graphs.end())
        if (drop_tree_graphs() != NBODY_OK) return hipErrorUnknown;
    TreeGraph &g = g_tree_graphs[key];
    if (g.exec) return hipGraphLaunch(g.exec, stream);
    if (g.seen++ == 0) return enqueue(stream);
    hipStream_t &cs = g_capture_stream[key.dev];
    hipError_t e = hipSuccess;
    if (!cs) e = hipStreamCreateWithFlags(&cs, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal);
    if (e != hipSuccess) return e;
    const hipError_t le = enqueue(cs);
    hipGraph_t graph = nullptr;
    e = hipStreamEndCapture(cs, &graph);
    if (le != hipSuccess || e != hipSuccess) {
        if (graph) hipGraphDestroy(graph);
        return le != hipSuccess ? le : e;
    }
    e = hipGraphInstantiate(&g.exec, graph, nullptr, nullptr, 0);
    hipGraphDestroy(graph);
    if (e != hipSuccess) {
        g.exec = nullptr;
        return e;
    }
    return hipGraphLaunch(g.exec, stream);
}

// While set (by nbody_step_noalloc, for the length of its enqueueing), scratch_get
// hands out this block instead of the cached one and never allocates.
struct FixedScratch {
    void *ptr = nullptr;
    size_t bytes = 0;
};
thread_local FixedScratch g_fixed;

struct FixedScratchScope {
    FixedScratchScope(void *p, size_t b) { g_fixed = FixedScratch{p, b}; }
    ~FixedScratchScope() { g_fixed = FixedScratch{}; }
};

// Returns scratch of at least `bytes` for (device, stream). Growing frees the
// old block first; hipFree waits for the device, so work still queued on the
// old block finishes before it is released.
int scratch_get(int dev, hipStream_t stream, size_t bytes, void **out, int slot = 0)
{
    if (g_fixed.ptr) {
        if (bytes > g_fixed.bytes)
            return fail(NBODY_EINVAL, "internal: %zu bytes of scratch exceed the static %zu",
                        bytes, g_fixed.bytes);
        *out = g_fixed.ptr;
        return NBODY_OK;
    }
    std::lock_guard<std::mutex> lk(g_mu);
    Scratch &s = g_scratch[std::make_tuple(dev, stream, slot)];
    if (s.bytes < bytes) {
        if (s.ptr) {
            hipError_t e = hipFree(s.ptr);
            s.ptr = nullptr;
            s.bytes = 0;
            if (e != hipSuccess) return hip_fail(e, "hipFree(scratch)");
        }
        size_t want = bytes + bytes / 4;  // some headroom for nearby sizes
        void *p = nullptr;
        hipError_t e = hipMalloc(&p, want);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            return fail(NBODY_ENOMEM, "hipMalloc(%zu bytes of scratch) failed: %s", want,
                        hipGetErrorString(e));
        }
        s.ptr = p;
        s.bytes = want;
    }
    *out = s.ptr;
    return NBODY_OK;
}

// ------------------------------------------------------------ kernel timing
// nbody_time_kernel: events of the calling thread, recorded around the first
// launch of a pair-term kernel in each later call.
struct KernelTimer {
    hipEvent_t start = nullptr, stop = nullptr;
    bool pending = false;  // the current call has not recorded them yet
};
thread_local KernelTimer g_timer;

// At the start of every entry point.
void timer_arm() { g_timer.pending = g_timer.start != nullptr; }

// fn() launches a pair-term kernel; the call's first such launch is bracketed
// by the events.
template <typename F>
hipError_t timed_launch(hipStream_t stream, F &&fn)
{
    if (!g_timer.pending) return fn();
    g_timer.pending = false;
    hipError_t e = hipEventRecord(g_timer.start, stream);
    if (e != hipSuccess) return e;
    e = fn();
    if (e != hipSuccess) return e;
    return hipEventRecord(g_timer.stop, stream);
}

// ------------------------------------------------------------ planning

constexpr int kMaxSplits = 4096;
// nbody_near_grid chooses the pair-symmetric kernel for 96 to 2048 bodies per cell on
// average and at least two cells per compute unit (it runs one workgroup per cell), while
// its slots fit 1/16 of device memory (N up to ~86 million on MI355X).
// Measured at N = 2^20 on D^3 grids (kernel time, one-sided -> pairs): D = 23 (86
// per cell) 0.80 -> 0.84 ms, D = 22 (98) 0.86 -> 0.78, D = 16 (256) 2.0 -> 1.6, D = 12
// (607) 4.4 -> 3.8, D = 8 (2048, 512 cells) 14.6 -> 12.6, D = 7 (3057, 343 cells)
// 20.5 -> 25.6.
constexpr int64_t kSymMinMean = 96;
constexpr int64_t kSymMaxMean = 2048;
constexpr int64_t kSymMinCellsPerCU = 2;

// Most cells a uniform grid of nbody_near_grid may have (one 32-bit key per body
// and one start index per cell).
constexpr int64_t kMaxGridCells = (int64_t)1 << 28;
// Most bodies nbody_near_tree takes (its scans run over N + 1 int entries).
constexpr int64_t kMaxTreeN = (int64_t)1 << 30;

// Largest N the automatic plan gives to NBODY_MODE_SMALL; pair-symmetric bands
// (scratch permitting) take every N above it.
constexpr int64_t kSmallMaxN = 6144;
// Largest N whose automatic band is 256 bodies (4 targets per lane): many
// small work items fill the GPU there; above it, 512-2048 with 8 per lane.
constexpr int64_t kBand256MaxN = 36863;

int valid_tpl(int t) { return t == 1 || t == 2 || t == 4 || t == 8; }

// Pair-symmetric bands: partial-sum scratch is (N / band) x N x 16 bytes. The
// automatic plan uses the mode only while that stays within 1/16 of device
// memory (about 18 GB on MI355X, enough for N = 2^20 with 2048-body bands).
constexpr size_t kPairsScratchShare = 16;

int valid_band(int b) { return b == 256 || b == 512 || b == 1024 || b == 2048 || b == 4096; }

// Largest run length a plan may ask for (items per pair workgroup).
constexpr int kMaxRun = 1 << 16;

size_t pairs_scratch(int64_t n, int band, int run)
{
    const int64_t nb = (n + band - 1) / band;
    return (size_t)nbk::pair_slots((int)nb, run) * (size_t)n * sizeof(float4);
}

// Grid limit of the second launch dimension (pair items, split-j chunks).
constexpr int64_t kMaxGridY = 65535;

// Pair evaluation in `passes` passes over owner-band ranges of at most
// ceil(nb / passes) bands each: per pass the own slots of the range's bodies
// (1 + R each), the partner sides of every body from the range's owners (one
// record per owner and body), and across passes the compensated running totals
// (two records per body), plus, for a step, the accelerations handed to the
// Euler kernel.
size_t pairs_pass_scratch(int64_t n, int band, int run, int64_t passes, bool step)
{
    const int64_t nb = (n + band - 1) / band;
    const int64_t per = (nb + passes - 1) / passes;
    const int64_t own = per * band < n ? per * band : n;
    const int64_t recs = (1 + nbk::pair_runs((int)nb, run)) * own + per * n + 2 * n + (step ? n : 0);
    return (size_t)recs * sizeof(float4);
}

// Band range [first, end) of pass q of `passes` over nb bands (balanced).
int pass_band(int64_t q, int64_t nb, int64_t passes) { return (int)(q * nb / passes); }

// Automatic layout, chosen by measurement on MI355X (layout sweeps of the
// five workloads and of uniform cubes from N = 1024 to 131072):
//   - up to N = 6144, the small-N kernel (one kernel per evaluation or step;
//     round-robin on uniform cubes: 20.9 us against 25.3 for 256-body pair
//     bands at 6144, but 28.2 against 25.4 at 6656, where its last 1024-body
//     tile is half empty): 4 targets per workgroup to N = 2048, 8 above;
//   - above it, pair-symmetric bands when their scratch fits: 256 bodies with
//     4 targets per lane to N = 36863 (tied with 512 with 8 per lane at 32768;
//     from 36864 to 49152 within +-3 %, one way on one box and the other way on
//     another, in round-robin timing), then the largest band
//     that still yields at least 64 work items per compute unit, with 8
//     targets per lane;
//   - otherwise one-sided tiles with the LDS broadcast and one target per lane:
//     every VALU operand of the inner step is then a VGPR, which issues about
//     twice as fast as an SGPR operand; 512-thread workgroups (512-body LDS
//     tiles) from N = 65536 up, 256 below; split-j chunks until there are about
//     128 workgroups per compute unit over the run (finer load balance; a
//     chunk's sources stay L2-resident), at least 4 tiles per chunk from
//     N = 65536 up and 1 below.
int small_tw(int64_t n) { return n <= 2048 ? 4 : (n <= 6144 ? 8 : 16); }

// The automatic pair band for N and a requested tpl (0 = any): 256 bodies to
// N = 36863, above it the largest band with at least 64 work items per
// compute unit (512 at least). 4096-body bands (half the slots of 2048, on
// request) measured 0.3-1.3 % slower at N = 2^20, 0.25 % slower at 1.5 M
// (one pass against two of 2048), 0.25 % faster at 2^21 and 1 % slower at
// 2^22 (round-robin), so they are not chosen automatically.
int auto_band(int64_t n, int tpl, const DeviceFacts &dev)
{
    if (n <= kBand256MaxN && tpl != 8) return 256;
    for (int band : {2048, 1024}) {
        const int64_t nb = (n + band - 1) / band;
        if (nb * (nb / 2 + 1) >= (int64_t)dev.cus * 64) return band;
    }
    return 512;
}

// Passes for a pair evaluation: one while all nb slots per body fit the
// scratch share of device memory, else the fewest that fit (searched in
// steps of ~25 %); 0 when even one band per pass does not fit.
int64_t auto_passes(int64_t n, int band, int run, const DeviceFacts &dev, bool step)
{
    const size_t cap = dev.mem_bytes / kPairsScratchShare;
    if (pairs_scratch(n, band, run) <= cap) return 1;
    const int64_t nb = (n + band - 1) / band;
    for (int64_t q = 2; q <= nb; q = q < 8 ? q + 1 : q + q / 4)
        if (pairs_pass_scratch(n, band, run, q, step) <= cap) return q;
    return pairs_pass_scratch(n, band, run, nb, step) <= cap ? nb : 0;
}

// Items per pair workgroup (run length K): the longest power of two up to
// kMaxAutoRun whose shortest runs (K, or K / 4 where the last K band pairs of an
// owner are split) hold at most 1/kRunTailShare of the items each resident
// workgroup slot (four per CU) takes on average, so that the launch ends on
// short workgroups. Measured round-robin on MI355X (whole calls): N = 2^20 in
// 2048-body bands (128 items per slot) 208.4, 207.8, 208.3 and 209.7 ms at K = 8,
// 16, 32 and 64 with the split tail (without it 32 had cost 2.4 %); N = 2^21 827.1,
// 830.4 and 832.7 ms at K = 16, 32, 64; two Plummer spheres of 300,007 in 1024-body
// bands (42 items per slot) 17.99, 18.09 and 18.83 ms at K = 1, 2 and 16 (17.34 ms
// at 4 and 17.57 at 8 against 17.24 at 1 on another box); 65,536 in 512-body bands
// (8 items per slot) 0.839 ms at K = 1, 0.848 at 2.
constexpr int kMaxAutoRun = 32;
constexpr int64_t kRunTailShare = 16;
int auto_run(int64_t n, int band, const DeviceFacts &dev)
{
    const int64_t nb = (n + band - 1) / band;
    const int64_t per_slot = nb * (nb / 2 + 1) / (4 * (int64_t)dev.cus);
    int run = 1;
    for (int k = 2; k <= kMaxAutoRun; k *= 2) {
        const int64_t tail = nbk::run_split((int)nb, k) ? k / nbk::kRunSplit : k;
        if (tail * kRunTailShare <= per_slot) run = k;
    }
    return run;
}

void auto_plan(int64_t n, const DeviceFacts &dev, nbody_plan *p)
{
    const bool big = n >= 65536;
    if (p->mode == NBODY_MODE_AUTO) {
        p->mode = NBODY_MODE_TILES;
        if (n <= kSmallMaxN && p->bcast == NBODY_BCAST_AUTO && p->tpl == 0 && p->splits == 0 &&
            p->wg == 0 && p->band == 0)
            p->mode = NBODY_MODE_SMALL;
        if (n > kSmallMaxN && p->bcast == NBODY_BCAST_AUTO && p->tpl == 0 && p->splits == 0 &&
            p->wg == 0) {
            const int band = p->band != 0 ? p->band : auto_band(n, 0, dev);
            const int run = p->run != 0 ? p->run : auto_run(n, band, dev);
            const int64_t q = p->passes != 0 ? p->passes : auto_passes(n, band, run, dev, true);
            if (q != 0 && (n + band - 1) / band / 2 + 1 <= kMaxGridY) {
                p->mode = NBODY_MODE_PAIRS;
                p->band = band;
                p->run = run;
                p->passes = (int32_t)q;
            }
        }
    }
    if (p->mode == NBODY_MODE_SMALL) {
        p->bcast = NBODY_BCAST_LDS;
        if (p->tpl == 0) p->tpl = small_tw(n);
        p->wg = 256;
        return;
    }
    if (p->mode == NBODY_MODE_PAIRS) {
        p->bcast = NBODY_BCAST_LDS;
        if (p->band == 0) p->band = auto_band(n, p->tpl, dev);
        if (p->tpl == 0) p->tpl = (p->band == 256 || (n < 24576 && p->band != 4096)) ? 4 : 8;
        if (p->run == 0) p->run = auto_run(n, p->band, dev);
        if (p->passes == 0) {
            // explicit pair mode: if nothing fits, the most passes (the scratch
            // allocation then reports what is missing)
            const int64_t q = auto_passes(n, p->band, p->run, dev, true);
            p->passes = (int32_t)(q != 0 ? q : (n + p->band - 1) / p->band);
        }
        p->wg = 256;
        return;
    }
    if (p->bcast == NBODY_BCAST_AUTO) p->bcast = NBODY_BCAST_LDS;
    if (p->tpl == 0) p->tpl = 1;
    if (p->wg == 0) p->wg = (big && p->bcast == NBODY_BCAST_LDS) ? 512 : 256;
    if (p->splits == 0) {
        const int64_t per = (int64_t)p->wg * p->tpl;
        const int64_t gx = (n + per - 1) / per;  // target workgroups
        const int64_t want = (int64_t)dev.cus * 128;
        int64_t s = (want + gx - 1) / gx;
        const int64_t tile = p->bcast == NBODY_BCAST_LDS ? p->wg : nbk::kFlush;
        const int64_t min_chunk = tile * (big ? 4 : 1);
        const int64_t smax = (n + min_chunk - 1) / min_chunk;
        if (s > smax) s = smax;
        if (s < 1) s = 1;
        if (s > kMaxSplits) s = kMaxSplits;
        p->splits = (int32_t)s;
    }
}

// Final chunking. Tiles: chunk is a whole number of tiles (LDS tile or
// accumulation block) and S = ceil(N / chunk), so no chunk is empty. Pairs:
// splits = number of bands = number of partial slots, chunk = band.

void finish_plan(int64_t n, nbody_plan *p)
{
    if (p->mode == NBODY_MODE_SMALL) {
        p->splits = 1;
        p->chunk = (int32_t)n;
        p->band = 0;
        p->passes = 0;
        p->run = 0;
        return;
    }
    if (p->mode == NBODY_MODE_PAIRS) {
        p->splits = (int32_t)((n + p->band - 1) / p->band);
        p->chunk = p->band;
        if (p->passes < 1) p->passes = 1;
        if (p->passes > p->splits) p->passes = p->splits;
        return;
    }
    p->band = 0;
    p->passes = 0;
    p->run = 0;
    const int64_t tile = p->bcast == NBODY_BCAST_LDS ? p->wg : nbk::kFlush;
    int64_t s = p->splits;
    int64_t c = (n + s - 1) / s;
    c = (c + tile - 1) / tile * tile;
    if (c < tile) c = tile;
    if (c > INT32_MAX) c = (int64_t)INT32_MAX / tile * tile;
    s = (n + c - 1) / c;
    if (s < 1) s = 1;
    p->splits = (int32_t)s;
    p->chunk = (int32_t)c;
}

int make_plan(int64_t n, const nbody_plan *user, int *dev_out, nbody_plan *p)
{
    *p = user ? *user : nbody_plan{0, 0, 0, 0, 0, 0, 0, 0, 0};
    p->chunk = 0;
    if (p->passes < 0)
        return fail(NBODY_EINVAL, "plan.passes=%d must be >= 0", p->passes);
    if (p->run < 0 || p->run > kMaxRun)
        return fail(NBODY_EINVAL, "plan.run=%d must be in [0, %d]", p->run, kMaxRun);
    if (p->run != 0 && p->mode != NBODY_MODE_AUTO && p->mode != NBODY_MODE_PAIRS)
        return fail(NBODY_EINVAL, "plan.run is for pair mode (NBODY_MODE_PAIRS or AUTO)");
    if (p->passes != 0 && p->mode != NBODY_MODE_AUTO && p->mode != NBODY_MODE_PAIRS)
        return fail(NBODY_EINVAL, "plan.passes is for pair mode (NBODY_MODE_PAIRS or AUTO)");
    if (p->mode < 0 || p->mode > NBODY_MODE_SMALL)
        return fail(NBODY_EINVAL, "plan.mode=%d is not a NBODY_MODE_* value", p->mode);
    if (p->mode == NBODY_MODE_SMALL &&
        ((p->bcast != 0 && p->bcast != NBODY_BCAST_LDS) ||
         (p->tpl != 0 && p->tpl != 4 && p->tpl != 8 && p->tpl != 16 && p->tpl != 32) ||
         p->splits != 0 || (p->wg != 0 && p->wg != 256) || p->band != 0))
        return fail(NBODY_EINVAL, "plan.mode=NBODY_MODE_SMALL takes only plan.tpl 4, 8, 16 or 32 "
                                  "(targets per workgroup; bcast LDS, wg 256 implied)");
    if (p->bcast < 0 || p->bcast > NBODY_BCAST_READLANE)
        return fail(NBODY_EINVAL, "plan.bcast=%d is not a NBODY_BCAST_* value", p->bcast);
    if (p->tpl != 0 && !valid_tpl(p->tpl) && p->mode != NBODY_MODE_SMALL)
        return fail(NBODY_EINVAL, "plan.tpl=%d must be 0, 1, 2, 4 or 8", p->tpl);
    if (p->splits < 0 || p->splits > kMaxSplits)
        return fail(NBODY_EINVAL, "plan.splits=%d must be in [0, %d]", p->splits, kMaxSplits);
    if (p->wg != 0 && p->wg != 256 &&
        !((p->wg == 64 || p->wg == 128 || p->wg == 512) && p->bcast == NBODY_BCAST_LDS))
        return fail(NBODY_EINVAL,
                    "plan.wg=%d must be 0 or 256 (or 64, 128, 512 with the LDS broadcast)", p->wg);
    if (p->band != 0 && !valid_band(p->band))
        return fail(NBODY_EINVAL, "plan.band=%d must be 0, 256, 512, 1024, 2048 or 4096",
                    p->band);
    if (p->band == 256 && p->tpl == 8)
        return fail(NBODY_EINVAL, "plan.band=256 takes plan.tpl 4 (an i-set of 8 targets per "
                                  "lane is 512 bodies)");
    if (p->band == 4096 && p->tpl != 0 && p->tpl != 8)
        return fail(NBODY_EINVAL, "plan.band=4096 takes plan.tpl 8");
    if (p->mode == NBODY_MODE_PAIRS &&
        ((p->bcast != 0 && p->bcast != NBODY_BCAST_LDS) ||
         (p->tpl != 0 && p->tpl != 4 && p->tpl != 8) || p->splits != 0 ||
         (p->wg != 0 && p->wg != 256)))
        return fail(NBODY_EINVAL, "plan.mode=NBODY_MODE_PAIRS takes only plan.band, plan.run, "
                                  "plan.passes and plan.tpl 4 or 8 (bcast LDS, wg 256 and splits "
                                  "are implied)");
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    DeviceFacts facts;
    int rc = device_facts(dev, &facts);
    if (rc != NBODY_OK) return rc;
    auto_plan(n, facts, p);
    finish_plan(n, p);
    if (p->mode == NBODY_MODE_PAIRS && p->splits / 2 + 1 > kMaxGridY)
        return fail(NBODY_EINVAL, "N=%lld needs %d bands of %d bodies: more than the launch "
                                  "grid takes (use a larger band or tiles mode)",
                    (long long)n, (int)p->splits, (int)p->band);
    *dev_out = dev;
    return NBODY_OK;
}

unsigned grid_x(int64_t n, int tpl, int wg)
{
    const int64_t per = (int64_t)wg * tpl;
    return (unsigned)((n + per - 1) / per);
}

// Largest N any entry point takes: body indices, tile cursors and chunk ends
// are 32-bit in the kernels and run up to a few tiles past N, so N stays a
// safe distance below 2^31 (an evaluation at 2^30 bodies is ~10^18
// interactions, days of work).
constexpr int64_t kMaxN = int64_t(1) << 30;

int check_n(int64_t n)
{
    if (n < 0) return fail(NBODY_EINVAL, "N=%lld must be >= 0", (long long)n);
    if (n > kMaxN) return fail(NBODY_EINVAL, "N=%lld exceeds 2^30", (long long)n);
    return NBODY_OK;
}

// A pair evaluation in p.passes passes over band ranges (compact layout: the
// scratch holds one pass's sums, reused, and the running totals). The last pass
// writes acc/pot, or for a step the accelerations that the Euler kernel reads.
int enqueue_pair_passes(const float4 *pos, int n, float eps2, float4 *acc_out, float *pot_out,
                        const nbody_plan &p, int dev, hipStream_t stream, float4 *euler_pos,
                        float4 *euler_vel, float dt)
{
    const bool step = euler_pos != nullptr;
    const int nb = p.splits, band = p.band, nruns = nbk::pair_runs(nb, p.run);
    const int64_t per = (nb + p.passes - 1) / p.passes;
    const int64_t own_max = per * band < n ? per * band : n;
    void *ws = nullptr;
    int rc = scratch_get(dev, stream, pairs_pass_scratch(n, band, p.run, p.passes, step), &ws);
    if (rc != NBODY_OK) return rc;
    float4 *own = (float4 *)ws;
    float4 *partner = own + (size_t)(1 + nruns) * (size_t)own_max;
    float4 *tot_s = partner + (size_t)per * (size_t)n;
    float4 *tot_e = tot_s + n;
    float4 *accbuf = step ? tot_e + n : nullptr;
    for (int64_t q = 0; q < p.passes; ++q) {
        const int b0 = pass_band(q, nb, p.passes), b1 = pass_band(q + 1, nb, p.passes);
        const int own0 = b0 * band;
        const int own_end = (int64_t)b1 * band < n ? b1 * band : n;
        nbk::PairsArgs pa{pos, n, eps2, nb, b0, b1, p.run, nruns, own, own_end - own0, own0,
                          partner, n, 1};
        hipError_t e = timed_launch(
            stream, [&] { return nbk::launch_pairs(band, p.tpl, pot_out != nullptr, pa, stream); });
        if (e != hipSuccess) return hip_fail(e, "accel kernel launch");
        nbk::PassArgs ca{own, partner, n, band, nb, p.run, b0, b1, own0, own_end - own0, tot_s, tot_e,
                         q == 0, q + 1 == p.passes, step ? accbuf : acc_out,
                         step ? nullptr : pot_out};
        e = nbk::launch_pass_combine(ca, stream);
        if (e != hipSuccess) return hip_fail(e, "pass combine launch");
    }
    if (step) {
        hipError_t e = nbk::launch_euler(accbuf, n, 1, euler_pos, euler_vel, dt, stream);
        if (e != hipSuccess) return hip_fail(e, "euler kernel launch");
    }
    return NBODY_OK;
}

// Enqueue one evaluation: acc/pot into acc_out/pot_out, or with euler_pos and
// euler_vel set, one Euler step applied to them in place (tiles and pairs
// modes; small-mode steps alternate buffers and go through enqueue_steps).
int enqueue_eval(const float4 *pos, int n, float eps2, float4 *acc_out, float *pot_out,
                 const nbody_plan &p, int dev, hipStream_t stream, float4 *euler_pos,
                 float4 *euler_vel, float dt)
{
    const bool pot = pot_out != nullptr;
    const bool step = euler_pos != nullptr;
    const bool pairs = p.mode == NBODY_MODE_PAIRS;
    if (p.mode == NBODY_MODE_SMALL) {
        if (step) return fail(NBODY_EINVAL, "internal: small-mode steps go through enqueue_steps");
        nbk::SmallArgs sa{pos, n, eps2, acc_out, pot_out, nullptr, nullptr, 0.0f};
        hipError_t e = timed_launch(stream,
                                    [&] { return nbk::launch_small(p.tpl, pot, false, sa, stream); });
        return e == hipSuccess ? NBODY_OK : hip_fail(e, "small kernel launch");
    }
    if (pairs && p.passes > 1)
        return enqueue_pair_passes(pos, n, eps2, acc_out, pot_out, p, dev, stream, euler_pos,
                                   euler_vel, dt);
    if (pairs) {
        void *ws = nullptr;
        int rc = scratch_get(dev, stream, pairs_scratch(n, p.band, p.run), &ws);
        if (rc != NBODY_OK) return rc;
        float4 *part = (float4 *)ws;
        const int nb = p.splits, nruns = nbk::pair_runs(nb, p.run);
        nbk::PairsArgs pa{pos, n, eps2, nb, 0, nb, p.run, nruns, part, n, 0,
                          part + (size_t)(1 + nruns) * (size_t)n, n, 0};
        hipError_t e = timed_launch(stream, [&] { return nbk::launch_pairs(p.band, p.tpl, pot, pa, stream); });
        if (e != hipSuccess) return hip_fail(e, "accel kernel launch");
        nbk::PairsFinishArgs fa{part, n, p.band, nb, p.run, acc_out, pot_out, euler_pos, euler_vel, dt};
        e = nbk::launch_pairs_finish(fa, stream);
        return e == hipSuccess ? NBODY_OK : hip_fail(e, "pair finish launch");
    }
    nbk::AccelArgs a{pos, n, eps2, p.chunk, acc_out, pot_out, nullptr};
    if (p.splits > 1 || step) {
        void *ws = nullptr;
        const size_t bytes = (size_t)p.splits * (size_t)n * sizeof(float4);
        int rc = scratch_get(dev, stream, bytes, &ws);
        if (rc != NBODY_OK) return rc;
        a.part = (float4 *)ws;
    }
    hipError_t e = timed_launch(stream, [&] {
        return nbk::launch_accel(p.bcast, p.tpl, p.wg, pot, grid_x(n, p.tpl, p.wg),
                                 (unsigned)p.splits, a, stream);
    });
    if (e != hipSuccess) return hip_fail(e, "accel kernel launch");
    if (step) {
        e = nbk::launch_euler(a.part, n, p.splits, euler_pos, euler_vel, dt, stream);
        if (e != hipSuccess) return hip_fail(e, "euler kernel launch");
    } else if (a.part) {
        e = nbk::launch_combine(a.part, n, p.splits, acc_out, pot_out, stream);
        if (e != hipSuccess) return hip_fail(e, "combine kernel launch");
    }
    return NBODY_OK;
}

int accel_impl(const nbody_f4 *pos, int64_t N, float eps2, nbody_f4 *acc, float *pot,
               const nbody_plan *plan, hipStream_t stream)
{
    int rc = check_n(N);
    if (rc != NBODY_OK) return rc;
    if (N == 0) return ok();
    if (!pos) return fail(NBODY_EINVAL, "pos_xyzm is NULL");
    if (!acc) return fail(NBODY_EINVAL, "acc_out is NULL");
    if (!eps2_ok(eps2))
        return eps2_fail(eps2);
    if (!aligned(pos, 16)) return fail(NBODY_EALIGN, "pos_xyzm is not 16-byte aligned");
    if (!aligned(acc, 16)) return fail(NBODY_EALIGN, "acc_out is not 16-byte aligned");
    if (pot && !aligned(pot, 4)) return fail(NBODY_EALIGN, "pot_out is not 4-byte aligned");
    const size_t b16 = (size_t)N * 16, b4 = (size_t)N * 4;
    if (overlap(pos, b16, acc, b16)) return fail(NBODY_EINVAL, "acc_out overlaps pos_xyzm");
    if (pot && (overlap(pot, b4, pos, b16) || overlap(pot, b4, acc, b16)))
        return fail(NBODY_EINVAL, "pot_out overlaps another buffer");
    nbody_plan p;
    int dev = 0;
    rc = make_plan(N, plan, &dev, &p);
    if (rc != NBODY_OK) return rc;
    rc = enqueue_eval((const float4 *)pos, (int)N, eps2, (float4 *)acc, pot, p, dev, stream,
                      nullptr, nullptr, 0.0f);
    return rc == NBODY_OK ? ok() : rc;
}

// Scratch bytes an evaluation (or, with step, a step loop) of plan p uses from
// the start of the (device, stream) block.
size_t eval_scratch(int64_t n, const nbody_plan &p, bool step)
{
    if (p.mode == NBODY_MODE_SMALL) return step ? (size_t)n * sizeof(float4) : 0;
    if (p.mode == NBODY_MODE_PAIRS && p.passes > 1)
        return pairs_pass_scratch(n, p.band, p.run, p.passes, step);
    if (p.mode == NBODY_MODE_PAIRS) return pairs_scratch(n, p.band, p.run);
    if (p.splits > 1 || step) return (size_t)p.splits * (size_t)n * sizeof(float4);
    return 0;
}

// nsteps Euler steps of (pos, vel) in place with plan p.
int enqueue_steps(float4 *pos, float4 *vel, int n, float dt, float eps2, int64_t nsteps,
                  const nbody_plan &p, int dev, hipStream_t stream)
{
    if (p.mode != NBODY_MODE_SMALL) {
        for (int64_t s = 0; s < nsteps; ++s) {
            int rc = enqueue_eval(pos, n, eps2, nullptr, nullptr, p, dev, stream, pos, vel, dt);
            if (rc != NBODY_OK) return rc;
        }
        return NBODY_OK;
    }
    // One kernel per step reads every position while it writes new ones, so the
    // steps alternate between the caller's array and a scratch copy; after an
    // odd step count the final positions are copied back on the stream.
    const size_t b16 = (size_t)n * sizeof(float4);
    void *ws = nullptr;
    int rc = scratch_get(dev, stream, b16, &ws);
    if (rc != NBODY_OK) return rc;
    float4 *other = (float4 *)ws;
    for (int64_t s = 0; s < nsteps; ++s) {
        float4 *src = (s % 2 == 0) ? pos : other;
        float4 *dst = (s % 2 == 0) ? other : pos;
        nbk::SmallArgs sa{src, n, eps2, nullptr, nullptr, dst, vel, dt};
        hipError_t e =
            timed_launch(stream, [&] { return nbk::launch_small(p.tpl, false, true, sa, stream); });
        if (e != hipSuccess) return hip_fail(e, "small kernel launch");
    }
    if (nsteps % 2 == 1) {
        hipError_t e = hipMemcpyAsync(pos, other, b16, hipMemcpyDeviceToDevice, stream);
        if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync(positions)");
    }
    return NBODY_OK;
}

// noalloc: take the scratch from the static array (nbody_step_noalloc) and
// reject plans that need more than it holds; nothing is allocated.
int step_impl(nbody_f4 *pos, nbody_f4 *vel, int64_t N, float dt, float eps2, int64_t nsteps,
              const nbody_plan *plan, hipStream_t stream, bool noalloc = false)
{
    int rc = check_n(N);
    if (rc != NBODY_OK) return rc;
    if (nsteps < 0) return fail(NBODY_EINVAL, "nsteps=%lld must be >= 0", (long long)nsteps);
    if (N == 0 || nsteps == 0) return ok();
    if (!pos) return fail(NBODY_EINVAL, "pos is NULL");
    if (!vel) return fail(NBODY_EINVAL, "vel is NULL");
    if (!std::isfinite(dt)) return fail(NBODY_EINVAL, "dt=%g must be finite", (double)dt);
    if (!eps2_ok(eps2))
        return eps2_fail(eps2);
    if (!aligned(pos, 16)) return fail(NBODY_EALIGN, "pos is not 16-byte aligned");
    if (!aligned(vel, 16)) return fail(NBODY_EALIGN, "vel is not 16-byte aligned");
    const size_t b16 = (size_t)N * 16;
    if (overlap(pos, b16, vel, b16)) return fail(NBODY_EINVAL, "vel overlaps pos");
    nbody_plan p;
    int dev = 0;
    rc = make_plan(N, plan, &dev, &p);
    if (rc != NBODY_OK) return rc;
    if (!noalloc) {
        rc = enqueue_steps((float4 *)pos, (float4 *)vel, (int)N, dt, eps2, nsteps, p, dev, stream);
        return rc == NBODY_OK ? ok() : rc;
    }
    const size_t need = eval_scratch(N, p, true);
    if (need > kStaticScratchBytes)
        return fail(NBODY_EINVAL, "N=%lld: its step plan needs %zu bytes of scratch, more than the "
                                  "%zu of nbody_step_noalloc's static array (use nbody_step)",
                    (long long)N, need, kStaticScratchBytes);
    void *fixed = nullptr;
    rc = static_scratch(dev, &fixed);
    if (rc != NBODY_OK) return rc;
    FixedScratchScope scope(fixed, kStaticScratchBytes);
    rc = enqueue_steps((float4 *)pos, (float4 *)vel, (int)N, dt, eps2, nsteps, p, dev, stream);
    return rc == NBODY_OK ? ok() : rc;
}

// ------------------------------------------------------------ SoA entry points

bool disjoint(const void *const *p, const size_t *bytes, int k)
{
    for (int i = 0; i < k; ++i)
        for (int j = i + 1; j < k; ++j)
            if (p[i] && p[j] && overlap(p[i], bytes[i], p[j], bytes[j])) return false;
    return true;
}

size_t align256(size_t b) { return (b + 255) / 256 * 256; }

int accel_soa_impl(const float *x, const float *y, const float *z, const float *m, int64_t N,
                   float eps2, float *ax, float *ay, float *az, float *pot, hipStream_t stream)
{
    int rc = check_n(N);
    if (rc != NBODY_OK) return rc;
    if (N == 0) return ok();
    const float *in[4] = {x, y, z, m};
    float *out[3] = {ax, ay, az};
    const char *in_name[4] = {"x", "y", "z", "m"}, *out_name[3] = {"ax", "ay", "az"};
    for (int i = 0; i < 4; ++i) {
        if (!in[i]) return fail(NBODY_EINVAL, "%s is NULL", in_name[i]);
        if (!aligned(in[i], 4)) return fail(NBODY_EALIGN, "%s is not 4-byte aligned", in_name[i]);
    }
    for (int i = 0; i < 3; ++i) {
        if (!out[i]) return fail(NBODY_EINVAL, "%s is NULL", out_name[i]);
        if (!aligned(out[i], 4)) return fail(NBODY_EALIGN, "%s is not 4-byte aligned", out_name[i]);
    }
    if (pot && !aligned(pot, 4)) return fail(NBODY_EALIGN, "pot is not 4-byte aligned");
    if (!eps2_ok(eps2))
        return eps2_fail(eps2);
    const size_t b4 = (size_t)N * 4;
    const void *all[8] = {ax, ay, az, pot, x, y, z, m};
    const size_t sz[8] = {b4, b4, b4, b4, b4, b4, b4, b4};
    // outputs must not overlap each other or the inputs (inputs may share storage)
    for (int o = 0; o < 4; ++o)
        for (int j = 0; j < 8; ++j)
            if (j != o && all[o] && all[j] && overlap(all[o], sz[o], all[j], sz[j]))
                return fail(NBODY_EINVAL, "an output array overlaps another array");
    nbody_plan p;
    int dev = 0;
    rc = make_plan(N, nullptr, &dev, &p);
    if (rc != NBODY_OK) return rc;
    const size_t b16 = (size_t)N * 16, base = align256(eval_scratch(N, p, false));
    void *ws = nullptr;
    rc = scratch_get(dev, stream, base + 2 * b16, &ws);
    if (rc != NBODY_OK) return rc;
    float4 *pos4 = (float4 *)((char *)ws + base), *acc4 = pos4 + N;
    hipError_t e = nbk::launch_pack(x, y, z, m, (int)N, pos4, stream);
    if (e != hipSuccess) return hip_fail(e, "pack kernel launch");
    rc = enqueue_eval(pos4, (int)N, eps2, acc4, pot, p, dev, stream, nullptr, nullptr, 0.0f);
    if (rc != NBODY_OK) return rc;
    e = nbk::launch_unpack(acc4, (int)N, ax, ay, az, stream);
    if (e != hipSuccess) return hip_fail(e, "unpack kernel launch");
    return ok();
}

int step_soa_impl(float *x, float *y, float *z, const float *m, float *vx, float *vy, float *vz,
                  int64_t N, float dt, float eps2, int64_t nsteps, hipStream_t stream)
{
    int rc = check_n(N);
    if (rc != NBODY_OK) return rc;
    if (nsteps < 0) return fail(NBODY_EINVAL, "nsteps=%lld must be >= 0", (long long)nsteps);
    if (N == 0 || nsteps == 0) return ok();
    const void *arr[7] = {x, y, z, m, vx, vy, vz};
    const char *name[7] = {"x", "y", "z", "m", "vx", "vy", "vz"};
    for (int i = 0; i < 7; ++i) {
        if (!arr[i]) return fail(NBODY_EINVAL, "%s is NULL", name[i]);
        if (!aligned(arr[i], 4)) return fail(NBODY_EALIGN, "%s is not 4-byte aligned", name[i]);
    }
    if (!std::isfinite(dt)) return fail(NBODY_EINVAL, "dt=%g must be finite", (double)dt);
    if (!eps2_ok(eps2))
        return eps2_fail(eps2);
    const size_t b4 = (size_t)N * 4;
    const size_t sz[7] = {b4, b4, b4, b4, b4, b4, b4};
    if (!disjoint(arr, sz, 7)) return fail(NBODY_EINVAL, "the seven arrays must not overlap");
    nbody_plan p;
    int dev = 0;
    rc = make_plan(N, nullptr, &dev, &p);
    if (rc != NBODY_OK) return rc;
    const size_t b16 = (size_t)N * 16, base = align256(eval_scratch(N, p, true));
    void *ws = nullptr;
    rc = scratch_get(dev, stream, base + 2 * b16, &ws);
    if (rc != NBODY_OK) return rc;
    float4 *pos4 = (float4 *)((char *)ws + base), *vel4 = pos4 + N;
    hipError_t e = nbk::launch_pack(x, y, z, m, (int)N, pos4, stream);
    if (e == hipSuccess) e = nbk::launch_pack(vx, vy, vz, nullptr, (int)N, vel4, stream);
    if (e != hipSuccess) return hip_fail(e, "pack kernel launch");
    rc = enqueue_steps(pos4, vel4, (int)N, dt, eps2, nsteps, p, dev, stream);
    if (rc != NBODY_OK) return rc;
    e = nbk::launch_unpack(pos4, (int)N, x, y, z, stream);
    if (e == hipSuccess) e = nbk::launch_unpack(vel4, (int)N, vx, vy, vz, stream);
    if (e != hipSuccess) return hip_fail(e, "unpack kernel launch");
    return ok();
}

// First band of shard s when nb bands are split into S contiguous ranges.
int shard_band(int s, int nb, int S) { return (int)((int64_t)s * nb / S); }

int shard_impl(const nbody_f4 *pos, int64_t N, float eps2, int32_t shard, int32_t nshards,
               int want_pot, const nbody_plan *plan, nbody_f4 *partial_out, hipStream_t stream)
{
    int rc = check_n(N);
    if (rc != NBODY_OK) return rc;
    if (nshards < 1) return fail(NBODY_EINVAL, "nshards=%d must be >= 1", (int)nshards);
    if (shard < 0 || shard >= nshards)
        return fail(NBODY_EINVAL, "shard=%d must be in [0, nshards=%d)", (int)shard, (int)nshards);
    if (plan && plan->mode != NBODY_MODE_PAIRS)
        return fail(NBODY_EINVAL, "plan.mode=%d: a shard is a share of the pair-symmetric "
                                  "evaluation (plan NULL or mode NBODY_MODE_PAIRS)", plan->mode);
    if (N == 0) return ok();
    if (!pos) return fail(NBODY_EINVAL, "pos_xyzm is NULL");
    if (!partial_out) return fail(NBODY_EINVAL, "partial_out is NULL");
    if (!eps2_ok(eps2))
        return eps2_fail(eps2);
    if (!aligned(pos, 16) || !aligned(partial_out, 16))
        return fail(NBODY_EALIGN, "pos_xyzm and partial_out must be 16-byte aligned");
    const size_t b16 = (size_t)N * 16;
    if (overlap(pos, b16, partial_out, b16))
        return fail(NBODY_EINVAL, "partial_out overlaps pos_xyzm");
    if (plan && valid_band(plan->band) && nshards > (N + plan->band - 1) / plan->band)
        return fail(NBODY_EINVAL, "nshards=%d exceeds the %lld bands of %d bodies (each shard "
                                  "needs at least one band)", (int)nshards,
                    (long long)((N + plan->band - 1) / plan->band), (int)plan->band);
    nbody_plan want = plan ? *plan : nbody_plan{0, 0, 0, 0, 0, NBODY_MODE_PAIRS, 0, 0, 0};
    nbody_plan p;
    int dev = 0;
    rc = make_plan(N, &want, &dev, &p);
    if (rc != NBODY_OK) return rc;
    const int nb = p.splits;
    if (nshards > nb)
        return fail(NBODY_EINVAL, "nshards=%d exceeds the %d bands of %d bodies (each shard "
                                  "needs at least one band)", (int)nshards, nb, (int)p.band);
    void *ws = nullptr;
    rc = scratch_get(dev, stream, pairs_scratch(N, p.band, p.run), &ws);  // the one-pass layout
    if (rc != NBODY_OK) return rc;
    const int n = (int)N, nruns = nbk::pair_runs(nb, p.run);
    float4 *part = (float4 *)ws;
    nbk::PairsArgs pa{(const float4 *)pos, n, eps2, nb, shard_band(shard, nb, nshards),
                      shard_band(shard + 1, nb, nshards), p.run, nruns, part, n, 0,
                      part + (size_t)(1 + nruns) * (size_t)n, n, 0};
    hipError_t e = timed_launch(
        stream, [&] { return nbk::launch_pairs(p.band, p.tpl, want_pot != 0, pa, stream); });
    if (e != hipSuccess) return hip_fail(e, "accel kernel launch");
    e = nbk::launch_shard_combine(part, n, p.band, nb, p.run, pa.band0, pa.band1,
                                  (float4 *)partial_out, stream);
    if (e != hipSuccess) return hip_fail(e, "shard combine launch");
    return ok();
}

}  // namespace

extern "C" {

int nbody_accel(const nbody_f4 *pos_xyzm, int64_t N, float eps2, nbody_f4 *acc_out,
                float *pot_out, hipStream_t stream)
{
    EnqueueLock lk(g_enqueue);
    timer_arm();
    return accel_impl(pos_xyzm, N, eps2, acc_out, pot_out, nullptr, stream);
}

int nbody_accel_plan(const nbody_f4 *pos_xyzm, int64_t N, float eps2, nbody_f4 *acc_out,
                     float *pot_out, const nbody_plan *plan, hipStream_t stream)
{
    EnqueueLock lk(g_enqueue);
    timer_arm();
    return accel_impl(pos_xyzm, N, eps2, acc_out, pot_out, plan, stream);
}

int nbody_step(nbody_f4 *pos, nbody_f4 *vel, int64_t N, float dt, float eps2, int64_t nsteps,
               hipStream_t stream)
{
    EnqueueLock lk(g_enqueue);
    timer_arm();
    return step_impl(pos, vel, N, dt, eps2, nsteps, nullptr, stream);
}

int nbody_step_plan(nbody_f4 *pos, nbody_f4 *vel, int64_t N, float dt, float eps2,
                    int64_t nsteps, const nbody_plan *plan, hipStream_t stream)
{
    EnqueueLock lk(g_enqueue);
    timer_arm();
    return step_impl(pos, vel, N, dt, eps2, nsteps, plan, stream);
}

int nbody_step_noalloc(nbody_f4 *pos, nbody_f4 *vel, int64_t N, float dt, float eps2,
                       int64_t nsteps, hipStream_t stream)
{
    EnqueueLock lk(g_enqueue);
    timer_arm();
    return step_impl(pos, vel, N, dt, eps2, nsteps, nullptr, stream, true);
}

int nbody_time_kernel(hipEvent_t start, hipEvent_t stop)
{
    if ((start == nullptr) != (stop == nullptr))
        return fail(NBODY_EINVAL, "start and stop must both be events or both be NULL");
    g_timer = KernelTimer{start, stop, false};
    return ok();
}

int nbody_accel_soa(const float *x, const float *y, const float *z, const float *m, int64_t N,
                    float eps2, float *ax, float *ay, float *az, float *pot_out,
                    hipStream_t stream)
{
    EnqueueLock lk(g_enqueue);
    timer_arm();
    return accel_soa_impl(x, y, z, m, N, eps2, ax, ay, az, pot_out, stream);
}

int nbody_step_soa(float *x, float *y, float *z, const float *m, float *vx, float *vy, float *vz,
                   int64_t N, float dt, float eps2, int64_t nsteps, hipStream_t stream)
{
    EnqueueLock lk(g_enqueue);
    timer_arm();
    return step_soa_impl(x, y, z, m, vx, vy, vz, N, dt, eps2, nsteps, stream);
}

int nbody_accel_shard(const nbody_f4 *pos_xyzm, int64_t N, float eps2, int32_t shard,
                      int32_t nshards, int want_pot, const nbody_plan *plan,
                      nbody_f4 *partial_out, hipStream_t stream)
{
    EnqueueLock lk(g_enqueue);
    timer_arm();
    return shard_impl(pos_xyzm, N, eps2, shard, nshards, want_pot, plan, partial_out, stream);
}

int nbody_shard_finish(const nbody_f4 *partials, int64_t N, int32_t nshards, int64_t t0,
                       int64_t t1, nbody_f4 *acc_out, float *pot_out, hipStream_t stream)
{
    int rc = check_n(N);
    if (rc != NBODY_OK) return rc;
    if (nshards < 1) return fail(NBODY_EINVAL, "nshards=%d must be >= 1", (int)nshards);
    if (t0 < 0 || t1 < t0 || t1 > N)
        return fail(NBODY_EINVAL, "target range [%lld, %lld) must lie in [0, N=%lld]",
                    (long long)t0, (long long)t1, (long long)N);
    if ((int64_t)nshards * N > INT64_MAX / 16)
        return fail(NBODY_EINVAL, "nshards x N records do not fit the address space");
    if (t0 == t1) return ok();
    if (!partials) return fail(NBODY_EINVAL, "partials is NULL");
    if (!acc_out) return fail(NBODY_EINVAL, "acc_out is NULL");
    if (!aligned(partials, 16) || !aligned(acc_out, 16))
        return fail(NBODY_EALIGN, "partials and acc_out must be 16-byte aligned");
    if (pot_out && !aligned(pot_out, 4)) return fail(NBODY_EALIGN, "pot_out is not 4-byte aligned");
    const size_t bp = (size_t)nshards * (size_t)N * 16, m = (size_t)(t1 - t0);
    if (overlap(partials, bp, acc_out, m * 16) || (pot_out && overlap(partials, bp, pot_out, m * 4)))
        return fail(NBODY_EINVAL, "an output overlaps partials");
    if (pot_out && overlap(acc_out, m * 16, pot_out, m * 4))
        return fail(NBODY_EINVAL, "pot_out overlaps acc_out");
    hipError_t e = nbk::launch_shard_finish((const float4 *)partials, (int)N, nshards, (int)t0,
                                            (int)t1, (float4 *)acc_out, pot_out, stream);
    if (e != hipSuccess) return hip_fail(e, "shard finish launch");
    return ok();
}

int nbody_p2p(const nbody_f4 *pos, int64_t N, float eps2, const int32_t *cell_start,
              int32_t ncell, const int32_t *list_off, const int32_t *cells, int64_t nlist,
              nbody_f4 *acc_out, float *pot_out, hipStream_t stream)
{
    int rc = check_n(N);
    if (rc != NBODY_OK) return rc;
    if (ncell < 0) return fail(NBODY_EINVAL, "ncell=%d must be >= 0", (int)ncell);
    if (nlist < 0 || nlist > INT32_MAX)
        return fail(NBODY_EINVAL, "nlist=%lld must be in [0, 2^31 - 1]", (long long)nlist);
    if (N == 0 || ncell == 0) return ok();
    if (!pos) return fail(NBODY_EINVAL, "pos_xyzm is NULL");
    if (!acc_out) return fail(NBODY_EINVAL, "acc_out is NULL");
    if (!cell_start || !list_off) return fail(NBODY_EINVAL, "cell_start or list_off is NULL");
    if (nlist > 0 && !cells) return fail(NBODY_EINVAL, "cells is NULL");
    if (!eps2_ok(eps2))
        return eps2_fail(eps2);
    if (!aligned(pos, 16) || !aligned(acc_out, 16))
        return fail(NBODY_EALIGN, "pos_xyzm and acc_out must be 16-byte aligned");
    if ((pot_out && !aligned(pot_out, 4)) || !aligned(cell_start, 4) || !aligned(list_off, 4) ||
        (cells && !aligned(cells, 4)))
        return fail(NBODY_EALIGN, "pot_out and the index arrays must be 4-byte aligned");
    const size_t b16 = (size_t)N * 16, b4 = (size_t)N * 4, bc = ((size_t)ncell + 1) * 4;
    const void *outs[2] = {acc_out, pot_out};
    const size_t osz[2] = {b16, b4};
    const void *ins[4] = {pos, cell_start, list_off, cells};
    const size_t isz[4] = {b16, bc, bc, (size_t)nlist * 4};
    for (int o = 0; o < 2; ++o) {
        if (!outs[o]) continue;
        for (int j = 0; j < 4; ++j)
            if (ins[j] && isz[j] && overlap(outs[o], osz[o], ins[j], isz[j]))
                return fail(NBODY_EINVAL, "an output overlaps an input");
    }
    if (pot_out && overlap(acc_out, b16, pot_out, b4))
        return fail(NBODY_EINVAL, "pot_out overlaps acc_out");
    timer_arm();
    nbk::P2PArgs a{(const float4 *)pos, (int)N, eps2, cell_start, ncell, list_off, cells,
                   (long long)nlist, (float4 *)acc_out, pot_out, nullptr};
    hipError_t e =
        timed_launch(stream, [&] { return nbk::launch_p2p(pot_out != nullptr, a, stream); });
    if (e != hipSuccess) return hip_fail(e, "p2p kernel launch");
    return ok();
}

int nbody_near_grid(const nbody_f4 *pos, int64_t N, float eps2, const float lo[3], float h,
                    const int32_t dims[3], nbody_f4 *acc_out, float *pot_out, hipStream_t stream)
{
    return nbody_near_grid_kernel(pos, N, eps2, lo, h, dims, NBODY_NEAR_AUTO, acc_out, pot_out,
                                  stream);
}

int nbody_near_grid_kernel(const nbody_f4 *pos, int64_t N, float eps2, const float lo[3], float h,
                           const int32_t dims[3], int32_t kernel, nbody_f4 *acc_out,
                           float *pot_out, hipStream_t stream)
{
    if (kernel < NBODY_NEAR_AUTO || kernel > NBODY_NEAR_PAIRS)
        return fail(NBODY_EINVAL, "kernel=%d is not a NBODY_NEAR_* value", (int)kernel);
    int rc = check_n(N);
    if (rc != NBODY_OK) return rc;
    if (!lo || !dims) return fail(NBODY_EINVAL, "lo or dims is NULL");
    int64_t ncell = 1;
    for (int d = 0; d < 3; ++d) {
        if (dims[d] < 1) return fail(NBODY_EINVAL, "dims[%d]=%d must be >= 1", d, (int)dims[d]);
        if (!std::isfinite(lo[d])) return fail(NBODY_EINVAL, "lo[%d] is not finite", d);
        ncell *= dims[d];
        if (ncell > kMaxGridCells)
            return fail(NBODY_EINVAL, "dims hold more than %lld cells", (long long)kMaxGridCells);
    }
    const float inv_h = 1.0f / h;
    if (!(h >= FLT_MIN) || !std::isfinite(h) || !std::isfinite(inv_h))
        return fail(NBODY_EINVAL, "h=%g must be a positive, finite, normal float with a finite "
                                  "reciprocal", (double)h);
    if (N == 0) return ok();
    if (!pos) return fail(NBODY_EINVAL, "pos_xyzm is NULL");
    if (!acc_out) return fail(NBODY_EINVAL, "acc_out is NULL");
    if (!eps2_ok(eps2))
        return eps2_fail(eps2);
    if (!aligned(pos, 16) || !aligned(acc_out, 16))
        return fail(NBODY_EALIGN, "pos_xyzm and acc_out must be 16-byte aligned");
    if (pot_out && !aligned(pot_out, 4)) return fail(NBODY_EALIGN, "pot_out is not 4-byte aligned");
    const size_t b16 = (size_t)N * 16, b4 = (size_t)N * 4;
    if (overlap(pos, b16, acc_out, b16)) return fail(NBODY_EINVAL, "acc_out overlaps pos_xyzm");
    if (pot_out && (overlap(pot_out, b4, pos, b16) || overlap(pot_out, b4, acc_out, b16)))
        return fail(NBODY_EINVAL, "pot_out overlaps another buffer");
    EnqueueLock lk(g_enqueue);
    timer_arm();
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    nbk::GridSpec g{{lo[0], lo[1], lo[2]}, inv_h, {dims[0], dims[1], dims[2]}};
    const int n = (int)N, nc = (int)ncell;
    bool pairs = kernel == NBODY_NEAR_PAIRS;
    if (kernel == NBODY_NEAR_AUTO && N >= kSymMinMean * ncell && N <= kSymMaxMean * ncell) {
        DeviceFacts facts;
        rc = device_facts(dev, &facts);
        if (rc != NBODY_OK) return rc;
        // and while its slots (kSymSlots records per body) fit the pair mode's share of
        // device memory; beyond that the one-sided kernel needs none
        pairs = ncell >= kSymMinCellsPerCU * facts.cus &&
                (size_t)nbk::kSymSlots * b16 <= facts.mem_bytes / kPairsScratchShare;
    }
    int end_bit = 1;
    while (end_bit < 32 && ((int64_t)1 << end_bit) < ncell) ++end_bit;
    const size_t sort_bytes = nbk::sort_temp_bytes(n);
    // scratch: keys, idx, sorted keys, perm (N x 4 each), sorted pos (N x 16), cell starts
    // ((ncell + 1) x 4), sort temp, and for the pair-symmetric kernel its slots. The
    // one-sided kernel, or the pair finish, writes each body's results straight to its
    // place in the caller's order (perm).
    size_t off[9];
    const size_t sz[8] = {b4, b4, b4, b4, b16, ((size_t)nc + 1) * 4, sort_bytes,
                          pairs ? (size_t)nbk::kSymSlots * b16 : 0};
    off[0] = 0;
    for (int i = 0; i < 8; ++i) off[i + 1] = align256(off[i] + sz[i]);
    void *ws = nullptr;
    rc = scratch_get(dev, stream, off[8], &ws);
    if (rc != NBODY_OK) return rc;
    char *b = (char *)ws;
    unsigned *keys = (unsigned *)(b + off[0]), *skeys = (unsigned *)(b + off[2]);
    int *idx = (int *)(b + off[1]), *perm = (int *)(b + off[3]);
    float4 *spos = (float4 *)(b + off[4]);
    int *start = (int *)(b + off[5]);
    void *temp = b + off[6];
    e = nbk::launch_grid_keys((const float4 *)pos, n, g, keys, idx, stream);
    if (e == hipSuccess)
        e = nbk::sort_pairs(temp, keys, skeys, idx, perm, n, end_bit, stream);
    if (e == hipSuccess) e = nbk::launch_gather((const float4 *)pos, perm, n, spos, stream);
    if (e == hipSuccess) e = nbk::launch_cell_starts(skeys, n, nc, start, stream);
    if (e == hipSuccess && pairs) {
        float4 *part = (float4 *)(b + off[7]);
        e = timed_launch(stream, [&] {
            return nbk::launch_p2p_sym(pot_out != nullptr, spos, n, eps2, start, g, part, stream);
        });
        if (e == hipSuccess)
            e = nbk::launch_sym_finish(part, n, skeys, start, g, perm, (float4 *)acc_out, pot_out,
                                       stream);
    } else if (e == hipSuccess) {
        nbk::P2PArgs a{spos, n, eps2, start, nc, nullptr, nullptr, 0, (float4 *)acc_out, pot_out,
                       perm};
        e = timed_launch(stream,
                         [&] { return nbk::launch_p2p_grid(pot_out != nullptr, a, g, stream); });
    }
    if (e != hipSuccess) return hip_fail(e, "near-grid launch");
    return ok();
}

int nbody_near_tree(const nbody_f4 *pos, int64_t N, float eps2, int64_t leaf_size,
                    nbody_f4 *acc_out, float *pot_out, nbody_tree_stats *stats,
                    hipStream_t stream)
{
    int rc = check_n(N);
    if (rc != NBODY_OK) return rc;
    if (N > kMaxTreeN) return fail(NBODY_EINVAL, "N=%lld exceeds 2^30", (long long)N);
    if (leaf_size < 1) return fail(NBODY_EINVAL, "leaf_size=%lld must be >= 1", (long long)leaf_size);
    if (stats) *stats = nbody_tree_stats{0, 0, 0};
    if (N == 0) return ok();
    if (!pos) return fail(NBODY_EINVAL, "pos_xyzm is NULL");
    if (!acc_out) return fail(NBODY_EINVAL, "acc_out is NULL");
    if (!eps2_ok(eps2))
        return eps2_fail(eps2);
    if (!aligned(pos, 16) || !aligned(acc_out, 16))
        return fail(NBODY_EALIGN, "pos_xyzm and acc_out must be 16-byte aligned");
    if (pot_out && !aligned(pot_out, 4)) return fail(NBODY_EALIGN, "pot_out is not 4-byte aligned");
    const size_t b16 = (size_t)N * 16, b4 = (size_t)N * 4;
    if (overlap(pos, b16, acc_out, b16)) return fail(NBODY_EINVAL, "acc_out overlaps pos_xyzm");
    if (pot_out && (overlap(pot_out, b4, pos, b16) || overlap(pot_out, b4, acc_out, b16)))
        return fail(NBODY_EINVAL, "pot_out overlaps another buffer");
    EnqueueLock lk(g_enqueue);
    timer_arm();
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    const int n = (int)N;
    const int S = leaf_size < N ? (int)leaf_size : n;  // a node never holds more than N
    // Scratch slot 0, sized by N: keys, idx, sorted keys, perm, sorted pos, leaf level and
    // leaf number of each sorted body, cell (leaf) starts, leaf keys and cubes, list
    // offsets, counters, frame, sort temp, scan temp, bounds temp.
    const size_t b8 = (size_t)N * 8, b4p = ((size_t)N + 1) * 4;
    const size_t sz[16] = {b8,  b4,  b8,  b4,  b16, b4,  b4,  b4p,
                           b8,  b16, b4p, 256, 16,  nbk::sort_temp_bytes(n, 8),
                           nbk::scan_temp_bytes(N), nbk::tree_frame_temp_bytes(n)};
    size_t off[17];
    off[0] = 0;
    for (int i = 0; i < 16; ++i) off[i + 1] = align256(off[i] + sz[i]);
    void *ws = nullptr;
    rc = scratch_get(dev, stream, off[16], &ws);
    if (rc != NBODY_OK) return rc;
    char *b = (char *)ws;
    auto *keys = (unsigned long long *)(b + off[0]), *skeys = (unsigned long long *)(b + off[2]);
    int *idx = (int *)(b + off[1]), *perm = (int *)(b + off[3]);
    float4 *spos = (float4 *)(b + off[4]);
    int *level = (int *)(b + off[5]), *ids = (int *)(b + off[6]), *start = (int *)(b + off[7]);
    auto *leaf_key = (unsigned long long *)(b + off[8]);
    int4 *leaf_box = (int4 *)(b + off[9]);
    int *list_off = (int *)(b + off[10]), *counters = (int *)(b + off[11]);
    float4 *frame = (float4 *)(b + off[12]);
    void *sort_temp = b + off[13], *scan_temp = b + off[14];
    float *bounds_temp = (float *)(b + off[15]);
    int host[nbk::kTreeCounters] = {0, 0, 0, 0, 0, 0};
    auto build = [&](hipStream_t s) {
        hipError_t x = nbk::launch_tree_frame((const float4 *)pos, n, bounds_temp, frame, counters, s);
        if (x == hipSuccess) x = nbk::launch_tree_keys((const float4 *)pos, n, frame, keys, idx, s);
        if (x == hipSuccess) x = nbk::sort_pairs64(sort_temp, keys, skeys, idx, perm, n, 63, s);
        if (x == hipSuccess) x = nbk::launch_gather((const float4 *)pos, perm, n, spos, s);
        if (x == hipSuccess) x = nbk::launch_tree_levels(skeys, n, S, level, ids, s);
        if (x == hipSuccess) x = nbk::scan_exclusive(ids, n, counters, scan_temp, s);
        if (x == hipSuccess)
            x = nbk::launch_tree_leaves(skeys, level, ids, n, start, leaf_key, leaf_box, s);
        return x;
    };
    e = run_graphed(TreeGraphKey{dev, 0, stream, {n, S, 0, 0, 0, 0}, {pos, ws, nullptr, nullptr, nullptr, nullptr}},
                    stream, build);
    // first wait: the number of leaves sizes the list counts
    if (e == hipSuccess) e = hipMemcpyAsync(host, counters, 4, hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return hip_fail(e, "near-tree build");
    const int nleaf = host[0];
    if (nleaf < 1 || nleaf > n)
        return fail(NBODY_EHIP, "near-tree build: %d leaves for %d bodies", nleaf, n);
    if (nleaf > nbk::kTreeMaxLeaves)
        return fail(NBODY_EINVAL, "near-tree: %d leaves exceed %d (raise leaf_size)", nleaf,
                    nbk::kTreeMaxLeaves);
    // Scratch slot 1, sized by the leaves: coarse table, list part counts, their scan
    // temp, per-workgroup totals of the count pass, and the parts' first entries kept by
    // the count pass for the fill pass (up to kTreeKeepMax per part and kTreeKeepBytes in
    // all; Plummer 65,536, leaf_size 64: the fill pass 62 -> ~10 us).
    const int lt = nbk::tree_table_level(nleaf);
    const long long parts = 27ll * nleaf + 1;
    const long long keep_fit = (long long)(nbk::kTreeKeepBytes / ((size_t)27 * nleaf * 4));
    const int keep_cap = keep_fit < nbk::kTreeKeepMax ? (int)keep_fit : nbk::kTreeKeepMax;
    const size_t s1[5] = {(((size_t)1 << (3 * lt)) + 1) * 4, (size_t)parts * 4,
                          nbk::scan_temp_bytes(parts), nbk::tree_parts_bytes(nleaf),
                          (size_t)27 * nleaf * keep_cap * 4};
    size_t o1[6];
    o1[0] = 0;
    for (int i = 0; i < 5; ++i) o1[i + 1] = align256(o1[i] + s1[i]);
    void *ws1 = nullptr;
    rc = scratch_get(dev, stream, o1[5], &ws1, 1);
    if (rc != NBODY_OK) return rc;
    char *b1 = (char *)ws1;
    int *table = (int *)(b1 + o1[0]), *cnt = (int *)(b1 + o1[1]);
    void *scan_temp1 = b1 + o1[2], *wg_totals = b1 + o1[3];
    int *keep = keep_cap > 0 ? (int *)(b1 + o1[4]) : nullptr;
    const nbk::TreeLeaves lv{leaf_key, leaf_box, table, start, nleaf, lt};
    auto count_lists = [&](hipStream_t s) {
        hipError_t x = nbk::launch_tree_table(leaf_key, counters, lt, table, s);
        if (x == hipSuccess)
            x = nbk::launch_tree_lists(lv, counters, wg_totals, cnt, nullptr, nullptr, 0, nullptr,
                                       keep, keep_cap, s);
        if (x == hipSuccess) x = nbk::scan_exclusive(cnt, parts, counters + 1, scan_temp1, s);
        return x;
    };
    // A leaf meets at most 27 leaves no smaller than itself (each holds a different one of
    // the 27 cells of its level around it). A leaf may meet any number of smaller ones, but
    // each such pair is also a pair of the smaller leaf with a larger one, of which that
    // leaf has at most 26; so all lists together hold at most 27 + 26 = 53 entries per
    // leaf. Their scratch is sized from the leaf count without a second wait (which
    // remains for leaf counts whose bound passes 2^31 - 1 entries).
    const long long bound = (long long)nbk::kTreeListsPerLeaf * nleaf;
    unsigned long long nlist = 0, terms = 0;
    auto read_totals = [&]() -> int {
        hipError_t x = hipMemcpyAsync(host, counters, sizeof(host), hipMemcpyDeviceToHost, stream);
        if (x == hipSuccess) x = hipStreamSynchronize(stream);
        if (x != hipSuccess) return hip_fail(x, "near-tree lists");
        std::memcpy(&nlist, host + 2, 8);
        std::memcpy(&terms, host + 4, 8);
        if (nlist > (unsigned long long)INT32_MAX)
            return fail(NBODY_EINVAL, "near-tree lists hold %llu entries (at most 2^31 - 1)",
                        nlist);
        if ((unsigned long long)(unsigned)host[1] != nlist)
            return fail(NBODY_EHIP, "near-tree build: list offsets end at %d, counted %llu",
                        host[1], nlist);
        return NBODY_OK;
    };
    long long cap = bound;
    void *lw = nullptr;
    int *list = nullptr;
    auto fill_lists = [&](hipStream_t s) {
        return nbk::launch_tree_lists(lv, counters, nullptr, nullptr, cnt, list, (int)cap, list_off,
                                      keep, keep_cap, s);
    };
    if (bound > INT32_MAX) {
        // the lists' true length sizes their scratch: a second wait, no graph
        e = count_lists(stream);
        if (e != hipSuccess) return hip_fail(e, "near-tree lists");
        rc = read_totals();
        if (rc != NBODY_OK) return rc;
        cap = (long long)nlist;
        rc = scratch_get(dev, stream, ((size_t)cap + 1) * 4, &lw, 2);
        if (rc != NBODY_OK) return rc;
        list = (int *)lw;
        e = fill_lists(stream);
    } else {
        rc = scratch_get(dev, stream, ((size_t)cap + 1) * 4, &lw, 2);
        if (rc != NBODY_OK) return rc;
        list = (int *)lw;
        e = run_graphed(TreeGraphKey{dev, 1, stream, {n, nleaf, lt, keep_cap, cap, S},
                                     {ws, ws1, lw, nullptr, nullptr, nullptr}},
                        stream, [&](hipStream_t s) {
                            hipError_t x = count_lists(s);
                            return x == hipSuccess ? fill_lists(s) : x;
                        });
    }
    if (e == hipSuccess) {
        nbk::P2PArgs a{spos, n, eps2, start, nleaf, list_off, list, cap, (float4 *)acc_out,
                       pot_out, perm};
        e = timed_launch(stream, [&] { return nbk::launch_p2p(pot_out != nullptr, a, stream); });
    }
    if (e != hipSuccess) return hip_fail(e, "near-tree launch");
    if (stats) {
        // the totals of this call: a wait for the whole call
        if (bound <= INT32_MAX) {
            rc = read_totals();
            if (rc != NBODY_OK) return rc;
            if ((long long)nlist > bound)
                return fail(NBODY_EHIP, "near-tree lists: %llu entries exceed the bound %lld",
                            nlist, bound);
        }
        *stats = nbody_tree_stats{nleaf, (int64_t)nlist, (int64_t)terms};
    }
    return ok();
}

int nbody_diagnostics(const nbody_f4 *pos, const nbody_f4 *vel, const float *pot, int64_t N,
                      float eps2, nbody_diag *out, hipStream_t stream)
{
    int rc = check_n(N);
    if (rc != NBODY_OK) return rc;
    if (!out) return fail(NBODY_EINVAL, "out is NULL");
    if (N > 0 && !pos) return fail(NBODY_EINVAL, "pos is NULL");
    if (N > 0 && !vel) return fail(NBODY_EINVAL, "vel is NULL");
    if (!eps2_ok(eps2))
        return eps2_fail(eps2);
    if (!aligned(out, 8)) return fail(NBODY_EALIGN, "out is not 8-byte aligned");
    if (pos && !aligned(pos, 16)) return fail(NBODY_EALIGN, "pos is not 16-byte aligned");
    if (vel && !aligned(vel, 16)) return fail(NBODY_EALIGN, "vel is not 16-byte aligned");
    if (pot && !aligned(pot, 4)) return fail(NBODY_EALIGN, "pot is not 4-byte aligned");
    const size_t b16 = (size_t)N * 16, b4 = (size_t)N * 4, bo = sizeof(nbody_diag);
    if (N > 0 && (overlap(out, bo, pos, b16) || overlap(out, bo, vel, b16) ||
                  (pot && overlap(out, bo, pot, b4))))
        return fail(NBODY_EINVAL, "out overlaps an input");
    EnqueueLock lk(g_enqueue);
    timer_arm();
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    // Scratch: [evaluation partials | acc (N x 16) | pot (N x 4) | workgroup sums]. The
    // evaluation takes its partials from the start of the same block.
    nbody_plan p{};
    size_t part_bytes = 0;
    if (!pot && N > 0) {
        rc = make_plan(N, nullptr, &dev, &p);
        if (rc != NBODY_OK) return rc;
        part_bytes = align256(eval_scratch(N, p, false));
    }
    const size_t eval_bytes = (!pot && N > 0) ? b16 + b4 : 0;
    const int nb = nbk::diag_blocks((int)N);
    const size_t sums_off = (part_bytes + eval_bytes + 255) / 256 * 256;
    const size_t total = sums_off + (size_t)nb * nbk::kDiagSums * sizeof(double);
    void *ws = nullptr;
    rc = scratch_get(dev, stream, total, &ws);
    if (rc != NBODY_OK) return rc;
    char *base = (char *)ws;
    const float *use_pot = pot;
    if (!pot && N > 0) {
        float4 *acc = (float4 *)(base + part_bytes);
        float *pp = (float *)(base + part_bytes + b16);
        rc = enqueue_eval((const float4 *)pos, (int)N, eps2, acc, pp, p, dev, stream, nullptr,
                          nullptr, 0.0f);
        if (rc != NBODY_OK) return rc;
        use_pot = pp;
    }
    e = nbk::launch_diagnostics((const float4 *)pos, (const float4 *)vel, use_pot, (int)N,
                                1.0 / std::sqrt((double)eps2), (double *)(base + sums_off),
                                (double *)out, stream);
    if (e != hipSuccess) return hip_fail(e, "diagnostics kernel launch");
    return ok();
}

int nbody_plan_for(int64_t N, int want_pot, nbody_plan *out)
{
    if (!out) return fail(NBODY_EINVAL, "out is NULL");
    int rc = check_n(N);
    if (rc != NBODY_OK) return rc;
    int dev = 0;
    nbody_plan p;
    (void)want_pot;
    rc = make_plan(N < 1 ? 1 : N, nullptr, &dev, &p);
    if (rc != NBODY_OK) return rc;
    *out = p;
    return ok();
}

const char *nbody_last_error(void) { return g_err.c_str(); }

int nbody_release_workspace(void)
{
    EnqueueLock el(g_enqueue);
    int rc = drop_tree_graphs();  // they hold scratch addresses
    std::lock_guard<std::mutex> lk(g_mu);
    for (auto &kv : g_scratch) {
        if (kv.second.ptr) {
            hipError_t e = hipFree(kv.second.ptr);
            if (e != hipSuccess && rc == NBODY_OK) rc = hip_fail(e, "hipFree(scratch)");
        }
    }
    g_scratch.clear();
    return rc == NBODY_OK ? ok() : rc;
}

const char *nbody_version(void) { return "direct_all_pairs_amd 0.1.0 (gfx950)"; }

}  // extern "C"
