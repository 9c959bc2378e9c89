/*
 * nbody.h - C ABI of the MI355X (gfx950) direct all-pairs softened-gravity library.
 *
 * What the library computes (G = 1, sums over ALL j including j = i):
 *   a_i = sum_j m_j (x_j - x_i) / (|x_j - x_i|^2 + eps2)^(3/2)
 *   p_i = -sum_j m_j / (|x_j - x_i|^2 + eps2)^(1/2)
 * and the explicit Euler update, position first with the old velocity:
 *   x^{n+1} = x^n + dt v^n,   v^{n+1} = v^n + dt a(x^n).
 * Sources on the pages:
 *   - Degawa, "N 体問題" lecture slides: slide 4 (acceleration sum), slide 12
 *     (softening instead of the j != i test; the self term has a zero
 *     numerator), slides 5-6 and the CPU program's integrate() on slide 15
 *     (Euler, always position first).
 *   - Nakasato, "スライド 1" (ATI Stream SDK): No.4 (acceleration and potential;
 *     input is position + mass, output is acceleration + potential) and No.5
 *     (four floats per particle, mass in the fourth slot).
 *   - GPU Gems 3 ch. 31 as retold on the CSDN page "Cuda Nbody笔记" and the
 *     blog.luozichu.ink study page: float4 bodies, r_ij = x_j - x_i, the
 *     float4 acceleration with w = 0.
 * Readings where the pages are damaged or silent: the potential includes the
 * j = i term -m_i/sqrt(eps2) and is negative; eps2 is the softening squared,
 * added to |r|^2 (the lecture's "Soften" constant).
 *
 * Conventions for every call:
 *   - Every pointer is a DEVICE pointer on the current HIP device, owned by the
 *     caller; the library keeps none of them after the call returns.
 *   - Work is enqueued on `stream` (0 = the null stream) and the call returns
 *     without synchronising. The caller keeps buffers alive until the stream has
 *     run the work. Asynchronous faults surface at the caller's next sync.
 *   - All arithmetic is IEEE fp32, round-to-nearest-even, with fused multiply-
 *     add; results are deterministic: the same call on the same device and
 *     inputs gives the same bits.
 *   - Argument checks happen before any HIP call; on failure nothing is
 *     enqueued and nbody_last_error() describes the problem.
 *   - The library owns a cached scratch area per (device, stream) for split-j
 *     partial sums and the accelerations inside nbody_step. Calls that overlap
 *     in time on the SAME stream are ordered by the stream; calls on different
 *     streams use different scratch areas. The area is keyed by the stream
 *     handle: destroy a stream only after its work has finished (or call
 *     nbody_release_workspace) if a new stream may reuse the handle.
 *   - Any host thread may call the library. Calls that use scratch hold a
 *     process-wide lock while they enqueue (not while the GPU runs the work).
 */
#ifndef NBODY_H
#define NBODY_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* One body: (x, y, z, m) for positions, (vx, vy, vz, unused) for velocities,
 * (ax, ay, az, 0) for accelerations. 16 bytes, 16-byte aligned. */
typedef struct nbody_f4 {
    float x, y, z, w;
} nbody_f4;

/* Return codes. */
enum {
    NBODY_OK = 0,
    NBODY_EINVAL = 1, /* bad argument: NULL pointer, N out of range, eps2/dt invalid, overlap */
    NBODY_EALIGN = 2, /* a pointer is not aligned (16 bytes for nbody_f4, 4 for float) */
    NBODY_EHIP = 3,   /* a HIP runtime call or kernel launch failed */
    NBODY_ENOMEM = 4  /* the library could not allocate its scratch area */
};

/* Source-broadcast schemes of the acceleration kernel (nbody_plan.bcast). */
enum {
    NBODY_BCAST_AUTO = 0,
    NBODY_BCAST_LDS = 1,      /* workgroup stages float4 source tiles in LDS; uniform-address LDS reads */
    NBODY_BCAST_SCALAR = 2,   /* each wave reads sources with scalar (uniform) loads into SGPRs */
    NBODY_BCAST_READLANE = 3  /* each lane loads one source; v_readlane broadcasts it to the wave */
};

/* Evaluation modes (nbody_plan.mode). */
enum {
    NBODY_MODE_AUTO = 0,
    NBODY_MODE_TILES = 1, /* one-sided: every target sums over every source (N^2 pair terms) */
    NBODY_MODE_PAIRS = 2, /* pair-symmetric: each unordered pair evaluated once, applied to
                             both bodies (r_ji = -r_ij), over bands of `band` bodies */
    NBODY_MODE_SMALL = 3  /* one-sided, for small N: each 256-thread workgroup owns `tpl`
                             targets and sums over every source; no partial sums, one kernel
                             per evaluation and per Euler step */
};

/* How an evaluation is laid out on the GPU. Zero in a field means "choose
 * automatically". nbody_plan_for() returns the automatic choice.
 *   bcast  - source-broadcast scheme (NBODY_BCAST_*).
 *   tpl    - targets held in registers per lane: 1, 2, 4 or 8.
 *   splits - split-j source chunks S >= 1. With S > 1 each chunk's partial sums
 *            go to scratch and a second kernel adds them in ascending chunk
 *            order (deterministic). S = 1 writes results directly.
 *   chunk  - (output only) sources per chunk; chunks are [s*chunk, min((s+1)*chunk, N)).
 *   wg     - threads per workgroup: 64, 128, 256 or 512 for NBODY_BCAST_LDS (also
 *            the LDS tile, in bodies), 256 for the other schemes.
 *   mode   - NBODY_MODE_*. The fields above describe NBODY_MODE_TILES. With
 *            NBODY_MODE_PAIRS only `band` (256, 512, 1024, 2048 or 4096 bodies),
 *            `tpl` (4 or 8 targets per lane, 4 only with 256-body bands, 8 only
 *            with 4096-body bands), `run` and `passes` may be set (0 =
 *            automatic); the output then has splits = nb = number of bands,
 *            chunk = band, bcast = LDS, wg = 256. Each workgroup evaluates `run`
 *            band pairs that share one band, whose sums it keeps on chip across
 *            them, so a body receives 1 + R + floor(nb / 2) partial sums with
 *            R the number of runs. In one pass the scratch is that
 *            many records of N x 16 bytes (4.50 GB at N = 2^20 with 2048-body
 *            bands and run 32); when that would exceed 1/16 of device memory the
 *            automatic plan evaluates the band pairs in several passes over
 *            band ranges, each pass's sums added into running totals, with
 *            scratch of about (splits / passes + 3) x N x 16 bytes.
 *            With NBODY_MODE_SMALL only `tpl` may be set: targets per workgroup,
 *            4, 8, 16 or 32 (0 = automatic); the output has splits = 1, chunk =
 *            N, bcast = LDS, wg = 256. It needs no scratch for an evaluation and
 *            N x 16 bytes for steps.
 *   band   - see mode.
 *   passes - pair mode: passes over band ranges, 1 .. splits (0 = automatic:
 *            one while the full slot scratch fits, else the fewest that fit).
 *            Results with different pass counts differ in the last bits.
 *   run    - pair mode: band pairs per workgroup, 1 .. 65536 (0 = automatic:
 *            the longest power of two up to 32 that keeps the last workgroups of
 *            the launch short; 32 at N = 2^20). From 16 on, the last `run` band
 *            pairs of each band are split into four shorter runs. Results with
 *            different run lengths differ in the last bits.
 * The plan is a pure function of (N, device compute units and memory), so
 * nbody_accel and nbody_step use the same one for the same N, with or without
 * the potential. */
typedef struct nbody_plan {
    int32_t bcast;
    int32_t tpl;
    int32_t splits;
    int32_t chunk;
    int32_t wg;
    int32_t mode;
    int32_t band;
    int32_t passes;
    int32_t run;
} nbody_plan;

/*
 * nbody_accel - accelerations, and optionally potentials, of all N bodies.
 *   pos_xyzm : N bodies (x, y, z, m), read only.
 *   N        : body count, 0 <= N <= 2^30 (every entry point). N = 0 enqueues nothing.
 *   eps2     : softening squared; a finite float >= 2^-84 (about 5.2e-26), so that
 *              eps2^(-3/2), the 1/r^3 of the self pair, is finite in fp32 (every
 *              entry point takes eps2 under this rule; NBODY_EINVAL otherwise).
 *   acc_out  : N records written as (ax, ay, az, 0). Must not overlap pos_xyzm.
 *   pot_out  : N floats p_i, or NULL to skip the potential. Must not overlap
 *              the other buffers.
 * Returns NBODY_OK or an error code.
 */
int nbody_accel(const nbody_f4 *pos_xyzm, int64_t N, float eps2, nbody_f4 *acc_out,
                float *pot_out, hipStream_t stream);

/*
 * nbody_accel_plan - nbody_accel with an explicit layout (NULL = automatic).
 * Fields left 0 are chosen automatically. Any accepted plan gives results
 * within the same error bound; different plans may differ in the last bits.
 */
int nbody_accel_plan(const nbody_f4 *pos_xyzm, int64_t N, float eps2, nbody_f4 *acc_out,
                     float *pot_out, const nbody_plan *plan, hipStream_t stream);

/*
 * nbody_step - nsteps explicit Euler steps, in place.
 *   pos : N bodies (x, y, z, m); x, y, z are updated, m is never written.
 *   vel : N records (vx, vy, vz, w); vx, vy, vz are updated, w is never written.
 *   dt  : time step, any finite float (0 and negative allowed).
 *   eps2: as for nbody_accel.
 *   nsteps >= 0; 0 enqueues nothing.
 * Each step evaluates a(x^n) with the same plan as nbody_accel(N, no potential),
 * then x += dt v (old v) and v += dt a, both as single fused multiply-adds.
 * pos and vel must not overlap.
 */
int nbody_step(nbody_f4 *pos, nbody_f4 *vel, int64_t N, float dt, float eps2, int64_t nsteps,
               hipStream_t stream);

/*
 * nbody_step_plan - nbody_step with an explicit layout (NULL = automatic), as
 * nbody_accel_plan is to nbody_accel.
 */
int nbody_step_plan(nbody_f4 *pos, nbody_f4 *vel, int64_t N, float dt, float eps2,
                    int64_t nsteps, const nbody_plan *plan, hipStream_t stream);

/*
 * nbody_step_noalloc - nbody_step for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving or simulation loops,
 * harnesses that forbid hipMalloc. Same arguments, plan, kernels and bits as
 * nbody_step, but no hipMalloc, hipFree or allocating library routine is
 * called: the scratch (the second position buffer of small-N steps, the pair
 * or split-j partial sums of larger N) comes from a static 128 MiB array
 * that each GPU holds, inside the library's code object, until the process
 * ends (looked up on a device's first call).
 *   Limit: the step plan's scratch must fit 128 MiB; with the automatic plan
 *   (a function of N) that is N <= 65027: at N = 65536 the pair slots take
 *   129 x N x 16 bytes (NBODY_EINVAL, with the bytes it would need, beyond it).
 *   The array keeps the last call's contents; nothing in it needs to start at
 *   zero (every entry is written before it is read within a step). All calls
 *   on one GPU share it: calls that overlap in time on that GPU (on different
 *   streams or from different host threads) race; calls on one stream are
 *   ordered by the stream.
 */
int nbody_step_noalloc(nbody_f4 *pos, nbody_f4 *vel, int64_t N, float dt, float eps2,
                       int64_t nsteps, hipStream_t stream);

/*
 * nbody_accel_soa - nbody_accel for bodies held as separate arrays (the host
 * layout of the lecture's CPU program): x, y, z, m in; ax, ay, az and, if
 * pot_out is not NULL, the potentials out. All arrays hold N floats (4-byte
 * aligned, device memory); the outputs must not overlap any other array. The
 * library packs the inputs into its own 16-byte records, evaluates them with
 * the automatic plan and unpacks: the results equal nbody_accel's bit for bit
 * (cost: 2 x N x 16 bytes of scratch and ~N x 48 bytes of extra HBM traffic).
 */
int nbody_accel_soa(const float *x, const float *y, const float *z, const float *m, int64_t N,
                    float eps2, float *ax, float *ay, float *az, float *pot_out,
                    hipStream_t stream);

/*
 * nbody_step_soa - nbody_step for separate arrays: x, y, z and vx, vy, vz are
 * updated in place, m is read only; the seven arrays must not overlap. Packing
 * and unpacking happen once per call, not per step; results equal nbody_step's
 * bit for bit.
 */
int nbody_step_soa(float *x, float *y, float *z, const float *m, float *vx, float *vy, float *vz,
                   int64_t N, float dt, float eps2, int64_t nsteps, hipStream_t stream);

/*
 * nbody_accel_shard - one shard of a pair-symmetric evaluation: the unit of work
 * of one GPU when an evaluation is split over nshards GPUs (each holding every
 * position). The sum is the one above (Degawa slide 4, Nakasato No.4), cut
 * into partial sums that are merged afterwards, as the blog.luozichu.ink study
 * page ("GPU Gems 3 · Chapter 31", section 4) splits one body's row over
 * several threads for small N and merges their accelerations.
 *   The N bodies form nb bands of plan.band bodies (the plan is the automatic
 *   NBODY_MODE_PAIRS plan for N when plan is NULL; otherwise plan.mode must be
 *   NBODY_MODE_PAIRS). Shard s of S owns the bands [floor(s nb / S),
 *   floor((s+1) nb / S)) and evaluates their band-pair work items: item (A, d)
 *   covers every pair of a body of band A with a body of band (A + d) mod nb,
 *   d in [0, nb/2], where for even nb the item d = nb/2 exists only for A < nb/2
 *   (so every unordered pair of bodies, self pairs included, lies in exactly
 *   one item, hence in exactly one shard).
 *   partial_out : N records; record i receives this shard's contribution to
 *                 body i: (ax, ay, az, sum m_j / r) over the pairs of its items
 *                 (w = 0 when want_pot is 0), zero-valued terms included.
 *                 Must not overlap pos_xyzm.
 *   shard, nshards : 0 <= shard < nshards <= nb.
 * Scratch: nb x N x 16 bytes (the full slot array of a one-pass evaluation).
 * With nshards = 1 the result, finished by nbody_shard_finish, equals
 * nbody_accel_plan with the same plan in one pass (plan.passes = 1) bit for bit.
 */
int nbody_accel_shard(const nbody_f4 *pos_xyzm, int64_t N, float eps2, int32_t shard,
                      int32_t nshards, int want_pot, const nbody_plan *plan,
                      nbody_f4 *partial_out, hipStream_t stream);

/*
 * nbody_shard_finish - merges the nshards contributions of nbody_accel_shard for
 * the targets [t0, t1) (what a GPU owning those bodies does after the
 * contributions have reached it): partials holds nshards x N records, shard s
 * at partials[s N .. s N + N); they are added in ascending s (compensated).
 *   acc_out : t1 - t0 records (ax, ay, az, 0) of bodies t0 .. t1 - 1.
 *   pot_out : t1 - t0 floats p_i = -sum, or NULL.
 * 0 <= t0 <= t1 <= N; t0 = t1 enqueues nothing. Outputs must not overlap
 * partials or each other.
 */
int nbody_shard_finish(const nbody_f4 *partials, int64_t N, int32_t nshards, int64_t t0,
                       int64_t t1, nbody_f4 *acc_out, float *pot_out, hipStream_t stream);

/*
 * nbody_p2p - the all-pairs sum restricted to cell interaction lists: the near
 * field of a hierarchical method (GPU Gems 3 ch. 31 study page, section 6;
 * Nakasato "スライド 1", No.34), with the lists a tree or grid code provides.
 *   pos_xyzm   : N bodies grouped by cell: cell c owns [cell_start[c], cell_start[c+1]).
 *   cell_start : ncell + 1 device ints, non-decreasing, within [0, N].
 *   list_off, cells : CSR lists, device ints: target cell c interacts with
 *                cells[list_off[c]] .. cells[list_off[c+1] - 1] (list_off has
 *                ncell + 1 non-decreasing entries within [0, nlist]).
 *   acc_out, pot_out : per body inside a cell range, the sums over the bodies of
 *                the listed cells (a cell listing itself includes j = i, whose
 *                term is the softened self term as in nbody_accel); bodies
 *                outside every cell range are not written.
 * List entries outside [0, ncell) add nothing. The index arrays are read on the
 * device, so their contents are not checked on the host; the kernel checks every
 * range and entry before use (an invalid cell range is skipped, an invalid list
 * range is empty), so malformed lists cannot make it read or write out of bounds.
 * Results within the error bound of nbody_accel over the same terms; fixed order.
 */
int nbody_p2p(const nbody_f4 *pos_xyzm, int64_t N, float eps2, const int32_t *cell_start,
              int32_t ncell, const int32_t *list_off, const int32_t *cells, int64_t nlist,
              nbody_f4 *acc_out, float *pot_out, hipStream_t stream);

/*
 * nbody_near_grid - near field on a uniform grid: dims[0] x dims[1] x dims[2]
 * cubic cells of side h from the corner lo (host arrays); body i is in cell
 * clamp(floor((x_d - lo_d) * (1/h)), 0, dims_d - 1) per axis (float arithmetic,
 * bodies outside the box join the boundary cells), and gets the sum over every
 * body in its own and the 26 neighbouring cells (itself included). The library
 * bins the bodies (stable radix sort of the cell indices, so a cell keeps its
 * bodies in their input order), runs a near-field kernel and writes acc_out /
 * pot_out in the caller's body order. The kernel is the automatic choice of
 * nbody_near_grid_kernel.
 * At most 2^28 cells. Scratch: ~N x 41 bytes + 4 bytes per cell, plus N x 224
 * bytes for the pair-symmetric kernel.
 */
int nbody_near_grid(const nbody_f4 *pos_xyzm, int64_t N, float eps2, const float lo[3], float h,
                    const int32_t dims[3], nbody_f4 *acc_out, float *pot_out,
                    hipStream_t stream);

/* Near-field kernels of nbody_near_grid_kernel. */
enum {
    NBODY_NEAR_AUTO = 0,
    NBODY_NEAR_ONE_SIDED = 1, /* every cell sums over its 27-cell neighbourhood (the nbody_p2p
                                 kernel, the neighbourhood as 9 runs of 3 consecutive cells) */
    NBODY_NEAR_PAIRS = 2      /* each unordered pair of neighbouring cells evaluated once by the
                                 cell with the lower linear index and applied to both cells'
                                 bodies (one distance, one rsq per two interactions, as in
                                 NBODY_MODE_PAIRS); a cell's own pairs one-sided; every body's
                                 14 partial sums (its cell's, and one per forward direction of
                                 the cells below it) added in a fixed order */
};

/*
 * nbody_near_grid_kernel - nbody_near_grid with the near-field kernel chosen by
 * `kernel` (NBODY_NEAR_*; AUTO: pairs when the cells hold 96 to 2048 bodies on
 * average, there are at least two cells per compute unit and its N x 224 bytes of
 * scratch fit 1/16 of device memory, else one-sided). Same definition and error bound; results of the two
 * kernels differ in the last bits. NBODY_EINVAL for another value.
 */
int nbody_near_grid_kernel(const nbody_f4 *pos_xyzm, int64_t N, float eps2, const float lo[3],
                           float h, const int32_t dims[3], int32_t kernel, nbody_f4 *acc_out,
                           float *pot_out, hipStream_t stream);

/* What nbody_near_tree built (host struct, filled on success). */
typedef struct nbody_tree_stats {
    int64_t leaves;        /* leaf cells of the octree */
    int64_t list_entries;  /* total length of the leaves' interaction lists */
    int64_t pair_terms;    /* terms summed: sum over leaves A of |A| x sum over listed B of |B| */
} nbody_tree_stats;

/*
 * nbody_near_tree - near field over the leaves of an adaptive octree: the all-pairs
 * sum as the near part of a tree code (GPU Gems 3 ch. 31 study page, section 6;
 * Nakasato "スライド 1", No.31-38, where the tree code keeps the direct sum for
 * nearby bodies). The pages do not fix the tree; this one is, in float32:
 *   root cube: corner lo_d = the smallest coordinate d of any body, side = the
 *     largest extent over the three axes (1 when all bodies coincide);
 *   body i's cell at level 21 per axis: clamp(floor((x_d - lo_d) * (2^21 / side)),
 *     0, 2^21 - 1); its 63-bit Morton key has bit 3b + d equal to bit b of that cell;
 *   node (L, p), L = 0 .. 21: the bodies whose key shifted right by 3 (21 - L) is p;
 *   leaf of a body: the node on its path with the smallest L holding at most
 *     leaf_size bodies (its level-21 node when none does);
 *   body i gets the sum over every body j whose leaf's closed cube meets the closed
 *     cube of i's leaf (a shared face, edge or corner counts; j = i included).
 * The library sorts the bodies by key (stable), finds the leaves and their lists on
 * the GPU, runs the nbody_p2p kernel over them and writes acc_out / pot_out in the
 * caller's body order. leaf_size >= 1; N <= 2^30; positions finite (a non-finite
 * coordinate gives unspecified results for the bodies, never an access out of
 * bounds). stats (host, may be NULL) receives the leaf and list counts.
 * The call waits once on the stream, for the number of leaves (the host sizes the
 * lists' scratch from it: at most 53 list entries per leaf in total), and returns with the
 * rest enqueued; with stats it also waits for the end of the call. More than
 * 2^31 - 1 list entries (possible only with over 40 million leaves) is EINVAL.
 * Scratch: ~N x 100 bytes + ~300 bytes per leaf, plus the lists' first entries kept
 * between the two list passes (up to 3.5 KB per leaf, at most 256 MiB).
 * From the second call with the same N, leaf_size, positions pointer and stream, the
 * build and the list passes are replayed from cached HIP graphs (same results);
 * nbody_release_workspace destroys them.
 */
int nbody_near_tree(const nbody_f4 *pos_xyzm, int64_t N, float eps2, int64_t leaf_size,
                    nbody_f4 *acc_out, float *pot_out, nbody_tree_stats *stats,
                    hipStream_t stream);

/* Conserved-quantity diagnostics of a state (nbody_diagnostics), in fp64. */
typedef struct nbody_diag {
    double kinetic;             /* K = sum m |v|^2 / 2 */
    double potential;           /* W = sum m (p + m / sqrt(eps2)) / 2: the pair energy, each
                                   pair once, the softened self term of p removed */
    double total;               /* K + W */
    double momentum[3];         /* sum m v */
    double angular_momentum[3]; /* sum m (x cross v) */
    double mass;                /* sum m */
    double centre_of_mass[3];   /* sum m x / sum m (0 when the mass is 0) */
} nbody_diag;

/*
 * nbody_diagnostics - K, W, E, momentum, angular momentum, mass and centre of
 * mass of the state (pos, vel), written to *out.
 *   pos, vel : as for nbody_step (read only).
 *   pot      : the N potentials of pos as nbody_accel returns them (self term
 *              included), or NULL to have them evaluated here with the
 *              automatic plan (one more evaluation, into library scratch).
 *   eps2     : the softening squared the potentials belong to.
 *   out      : DEVICE pointer to one nbody_diag (8-byte aligned), written
 *              asynchronously on `stream`; it must not overlap the inputs.
 * The sums run in fp64 in an order fixed by N alone, so repeated calls on the
 * same state give identical bits. Not part of the pages' method: the textbook
 * definitions built on the potential it returns. N = 0 writes zeros.
 */
int nbody_diagnostics(const nbody_f4 *pos, const nbody_f4 *vel, const float *pot, int64_t N,
                      float eps2, nbody_diag *out, hipStream_t stream);

/*
 * nbody_plan_for - the automatic plan for N bodies on the current device
 * (want_pot is accepted for symmetry; the plan does not depend on it). Fills
 * *out. Queries the device's compute-unit count once per device.
 */
int nbody_plan_for(int64_t N, int want_pot, nbody_plan *out);

/*
 * nbody_time_kernel - measurement hook (not part of the pages' method). With
 * start and stop both non-NULL, every later call on the calling host thread
 * records `start` on its stream immediately before its first launch of a
 * pair-term kernel (the kernel that evaluates the interactions: the pair,
 * tile or small-N kernel, or the near-field kernel) and `stop` immediately
 * after that launch, so hipEventElapsedTime(start, stop) is that one kernel's
 * duration on the stream. Further launches of the same call (later passes or
 * steps) are not bracketed. NULL, NULL switches the hook off. The events are
 * created and owned by the caller (on the device the calls run on); the
 * library only records them, so switch the hook off before destroying them
 * (a call that records a destroyed event fails with NBODY_EHIP). The hook is
 * per host thread. NBODY_EINVAL if exactly one of them is NULL.
 */
int nbody_time_kernel(hipEvent_t start, hipEvent_t stop);

/* Message describing the last non-OK return on the calling thread ("" if none). */
const char *nbody_last_error(void);

/* Frees every cached scratch area of the calling process and destroys the cached
 * near-tree graphs (synchronises the devices that own them). Later calls allocate
 * again on demand. */
int nbody_release_workspace(void);

/* Library version string. */
const char *nbody_version(void);

#ifdef __cplusplus
}
#endif

#endif /* NBODY_H */
