// Internal interface between the C-ABI layer (api.hip) and the gfx950 kernels
// (kernels.hip). Not installed; the public interface is include/nbody.h.
#pragma once

#include <hip/hip_runtime.h>

namespace nbk {

// Threads per workgroup of the acceleration kernels (4 waves of 64).
constexpr int kWG = 256;
// Sources summed into a fresh per-target partial before it is added to the
// running total (two-level accumulation), and the granularity of split-j chunk
// boundaries. LDS tiles hold a multiple of it.
constexpr int kFlush = 256;

struct AccelArgs {
    const float4 *pos;  // N bodies (x, y, z, m)
    int n;              // N
    float eps2;         // softening squared (positive normal float)
    int chunk;          // sources per split-j chunk, a whole number of tiles; chunk s = blockIdx.y
    float4 *acc_out;    // direct mode: (ax, ay, az, 0) per body
    float *pot_out;     // direct mode: p_i per body, or nullptr
    float4 *part;       // split mode (non-null): part[s*N + i] = (ax, ay, az, sum m/r)
};

struct SmallArgs {
    const float4 *pos;  // N bodies (x, y, z, m); the positions a step starts from
    int n;              // N
    float eps2;         // softening squared (positive normal float)
    float4 *acc_out;    // evaluation: (ax, ay, az, 0) per body
    float *pot_out;     // evaluation: p_i per body, or nullptr
    float4 *pos_next;   // step: x + dt v per body (w copied); must not alias pos
    float4 *vel;        // step: v += dt a, in place
    float dt;           // step
};

// Pair-symmetric evaluation over nb = ceil(N / band) bands. The unordered band
// pair {X, X + d mod nb}, d in [1, nb/2], is item (X, d) of its owner band X
// (for even nb the opposite pair d = nb/2 belongs only to the lower X); item
// (X, 0) is band X against itself, one-sided. With D = nb/2 and run length K,
// owner X's items d >= 1 form R runs of consecutive d (run_start below), one
// workgroup each. Sums of a body of band x:
//   own slots     k = 0 (its diagonal item), k = 1 + r (run r of owner x: its
//                 band's sums over the run's items), at own[k * own_stride + i - own0];
//   partner slots the targets' side of item (x - d mod nb, d), d = 1..D, at
//                 partner[p * partner_stride + i] with p = d - 1, or in a pass
//                 over an owner range p = owner - band0.
// The one-pass layout is one array of 1 + R + D slots of N records (own slots
// first, stride N, own0 0), every existing entry written once.
struct PairsArgs {
    const float4 *pos;        // N bodies (x, y, z, m)
    int n;                    // N
    float eps2;               // softening squared (positive normal float)
    int nbands;               // nb
    int band0, band1;         // owner bands evaluated: [band0, band1) (all: 0, nb)
    int run;                  // K >= 1
    int nruns;                // R = pair_runs(nb, K) (0 when nb = 1)
    float4 *own;
    long long own_stride;
    int own0;
    float4 *partner;
    long long partner_stride;
    int partner_by_owner;     // 0: p = d - 1; 1: p = owner - band0
};

// Runs of an owner band's items d = 1 .. D (D = floor(nb / 2)): consecutive d in
// runs of K, except that for K >= kRunSplitMin and D > K the last K values of d
// form kRunSplit runs of K / kRunSplit, so that a launch ends on short
// workgroups. Run r covers d in [1 + run_start(r), run_start(r + 1)].
constexpr int kRunSplitMin = 16;
constexpr int kRunSplit = 4;
__host__ __device__ inline bool run_split(int nb, int run)
{
    return run >= kRunSplitMin && nb / 2 > run;
}
__host__ __device__ inline int pair_runs(int nb, int run)
{
    const int D = nb / 2;
    if (!run_split(nb, run)) return (D + run - 1) / run;
    return (D - run + run - 1) / run + kRunSplit;
}
__host__ __device__ inline int run_start(int r, int nb, int run)
{
    const int D = nb / 2;
    if (!run_split(nb, run)) return r * run < D ? r * run : D;
    const int head = (D - run + run - 1) / run;  // runs of K over d = 1 .. D - K
    if (r <= head) return r * run < D - run ? r * run : D - run;
    if (r >= head + kRunSplit) return D;  // the last run takes any remainder of K / kRunSplit
    return D - run + (r - head) * (run / kRunSplit);
}

// Slots per body of the one-pass layout: 1 + R + floor(nb / 2).
__host__ __device__ inline long long pair_slots(int nb, int run) { return 1 + pair_runs(nb, run) + nb / 2; }

// Pair-symmetric evaluation over bands of `band` bodies (256 to 4096) with tpl
// (4 or 8) targets per lane, grid (band1 - band0, 1 + R). launch_pairs_finish
// finishes a one-pass evaluation; with an owner range narrower than [0, nb)
// only the items of those owners are evaluated, and launch_shard_combine adds
// exactly their slots.
hipError_t launch_pairs(int band, int tpl, bool pot, const PairsArgs &args, hipStream_t stream);

// One-pass finish: every body's own slots (ascending k), then its partner slots
// (ascending d), in compensated sums; then acc_out = (ax, ay, az, 0) and pot_out
// = -sum m/r (if not null), or with pos/vel set one Euler step in place.
struct PairsFinishArgs {
    const float4 *part;       // the one-pass slot array
    int n, band, nbands, run;
    float4 *acc_out;
    float *pot_out;
    float4 *pos, *vel;
    float dt;
};
hipError_t launch_pairs_finish(const PairsFinishArgs &args, hipStream_t stream);

// One shard's contribution to every body from a one-pass slot array written by
// the owners [band0, band1): the slots of their items, in the finish's order
// (compensated), out[i] = (ax, ay, az, sum m/r) partial; N records.
hipError_t launch_shard_combine(const float4 *part, int n, int band, int nbands, int run,
                                int band0, int band1, float4 *out, hipStream_t stream);

// One pass of a multi-pass pair evaluation over owners [band0, band1) (own
// bodies [own0, own0 + own_count) with 1 + R own slots each in `own`, partner
// slots partner[(owner - band0) * N + i]): every body's sums from this pass are
// added, own slots first, then partners by ascending owner, into the
// compensated running totals (tot_s, tot_e) (started fresh when first). On the
// last pass the result goes to acc_out/pot_out, or to acc_out alone as (ax, ay,
// az, sum m/r) records when pot_out is null (the Euler step's input).
struct PassArgs {
    const float4 *own;
    const float4 *partner;
    int n, band, nbands, run, band0, band1, own0, own_count;
    float4 *tot_s, *tot_e;
    int first, last;
    float4 *acc_out;
    float *pot_out;
};
hipError_t launch_pass_combine(const PassArgs &args, hipStream_t stream);

// Targets [t0, t1): the nshards contributions partials[s*N + i] added in
// ascending s (compensated); acc_out[i - t0] = (ax, ay, az, 0) and, if
// pot_out is not null, pot_out[i - t0] = -sum m/r.
hipError_t launch_shard_finish(const float4 *partials, int n, int nshards, int t0, int t1,
                               float4 *acc_out, float *pot_out, hipStream_t stream);

// Launch the acceleration kernel: grid (ceil(N / (wg*tpl)), S), block wg.
// wg is 64, 128, 256 or 512 for the LDS broadcast and 256 for the others.
hipError_t launch_accel(int bcast, int tpl, int wg, bool pot, unsigned grid_x, unsigned splits,
                        const AccelArgs &args, hipStream_t stream);

// Small-N evaluation (step = false: acc_out/pot_out) or Euler step (step =
// true: pos_next/vel) in one kernel without partial sums: tw targets per
// 256-thread workgroup (4, 8, 16 or 32), grid ceil(N / tw).
hipError_t launch_small(int tw, bool pot, bool step, const SmallArgs &args, hipStream_t stream);

// Diagnostics: fp64 sums over the bodies in a fixed order (independent of
// timing). diag_blocks(n) workgroups write kDiagSums partial sums each to
// part; the final kernel adds them and writes the 13 values of nbody_diag.
constexpr int kDiagSums = 12;  // K, W, P (3), L (3), M, M x (3)
int diag_blocks(int n);
hipError_t launch_diagnostics(const float4 *pos, const float4 *vel, const float *pot, int n,
                              double inv_eps, double *part, double *out, hipStream_t stream);

// Near field: target cell c (bodies [cell_start[c], cell_start[c+1])) sums over
// the bodies of the cells in its interaction list. One to 1024 workgroups per
// target cell by the mean cell size, each taking every ny-th target chunk (64
// targets, one per lane, or a smaller rest with source groups); four waves per
// workgroup from 64 bodies per cell on average, sharing a chunk and splitting its
// source tiles.
struct P2PArgs {
    const float4 *pos;      // N bodies grouped by cell
    int n;                  // N
    float eps2;             // softening squared
    const int *cell_start;  // ncell + 1 entries (device)
    int ncell;
    const int *list_off;    // CSR lists: ncell + 1 entries (device); unused on a grid
    const int *list;        // nlist cell indices (device); unused on a grid
    long long nlist;
    float4 *acc_out;        // (ax, ay, az, 0) per body inside a cell range
    float *pot_out;         // p per body, or nullptr
    const int *out_index;   // body i's results go to acc_out/pot_out[out_index[i]]
                            // (nullptr: to index i)
};

// A uniform grid: dims cells per axis, corner lo, cell index per axis
// clamp(floor((x - lo) * inv_h), 0, dims - 1), linear index (z*dy + y)*dx + x.
struct GridSpec {
    float lo[3];
    float inv_h;
    int dims[3];
};

// One to 1024 workgroups per cell (by the mean cell size) taking the cell's target
// chunks in turn (64 targets, one per lane, or a smaller rest with source groups);
// four waves per workgroup from 64 bodies per cell on average, which take the
// chunk's source tiles round-robin.
hipError_t launch_p2p(bool pot, const P2PArgs &args, hipStream_t stream);
// The same kernel with the 27 neighbour cells of the grid as every cell's list.
hipError_t launch_p2p_grid(bool pot, const P2PArgs &args, const GridSpec &g, hipStream_t stream);
// The same near field with each unordered pair of neighbouring cells evaluated
// once, by the cell with the lower linear index, and applied to both cells'
// bodies (a cell's own pairs one-sided): one workgroup per cell holding up to 512
// of its bodies in registers at a time, the 13 forward neighbour cells walked as
// one sequence of 64-body blocks. part holds kSymSlots slots of N records (every
// slot a body has is written once); launch_sym_finish adds them in a fixed order
// and writes row out_index[i] (cell_of[i]: the cell of sorted body i).
constexpr int kSymSlots = 14;
hipError_t launch_p2p_sym(bool pot, const float4 *pos, int n, float eps2, const int *cell_start,
                          const GridSpec &g, float4 *part, hipStream_t stream);
hipError_t launch_sym_finish(const float4 *part, int n, const unsigned *cell_of,
                             const int *cell_start, const GridSpec &g, const int *out_index,
                             float4 *acc_out, float *pot_out, hipStream_t stream);
// keys[i] = linear cell of body i, idx[i] = i.
hipError_t launch_grid_keys(const float4 *pos, int n, const GridSpec &g, unsigned *keys, int *idx,
                            hipStream_t stream);
// out[k] = pos[perm[k]].
hipError_t launch_gather(const float4 *pos, const int *perm, int n, float4 *out,
                         hipStream_t stream);
// cell_start[c] = first k with sorted_keys[k] >= c, for c = 0 .. ncell.
hipError_t launch_cell_starts(const unsigned *sorted_keys, int n, int ncell, int *cell_start,
                              hipStream_t stream);
// Stable sort of (key, value) pairs on bits [0, end_bit) of the keys (keys below
// 2^end_bit): LSD radix sort, 8 bits per pass, 32- or 64-bit keys. temp holds
// sort_temp_bytes(n, key bytes) bytes; the inputs are read only.
size_t sort_temp_bytes(int n, int key_bytes = 4);
hipError_t sort_pairs(void *temp, const unsigned *keys_in, unsigned *keys_out, const int *vals_in,
                      int *vals_out, int n, int end_bit, hipStream_t stream);
hipError_t sort_pairs64(void *temp, const unsigned long long *keys_in,
                        unsigned long long *keys_out, const int *vals_in, int *vals_out, int n,
                        int end_bit, hipStream_t stream);

// Exclusive prefix sum of data[0 .. total) in place (int32, exact), in tiles of
// 4096 entries; *total_out (device, may be null) receives the sum of all entries.
// temp holds scan_temp_bytes(total) bytes.
size_t scan_temp_bytes(long long total);
hipError_t scan_exclusive(int *data, long long total, int *total_out, void *temp,
                          hipStream_t stream);

// ---- Near field over the leaves of an octree in Morton order (nbody_near_tree).
// Every decision is taken in float32 / integer arithmetic on the device:
//   root cube: lo_d = smallest coordinate d, side = largest extent (1 if not
//     positive); frame = (lo_x, lo_y, lo_z, 2^21 / side);
//   level-21 cell per axis: clamp(floor((x_d - lo_d) * (2^21 / side)), 0, 2^21 - 1);
//   63-bit key: bit 3b + d is bit b of the cell coordinate d;
//   node (L, p): the bodies whose key >> 3 (21 - L) is p; a body's leaf is the node
//     on its path with the smallest L holding at most leaf_size bodies (else L = 21);
//   leaves A and B are near when their closed cubes meet.
// Counters written by the build: [0] leaves, [1] list entries (the total of the
// lists when below 2^31), [2..3] the list total as 64 bits, [4..5] pair terms: sum
// over leaves of |A| x sum over listed B of |B| (64 bits).
constexpr int kTreeCounters = 6;
constexpr int kTreeTableMaxLevel = 7;                 // coarse table: at most 8^7 + 1 ints
constexpr int kTreeMaxLeaves = (0x7fffffff - 1) / 27;  // 27 list parts per leaf, int offsets
size_t tree_frame_temp_bytes(int n);
// frame[0] = (lo_x, lo_y, lo_z, 2^21 / side); zeroes counters[0 .. kTreeCounters).
hipError_t launch_tree_frame(const float4 *pos, int n, float *temp, float4 *frame,
                             int *counters, hipStream_t stream);
// keys[i] = 63-bit key of body i, idx[i] = i.
hipError_t launch_tree_keys(const float4 *pos, int n, const float4 *frame,
                            unsigned long long *keys, int *idx, hipStream_t stream);
// From the sorted keys: level[k] = level of the leaf of sorted body k; start[k] = 1
// if k begins its leaf (else 0).
hipError_t launch_tree_levels(const unsigned long long *skeys, int n, int leaf_size, int *level,
                              int *start, hipStream_t stream);
// After start has been scanned into leaf numbers (ids, total in counters[0]): for
// each leaf A, cell_start[A] = its first sorted body, leaf_key[A] = its first key
// cleared below its level, leaf_box[A] = (corner x, y, z in level-21 units, level);
// cell_start[nleaf] = n.
hipError_t launch_tree_leaves(const unsigned long long *skeys, const int *level, const int *ids,
                              int n, int *cell_start, unsigned long long *leaf_key, int4 *leaf_box,
                              hipStream_t stream);
// Coarse table level for nleaf leaves (8^lt cells, at least nleaf, at most 8^7), and
// the table: table[c] = first leaf whose key is at least the start of cell c of level
// lt, c = 0 .. 8^lt (8^lt + 1 ints; nleaf read from counters[0]).
int tree_table_level(int nleaf);
hipError_t launch_tree_table(const unsigned long long *leaf_key, const int *counters, int lt,
                             int *table, hipStream_t stream);
struct TreeLeaves {
    const unsigned long long *leaf_key;
    const int4 *leaf_box;
    const int *table;
    const int *cell_start;
    int nleaf, lt;
};
// Count pass (list == nullptr): cnt[27 A + q] = the length of part q of leaf A's list
// (27 nleaf + 1 entries, the last 0); the list total and the pair terms go to
// counters[2..5] through per-workgroup records in parts (tree_parts_bytes). Fill pass
// (off = the exclusive sums of cnt): part q of leaf A's list written at
// list[off[27 A + q] ..] (never at or past list_cap), list_off[A] = off[27 A],
// list_off[nleaf] = the total. All lists together hold at most kTreeListsPerLeaf entries
// per leaf (one leaf's list may hold more). keep (27 nleaf x keep_cap ints, keep_cap >= 0,
// the same for both passes): the count pass stores each part's first keep_cap entries
// there, and the fill pass copies a part of at most keep_cap entries instead of walking
// its cell again.
constexpr int kTreeListsPerLeaf = 53;
constexpr int kTreeKeepMax = 32;                        // most entries kept per part
constexpr size_t kTreeKeepBytes = (size_t)256 << 20;    // most bytes the kept entries take
size_t tree_parts_bytes(int nleaf);
hipError_t launch_tree_lists(const TreeLeaves &leaves, int *counters, void *parts, int *cnt,
                             const int *off, int *list, int list_cap, int *list_off, int *keep,
                             int keep_cap, hipStream_t stream);

// Layout conversion for the SoA entry points: out[i] = (a[i], b[i], c[i], d ? d[i] : 0),
// and back: a[i], b[i], c[i] = in[i].x, .y, .z.
hipError_t launch_pack(const float *a, const float *b, const float *c, const float *d, int n,
                       float4 *out, hipStream_t stream);
hipError_t launch_unpack(const float4 *in, int n, float *a, float *b, float *c, hipStream_t stream);

// acc_out[i] = (sum_s part[s][i].xyz, 0); pot_out[i] = -sum_s part[s][i].w (if non-null).
hipError_t launch_combine(const float4 *part, int n, int splits, float4 *acc_out, float *pot_out,
                          hipStream_t stream);

// a = sum_s part[s][i].xyz, then pos.xyz += dt * vel.xyz; vel.xyz += dt * a.
hipError_t launch_euler(const float4 *part, int n, int splits, float4 *pos, float4 *vel, float dt,
                        hipStream_t stream);

}  // namespace nbk
