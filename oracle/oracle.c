/*
 * fp64 CPU oracle for the direct all-pairs softened-gravity method.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or call
 * this code: it is used by tests/, by the smoke check in __graft_entry__.py and
 * by the cpu_baseline leg of bench.py. It shares no source with the HIP
 * library.
 *
 * The method is an exact direct sum (no approximation), so the oracle is that
 * sum written out in double precision, one target at a time, sources in
 * ascending index order, nothing blocked, fused or reordered. OpenMP only
 * splits the independent targets between threads; each target's sum is
 * sequential, so results do not depend on the thread count.
 *
 * What it computes (G = 1):
 *   a_i = sum_j m_j (x_j - x_i) / (|x_j - x_i|^2 + eps2)^(3/2)
 *   p_i = -sum_j m_j / (|x_j - x_i|^2 + eps2)^(1/2)
 * Sources:
 *   - Degawa, "N 体問題" (Nagaoka Univ. of Technology lecture), slide 4 for the
 *     acceleration sum and slide 12 for the softening term that replaces the
 *     j != i test: with it the j = i term has a zero numerator.
 *   - Nakasato, "ATI Stream SDK による天文物理計算の高速化" ("スライド 1"), No.4:
 *     the quantities to compute are the acceleration and the potential.
 *   - GPU Gems 3 ch. 31 study page (blog.luozichu.ink), section 1: r_ij = x_j - x_i.
 * Readings where the pages are damaged or silent:
 *   - the sum runs over ALL j, including j = i, for both a and p (the softened
 *     sum as written; the Stream SDK IL kernel loops over every particle with no
 *     branch). So p_i contains the self term -m_i/sqrt(eps2);
 *   - the sign of p is negative (the minus sign is lost in the slide text);
 *   - eps2 is the softening squared, added to |r|^2.
 *
 * Euler step (Degawa, slides 5-6 and the CPU program's integrate(), slide 15):
 *   x^{n+1} = x^n + dt v^n,   v^{n+1} = v^n + dt a(x^n)
 * position first, using the old velocity; a is computed from x^n.
 *
 * Per-body error scales reported beside the results (parity bounds):
 *   B_i = sum_j m_j |r_ij| / (|r_ij|^2 + eps2)^(3/2),  P_i = sum_j m_j / (|r_ij|^2 + eps2)^(1/2)
 *
 * Parity pins (tests/test_oracle.py): N = 1 and N = 2 closed forms, a regular
 * polygon (ring) closed form, zero force at the centre of symmetric sets,
 * Newton's third law, exact power-of-two scaling, a 50-digit decimal brute
 * force for small N, and the free-particle Euler step. Near fields: lists that
 * cover every cell give the full sum; the grid neighbourhood equals explicit
 * lists; the tree with one leaf is the full sum, on a full octree it is the grid
 * near field of the leaf lattice, and on a two-level tree it equals lists derived
 * by hand. The multi-step energy drift (oracle_energy over a trajectory) has no
 * closed form: parity unpinned.
 *
 * Layouts: pos is n x 4 doubles (x, y, z, m); vel is n x 4 doubles
 * (vx, vy, vz, unused). Return value 0 on success, -1 on bad arguments.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Sums of one target: a (3), -p, B, P. */
typedef struct {
    double ax, ay, az, pp, sa, sp;
} target_sums;

/* Source j acting on target i, added into the target's sums. */
static inline void add_pair(const double *pos, int64_t i, int64_t j, double eps2, target_sums *s)
{
    const double xi = pos[4 * i + 0], yi = pos[4 * i + 1], zi = pos[4 * i + 2];
    const double mj = pos[4 * j + 3];
    const double dx = pos[4 * j + 0] - xi;          /* r_ij = x_j - x_i */
    const double dy = pos[4 * j + 1] - yi;
    const double dz = pos[4 * j + 2] - zi;
    const double r2 = dx * dx + dy * dy + dz * dz;
    const double q = r2 + eps2;                     /* |r|^2 + eps^2 */
    const double q32 = q * sqrt(q);                 /* (|r|^2 + eps^2)^(3/2) */
    s->ax += mj * dx / q32;
    s->ay += mj * dy / q32;
    s->az += mj * dz / q32;
    s->pp -= mj / sqrt(q);
    s->sa += mj * sqrt(r2) / q32;
    s->sp += mj / sqrt(q);
}

/* One target against all n sources, j = 0 .. n-1 in order. */
static void one_target(const double *pos, int64_t n, double eps2, int64_t i,
                       double a[3], double *p, double *ba, double *bp)
{
    target_sums s = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
    for (int64_t j = 0; j < n; ++j) add_pair(pos, i, j, eps2, &s);
    a[0] = s.ax; a[1] = s.ay; a[2] = s.az;
    *p = s.pp; *ba = s.sa; *bp = s.sp;
}

/*
 * Accelerations (and potentials) of the listed targets.
 * targets: indices into [0, n), or NULL for all n bodies (then nt must equal n).
 * acc: nt x 3; pot, bound_a, bound_p: nt each; pot/bound_a/bound_p may be NULL.
 */
int oracle_accel(const double *pos, int64_t n, double eps2,
                 const int64_t *targets, int64_t nt,
                 double *acc, double *pot, double *bound_a, double *bound_p)
{
    if (n < 0 || nt < 0 || (n > 0 && !pos) || (nt > 0 && !acc)) return -1;
    if (!targets && nt != n) return -1;
    if (targets)
        for (int64_t k = 0; k < nt; ++k)
            if (targets[k] < 0 || targets[k] >= n) return -1;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t k = 0; k < nt; ++k) {
        const int64_t i = targets ? targets[k] : k;
        double a[3], p, ba, bp;
        one_target(pos, n, eps2, i, a, &p, &ba, &bp);
        acc[3 * k + 0] = a[0];
        acc[3 * k + 1] = a[1];
        acc[3 * k + 2] = a[2];
        if (pot) pot[k] = p;
        if (bound_a) bound_a[k] = ba;
        if (bound_p) bound_p[k] = bp;
    }
    return 0;
}

/*
 * nsteps explicit Euler steps in fp64, in place on pos and vel.
 * Mass (pos[.][3]) and vel[.][3] are never changed.
 */
int oracle_euler(double *pos, double *vel, int64_t n, double dt, double eps2, int64_t nsteps)
{
    if (n < 0 || nsteps < 0 || (n > 0 && (!pos || !vel))) return -1;
    if (n == 0 || nsteps == 0) return 0;
    double *acc = (double *)malloc((size_t)n * 3 * sizeof(double));
    if (!acc) return -1;
    for (int64_t s = 0; s < nsteps; ++s) {
        oracle_accel(pos, n, eps2, NULL, n, acc, NULL, NULL, NULL);  /* a(x^n) */
        for (int64_t i = 0; i < n; ++i) {
            for (int c = 0; c < 3; ++c) pos[4 * i + c] += dt * vel[4 * i + c];  /* old v */
            for (int c = 0; c < 3; ++c) vel[4 * i + c] += dt * acc[3 * i + c];
        }
    }
    free(acc);
    return 0;
}

/*
 * Total energy of the softened system:
 *   K = sum_i m_i |v_i|^2 / 2
 *   W = -(1/2) sum_i sum_{j != i} m_i m_j / sqrt(|r_ij|^2 + eps2)   (each pair once)
 * Returns K + W; kin and pe receive K and W when non-NULL.
 */
double oracle_energy(const double *pos, const double *vel, int64_t n, double eps2,
                     double *kin, double *pe)
{
    double k = 0.0, w = 0.0;
    double *wi = (double *)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
    if (!wi) return NAN;
    for (int64_t i = 0; i < n; ++i) {
        const double v2 = vel[4 * i] * vel[4 * i] + vel[4 * i + 1] * vel[4 * i + 1] +
                          vel[4 * i + 2] * vel[4 * i + 2];
        k += 0.5 * pos[4 * i + 3] * v2;
    }
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t i = 0; i < n; ++i) {
        double s = 0.0;
        for (int64_t j = 0; j < n; ++j) {
            if (j == i) continue;
            const double dx = pos[4 * j] - pos[4 * i];
            const double dy = pos[4 * j + 1] - pos[4 * i + 1];
            const double dz = pos[4 * j + 2] - pos[4 * i + 2];
            s -= pos[4 * j + 3] / sqrt(dx * dx + dy * dy + dz * dz + eps2);
        }
        wi[i] = 0.5 * pos[4 * i + 3] * s;
    }
    for (int64_t i = 0; i < n; ++i) w += wi[i];  /* fixed order: thread-count independent */
    free(wi);
    if (kin) *kin = k;
    if (pe) *pe = w;
    return k + w;
}

/*
 * Conserved-quantity diagnostics of a state (the pages give the potential,
 * Nakasato "スライド 1" No.4; the sums below are the textbook mechanics built
 * on it and on the velocities of the Euler scheme, Degawa slides 5-6):
 *   out[0]  K = sum_i m_i |v_i|^2 / 2
 *   out[1]  W = (1/2) sum_i m_i (p_i + m_i / sqrt(eps2))  (pair energy; each
 *           pair once, the softened self term of p_i removed)
 *   out[2]  E = K + W
 *   out[3..5]  momentum  P = sum_i m_i v_i
 *   out[6..8]  angular momentum  L = sum_i m_i (x_i x v_i)
 *   out[9]     M = sum_i m_i
 *   out[10..12] centre of mass  sum_i m_i x_i / M  (0 when M = 0)
 * pot: the potentials p_i to use (including the self term, as the method
 * returns them), or NULL to evaluate them here with the sum of oracle_accel.
 * Sums run in index order.
 */
int oracle_diagnostics(const double *pos, const double *vel, const double *pot, int64_t n,
                       double eps2, double *out)
{
    if (!pos || !vel || !out || n < 0 || !(eps2 > 0.0)) return -1;
    double *p = NULL;
    if (!pot) {
        p = (double *)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
        if (!p) return -1;
#pragma omp parallel for schedule(dynamic, 16)
        for (int64_t i = 0; i < n; ++i) {
            double a[3], ba, bp;
            one_target(pos, n, eps2, i, a, &p[i], &ba, &bp);
        }
        pot = p;
    }
    const double inv_eps = 1.0 / sqrt(eps2);
    double k = 0.0, w = 0.0, mom[3] = {0.0, 0.0, 0.0}, ang[3] = {0.0, 0.0, 0.0};
    double m_tot = 0.0, mx[3] = {0.0, 0.0, 0.0};
    for (int64_t i = 0; i < n; ++i) {
        const double m = pos[4 * i + 3];
        const double x = pos[4 * i], y = pos[4 * i + 1], z = pos[4 * i + 2];
        const double vx = vel[4 * i], vy = vel[4 * i + 1], vz = vel[4 * i + 2];
        k += 0.5 * m * (vx * vx + vy * vy + vz * vz);
        w += 0.5 * m * (pot[i] + m * inv_eps);
        mom[0] += m * vx;
        mom[1] += m * vy;
        mom[2] += m * vz;
        ang[0] += m * (y * vz - z * vy);
        ang[1] += m * (z * vx - x * vz);
        ang[2] += m * (x * vy - y * vx);
        m_tot += m;
        mx[0] += m * x;
        mx[1] += m * y;
        mx[2] += m * z;
    }
    free(p);
    out[0] = k;
    out[1] = w;
    out[2] = k + w;
    for (int c = 0; c < 3; ++c) {
        out[3 + c] = mom[c];
        out[6 + c] = ang[c];
        out[10 + c] = m_tot != 0.0 ? mx[c] / m_tot : 0.0;
    }
    out[9] = m_tot;
    return 0;
}

/*
 * Near field over cell interaction lists (the all-pairs kernel as the near
 * part of a hierarchical method: GPU Gems 3 ch. 31 study page, section 6;
 * Nakasato "スライド 1" No.34, neighbour-particle algorithms).
 * Bodies are grouped by cell: cell c owns bodies [cell_start[c], cell_start[c+1]).
 * Target cell c interacts with the cells list[list_off[c]] .. list[list_off[c+1]-1],
 * in list order; every body i of c gets
 *   a_i = sum over listed cells s, over j in s (ascending) of m_j r_ij / (|r_ij|^2 + eps2)^(3/2)
 *   p_i = -sum ... m_j / (|r_ij|^2 + eps2)^(1/2)
 * (j = i included when c lists itself), with the error scales B_i, P_i over the
 * same terms. List entries outside [0, ncell) are skipped. Bodies not in any
 * cell range get zeros. Returns -1 on bad arguments.
 */
int oracle_p2p(const double *pos, int64_t n, double eps2, const int32_t *cell_start,
               int32_t ncell, const int32_t *list_off, const int32_t *list, double *acc,
               double *pot, double *bound_a, double *bound_p)
{
    if (!pos || n < 0 || ncell < 0 || !(eps2 > 0.0) || !cell_start || !list_off) return -1;
    if (cell_start[0] < 0 || cell_start[ncell] > n) return -1;
    for (int32_t c = 0; c < ncell; ++c)
        if (cell_start[c + 1] < cell_start[c] || list_off[c + 1] < list_off[c]) return -1;
    for (int64_t i = 0; i < n; ++i) {
        acc[3 * i] = acc[3 * i + 1] = acc[3 * i + 2] = 0.0;
        pot[i] = bound_a[i] = bound_p[i] = 0.0;
    }
#pragma omp parallel for schedule(dynamic, 1)
    for (int32_t c = 0; c < ncell; ++c) {
        for (int64_t i = cell_start[c]; i < cell_start[c + 1]; ++i) {
            target_sums t = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
            for (int32_t e = list_off[c]; e < list_off[c + 1]; ++e) {
                const int32_t s = list[e];
                if (s < 0 || s >= ncell) continue;
                for (int64_t j = cell_start[s]; j < cell_start[s + 1]; ++j)
                    add_pair(pos, i, j, eps2, &t);
            }
            acc[3 * i] = t.ax;
            acc[3 * i + 1] = t.ay;
            acc[3 * i + 2] = t.az;
            pot[i] = t.pp;
            bound_a[i] = t.sa;
            bound_p[i] = t.sp;
        }
    }
    return 0;
}

/*
 * One shard of a split evaluation, by definition: the bodies form nb =
 * ceil(n / band) bands of `band` consecutive indices; the unordered pair of
 * bands {bi, bj} belongs to band pair_owner(bi, bj) (below), and shard s of S
 * owns the bands [floor(s nb / S), floor((s+1) nb / S)). For every target i
 * (or the listed ones) the sums run over the sources j, ascending, j = i
 * included, whose pair of bands the shard owns. Summed over all S shards this
 * is the whole direct sum, every pair once. Outputs as in oracle_accel.
 * (Splitting a body's sum into parts that are merged afterwards: the
 * blog.luozichu.ink study page of GPU Gems 3 ch. 31, section 4.)
 */
static int64_t pair_owner(int64_t bi, int64_t bj, int64_t nb)
{
    if (bi == bj) return bi;
    const int64_t up = ((bj - bi) % nb + nb) % nb;  /* steps from bi up to bj, mod nb */
    if (2 * up < nb) return bi;                     /* bj lies in bi's upper half-circle */
    if (2 * up > nb) return bj;                     /* bi lies in bj's upper half-circle */
    return bi < bj ? bi : bj;                       /* exactly opposite: the lower band */
}

int oracle_shard(const double *pos, int64_t n, double eps2, int64_t band, int64_t shard,
                 int64_t nshards, const int64_t *targets, int64_t nt, double *acc, double *pot,
                 double *bound_a, double *bound_p)
{
    if (!pos || n < 1 || nt < 0 || !(eps2 > 0.0) || band < 1 || nshards < 1 || shard < 0 ||
        shard >= nshards)
        return -1;
    if (!targets && nt != n) return -1;
    const int64_t nb = (n + band - 1) / band;
    if (nshards > nb) return -1;
    const int64_t b0 = shard * nb / nshards, b1 = (shard + 1) * nb / nshards;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t t = 0; t < nt; ++t) {
        const int64_t i = targets ? targets[t] : t;
        target_sums s = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
        if (i >= 0 && i < n)
            for (int64_t j = 0; j < n; ++j) {
                const int64_t o = pair_owner(i / band, j / band, nb);
                if (o >= b0 && o < b1) add_pair(pos, i, j, eps2, &s);
            }
        acc[3 * t] = s.ax;
        acc[3 * t + 1] = s.ay;
        acc[3 * t + 2] = s.az;
        if (pot) pot[t] = s.pp;
        if (bound_a) bound_a[t] = s.sa;
        if (bound_p) bound_p[t] = s.sp;
    }
    return 0;
}

/*
 * Near field on a uniform grid, by definition and without lists: the grid has
 * dims[0] x dims[1] x dims[2] cubic cells of side h from the corner lo; body i
 * lies in cell k_d = clamp(floor((x_d - lo_d) * inv_h), 0, dims_d - 1) per
 * axis, and a_i, p_i sum over every body j (ascending index, j = i included)
 * whose cell differs from i's by at most one in each axis. Bounds as in
 * oracle_p2p. targets/nt as in oracle_accel.
 * The cell index is an integer decided by floating point, so it is decided in
 * the GPU's precision: x_d - lo_d and the product are float operations with
 * inv_h = float(1 / h), h and lo given as floats.
 */
static int64_t grid_coord(double x, double lo, double h, int32_t dim)
{
    const float inv_h = 1.0f / (float)h;
    const float d = (float)x - (float)lo;
    float f = floorf(d * inv_h);
    if (!(f >= 0.0f)) f = 0.0f;
    if (f > (float)(dim - 1)) f = (float)(dim - 1);
    return (int64_t)f;
}

int oracle_near_grid(const double *pos, int64_t n, double eps2, const double *lo, double h,
                     const int32_t *dims, const int64_t *targets, int64_t nt, double *acc,
                     double *pot, double *bound_a, double *bound_p)
{
    if (!pos || n < 0 || nt < 0 || !(eps2 > 0.0) || !(h > 0.0) || !lo || !dims) return -1;
    if (dims[0] < 1 || dims[1] < 1 || dims[2] < 1) return -1;
    int64_t *cell = (int64_t *)malloc((size_t)(n > 0 ? n : 1) * 3 * sizeof(int64_t));
    if (!cell) return -1;
    for (int64_t j = 0; j < n; ++j)
        for (int d = 0; d < 3; ++d) cell[3 * j + d] = grid_coord(pos[4 * j + d], lo[d], h, dims[d]);
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t t = 0; t < nt; ++t) {
        const int64_t i = targets ? targets[t] : t;
        target_sums s = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
        for (int64_t j = 0; j < n; ++j) {
            int near = 1;
            for (int d = 0; d < 3; ++d) {
                const int64_t dd = cell[3 * j + d] - cell[3 * i + d];
                if (dd < -1 || dd > 1) near = 0;
            }
            if (near) add_pair(pos, i, j, eps2, &s);
        }
        acc[3 * t] = s.ax;
        acc[3 * t + 1] = s.ay;
        acc[3 * t + 2] = s.az;
        pot[t] = s.pp;
        bound_a[t] = s.sa;
        bound_p[t] = s.sp;
    }
    free(cell);
    return 0;
}

/*
 * Near field over the leaves of an octree in Morton order: the all-pairs sum as the
 * near part of a hierarchical method (GPU Gems 3 ch. 31 study page, section 6; the
 * tree codes of Nakasato "スライド 1", No.31-38). The tree itself is not on the
 * pages; it is defined here as follows, with D = TREE_LEVELS = 21 levels below the
 * root (63-bit keys, so that a centrally concentrated system whose outliers set the
 * root cube still splits into small leaves), every decision taken in float32 (an
 * integer decided by floating point is decided in the kernel's precision):
 *   root cube: lo_d = the smallest coordinate d of any body; side = the largest of
 *     (largest coordinate d - lo_d) over d, or 1 when that is not positive;
 *   cell of a body per axis at level D: c_d = floor((x_d - lo_d) * (2^D / side)),
 *     clamped to [0, 2^D - 1] (a NaN goes to 0);
 *   Morton key: bit 3b + d of the key is bit b of c_d (d = 0, 1, 2 for x, y, z);
 *   node (L, p), L = 0 .. D: the bodies whose key shifted right by 3 (D - L) is p;
 *   leaf of a body: the node on its path with the smallest L holding at most
 *     leaf_size bodies, or its level-D node when there is none;
 *   cube of node (L, p): per axis the closed interval [o_d, o_d + 2^(D - L)] in
 *     level-D units, where o_d / 2^(D - L) is made of the bits 3b + d of p;
 *   near field of body i: the sum over every body j whose leaf's cube meets the cube
 *     of i's leaf (touching counts; i's own leaf is included, so j = i is).
 * Sums as oracle_accel, over those j in ascending order, for the listed targets
 * (NULL: all n). leaf_size >= 1. Returns -1 on bad arguments.
 */
#define TREE_LEVELS 21

static int cmp_u64(const void *a, const void *b)
{
    const uint64_t x = *(const uint64_t *)a, y = *(const uint64_t *)b;
    return x < y ? -1 : (x > y ? 1 : 0);
}

/* Number of sorted keys k with a <= k < b (b = 2^63 + ... is allowed: unsigned). */
static int64_t keys_in(const uint64_t *sorted, int64_t n, uint64_t a, uint64_t b)
{
    int64_t l0 = 0, h0 = n, l1 = 0, h1 = n;
    while (l0 < h0) {
        const int64_t m = l0 + (h0 - l0) / 2;
        if (sorted[m] < a) l0 = m + 1; else h0 = m;
    }
    while (l1 < h1) {
        const int64_t m = l1 + (h1 - l1) / 2;
        if (sorted[m] < b) l1 = m + 1; else h1 = m;
    }
    return l1 - l0;
}

int oracle_near_tree(const double *pos, int64_t n, double eps2, int64_t leaf_size,
                     const int64_t *targets, int64_t nt, double *acc, double *pot,
                     double *bound_a, double *bound_p)
{
    if (!pos || n < 0 || nt < 0 || !(eps2 > 0.0) || leaf_size < 1) return -1;
    if (nt > 0 && (!acc || !pot || !bound_a || !bound_p)) return -1;
    const int64_t nn = n > 0 ? n : 1;
    const int D = TREE_LEVELS;
    uint64_t *key = (uint64_t *)malloc((size_t)nn * sizeof(uint64_t));
    uint64_t *sorted = (uint64_t *)malloc((size_t)nn * sizeof(uint64_t));
    int64_t *box = (int64_t *)malloc((size_t)nn * 4 * sizeof(int64_t)); /* o_x, o_y, o_z, size */
    if (!key || !sorted || !box) {
        free(key); free(sorted); free(box);
        return -1;
    }
    float lo[3] = {0.0f, 0.0f, 0.0f}, hi[3] = {0.0f, 0.0f, 0.0f};
    for (int d = 0; d < 3; ++d) {
        for (int64_t j = 0; j < n; ++j) {
            const float x = (float)pos[4 * j + d];
            if (j == 0 || x < lo[d]) lo[d] = x;
            if (j == 0 || x > hi[d]) hi[d] = x;
        }
    }
    float side = 0.0f;
    for (int d = 0; d < 3; ++d) {
        const float ext = hi[d] - lo[d];
        if (ext > side) side = ext;
    }
    if (!(side > 0.0f)) side = 1.0f;
    const float cells = (float)(1 << D);  /* 2^D, exact in float32 */
    const float inv = cells / side;
    for (int64_t j = 0; j < n; ++j) {
        uint64_t k = 0;
        for (int d = 0; d < 3; ++d) {
            float f = floorf(((float)pos[4 * j + d] - lo[d]) * inv);
            if (!(f >= 0.0f)) f = 0.0f;
            if (f > cells - 1.0f) f = cells - 1.0f;
            const uint64_t c = (uint64_t)f;
            for (int b = 0; b < D; ++b) k |= ((c >> b) & 1u) << (3 * b + d);
        }
        key[j] = k;
        sorted[j] = k;
    }
    qsort(sorted, (size_t)n, sizeof(uint64_t), cmp_u64);
    for (int64_t j = 0; j < n; ++j) {
        int level = D;
        for (int L = 0; L <= D; ++L) {
            const int s = 3 * (D - L);
            const uint64_t p = key[j] >> s;
            if (keys_in(sorted, n, p << s, (p + 1) << s) <= leaf_size) {
                level = L;
                break;
            }
        }
        const int s = 3 * (D - level);
        const uint64_t p = key[j] >> s;
        for (int d = 0; d < 3; ++d) {
            int64_t o = 0;
            for (int b = 0; b < level; ++b) o |= (int64_t)((p >> (3 * b + d)) & 1u) << b;
            box[4 * j + d] = o << (D - level);
        }
        box[4 * j + 3] = (int64_t)1 << (D - level);
    }
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 16) reduction(| : bad)
    for (int64_t t = 0; t < nt; ++t) {
        const int64_t i = targets ? targets[t] : t;
        if (i < 0 || i >= n) {
            bad = 1;
            continue;
        }
        target_sums s = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
        const int64_t *bi = box + 4 * i;
        for (int64_t j = 0; j < n; ++j) {
            const int64_t *bj = box + 4 * j;
            int near = 1;
            for (int d = 0; d < 3; ++d)
                if (bj[d] > bi[d] + bi[3] || bi[d] > bj[d] + bj[3]) near = 0;
            if (near) add_pair(pos, i, j, eps2, &s);
        }
        acc[3 * t] = s.ax;
        acc[3 * t + 1] = s.ay;
        acc[3 * t + 2] = s.az;
        pot[t] = s.pp;
        bound_a[t] = s.sa;
        bound_p[t] = s.sp;
    }
    free(key);
    free(sorted);
    free(box);
    return bad ? -1 : 0;
}
