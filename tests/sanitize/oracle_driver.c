/* Driver for the sanitizer test of the oracle (test infrastructure): every
 * function of oracle.c on small inputs, including ragged sizes, target lists,
 * empty and bad CSR lists, grids with clamped cells, shards at band-count
 * edges, and the argument checks. Built with AddressSanitizer and
 * UndefinedBehaviorSanitizer; any finding aborts. Prints the sum of all outputs
 * so nothing is optimised away. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_accel(const double *, int64_t, double, const int64_t *, int64_t, double *, double *,
                 double *, double *);
int oracle_euler(double *, double *, int64_t, double, double, int64_t);
double oracle_energy(const double *, const double *, int64_t, double, double *, double *);
int oracle_diagnostics(const double *, const double *, const double *, int64_t, double, double *);
int oracle_p2p(const double *, int64_t, double, const int32_t *, int32_t, const int32_t *,
               const int32_t *, double *, double *, double *, double *);
int oracle_shard(const double *, int64_t, double, int64_t, int64_t, int64_t, const int64_t *,
                 int64_t, double *, double *, double *, double *);
int oracle_near_grid(const double *, int64_t, double, const double *, double, const int32_t *,
                     const int64_t *, int64_t, double *, double *, double *, double *);

static double frand(uint64_t *s)
{
    *s = *s * 6364136223846793005ULL + 1442695040888963407ULL;
    return (double)(*s >> 11) / 9007199254740992.0 * 2.0 - 1.0;
}

int main(void)
{
    enum { N = 37 };
    double pos[4 * N], vel[4 * N], acc[3 * N], pot[N], ba[N], bp[N], out[13];
    uint64_t seed = 12345;
    for (int i = 0; i < N; ++i) {
        for (int c = 0; c < 3; ++c) {
            pos[4 * i + c] = frand(&seed);
            vel[4 * i + c] = frand(&seed);
        }
        pos[4 * i + 3] = 0.5 + 0.5 * (frand(&seed) + 1.0);
        vel[4 * i + 3] = 0.0;
    }
    double sum = 0.0;
    int bad = 0;
    const int64_t tg[3] = {0, 17, N - 1};
    bad |= oracle_accel(pos, N, 1e-3, NULL, N, acc, pot, ba, bp);
    bad |= oracle_accel(pos, N, 1e-3, tg, 3, acc, pot, ba, bp);
    bad |= oracle_accel(pos, 1, 1e-3, NULL, 1, acc, NULL, NULL, NULL);
    bad |= oracle_accel(pos, N, 1e-3, tg, 0, NULL, NULL, NULL, NULL);
    const int64_t tg_bad[1] = {N};
    if (oracle_accel(pos, N, 1e-3, tg_bad, 1, acc, pot, ba, bp) != -1) bad = 1;
    for (int i = 0; i < 3 * N; ++i) sum += acc[i];
    double p2[4 * N], v2[4 * N];
    for (int i = 0; i < 4 * N; ++i) { p2[i] = pos[i]; v2[i] = vel[i]; }
    bad |= oracle_euler(p2, v2, N, 1e-3, 1e-3, 3);
    if (oracle_euler(p2, v2, -1, 1e-3, 1e-3, 1) != -1) bad = 1;
    double ke = 0.0, pe = 0.0;
    sum += oracle_energy(p2, v2, N, 1e-3, &ke, &pe) + ke + pe;
    bad |= oracle_diagnostics(pos, vel, NULL, N, 1e-3, out);
    bad |= oracle_diagnostics(pos, vel, pot, N, 1e-3, out);
    for (int q = 0; q < 13; ++q) sum += out[q];
    /* CSR lists: 4 cells over the bodies, entries out of range and an empty list */
    const int32_t cs[5] = {0, 9, 9, 30, N};
    const int32_t off[5] = {0, 3, 3, 6, 9};
    const int32_t cells[9] = {0, 2, 3, -1, 1, 4, 3, 3, 0};
    bad |= oracle_p2p(pos, N, 1e-3, cs, 4, off, cells, acc, pot, ba, bp);
    const int32_t cs_bad[5] = {0, 9, 5, 30, N};
    if (oracle_p2p(pos, N, 1e-3, cs_bad, 4, off, cells, acc, pot, ba, bp) != -1) bad = 1;
    for (int i = 0; i < N; ++i) sum += pot[i];
    /* grids: clamped cells, one cell per axis, targets */
    const double lo[3] = {-0.5, -0.5, -0.5};
    const int32_t dims[3] = {3, 2, 1}, dims1[3] = {1, 1, 1};
    bad |= oracle_near_grid(pos, N, 1e-3, lo, 0.4, dims, NULL, N, acc, pot, ba, bp);
    bad |= oracle_near_grid(pos, N, 1e-3, lo, 0.4, dims1, tg, 3, acc, pot, ba, bp);
    for (int i = 0; i < N; ++i) sum += ba[i];
    /* shards: odd and even band counts, one shard per band, bad shard indices */
    for (int64_t band = 1; band <= 8; band += 7) {
        const int64_t nb = (N + band - 1) / band;
        for (int64_t S = 1; S <= nb; S = S * 2 + 1)
            for (int64_t s = 0; s < S; ++s) bad |= oracle_shard(pos, N, 1e-3, band, s, S, NULL, N,
                                                                acc, pot, ba, bp);
    }
    bad |= oracle_shard(pos, N, 1e-3, 4, 2, 7, tg, 3, acc, pot, ba, bp);
    if (oracle_shard(pos, N, 1e-3, 4, 7, 7, NULL, N, acc, pot, ba, bp) != -1) bad = 1;
    if (oracle_shard(pos, N, 1e-3, 8, 0, 6, NULL, N, acc, pot, ba, bp) != -1) bad = 1;
    for (int i = 0; i < N; ++i) sum += pot[i] + bp[i];
    printf("%s sum=%.17g\n", bad ? "FAILED" : "ok", sum);
    return bad ? 1 : 0;
}
