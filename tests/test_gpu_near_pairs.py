"""The pair-symmetric near-grid kernel (GPU): each unordered pair of neighbouring cells is
evaluated once and applied to both cells' bodies. Against the oracle's grid definition (every
target, or sampled at N = 2^20), through the C ABI: grid shapes with one to three cells per axis
(runs of one, two and three cells), cells of every register row count (1 to 8 rows of 64
targets) and above 512 bodies (several i-sets, whose partner sums are added in place), empty
cells, clamped outliers; determinism, independence of the potential, and the one-sided
kernel's results within the bound."""

from __future__ import annotations

import numpy as np
import pytest

import workloads
from gpu_util import assert_accel_parity, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nb():
    import direct_all_pairs_amd

    return direct_all_pairs_amd


def near(nb, pos, eps2, lo, h, dims, kernel, pot=True):
    import torch

    n = pos.shape[0]
    pd = to_dev(pos)
    acc = torch.full((n, 4), np.nan, device="cuda")
    p = torch.full((n,), np.nan, device="cuda") if pot else None
    nb.nbody_near_grid_kernel(pd, n, float(eps2), lo, h, dims, kernel, acc, p)
    torch.cuda.synchronize()
    return acc.cpu().numpy(), (p.cpu().numpy() if pot else None)


GRIDS = [(1, (1, 1, 1), 4.0), (700, (1, 1, 1), 4.0), (500, (2, 2, 2), 1.0),
         (3000, (5, 5, 5), 0.4), (20000, (8, 8, 8), 0.25), (20000, (13, 3, 7), 0.2),
         (3000, (1, 6, 5), 0.4), (3000, (7, 1, 1), 0.3), (3000, (2, 9, 1), 0.25),
         (20000, (16, 16, 1), 0.125), (40000, (3, 3, 3), 0.7), (9000, (2, 3, 2), 1.0)]


@pytest.mark.parametrize("n,dims,h", GRIDS)
def test_pairs_grid_against_definition(nb, n, dims, h):
    """Uniform cube on grids of several shapes: cells of a handful to ~4400 bodies (1 to 8
    register rows, and several 512-body i-sets), every target against the definition."""
    import oracle

    print(f"[near pairs] N={n} dims={dims}", flush=True)
    pos, _ = workloads.random_bodies(n, seed=7000 + n)
    lo = (-1.0, -1.0, -1.0)
    acc, pot = near(nb, pos, 1e-4, lo, h, dims, nb.NEAR_PAIRS)
    assert_accel_parity(acc, pot, oracle.near_grid(pos, 1e-4, lo, h, dims),
                        what=f"pairs near grid N={n} dims={dims}")
    a0, _ = near(nb, pos, 1e-4, lo, h, dims, nb.NEAR_PAIRS, pot=False)
    assert np.array_equal(a0, acc)
    a1, p1 = near(nb, pos, 1e-4, lo, h, dims, nb.NEAR_PAIRS)
    assert np.array_equal(a1, acc) and np.array_equal(p1, pot)


@pytest.mark.parametrize("rows", list(range(1, 10)))
def test_pairs_every_row_count(nb, rows):
    """A 3 x 3 x 3 grid whose cells all hold 64 (rows - 1) + 1 .. 64 rows bodies (the last row
    ragged), so that every cell takes the same register row count, 9 meaning two i-sets."""
    import oracle

    rng = np.random.default_rng(rows)
    cells = []
    for z in range(3):
        for y in range(3):
            for x in range(3):
                m = int(rng.integers(64 * (rows - 1) + 1, 64 * rows + 1))
                p = np.zeros((m, 4), np.float32)
                p[:, 0] = x + rng.uniform(0.01, 0.99, m)
                p[:, 1] = y + rng.uniform(0.01, 0.99, m)
                p[:, 2] = z + rng.uniform(0.01, 0.99, m)
                p[:, 3] = rng.uniform(0.5, 1.5, m) / 1000.0
                cells.append(p)
    pos = np.concatenate(cells)
    pos = pos[rng.permutation(pos.shape[0])]
    print(f"[near pairs] rows={rows} N={pos.shape[0]}", flush=True)
    args = ((0.0, 0.0, 0.0), 1.0, (3, 3, 3))
    acc, pot = near(nb, pos, 1e-3, *args, nb.NEAR_PAIRS)
    assert_accel_parity(acc, pot, oracle.near_grid(pos, np.float32(1e-3), *args),
                        what=f"rows={rows}")


def test_pairs_empty_cells_and_outliers(nb):
    """Bodies in a few separated clusters on a 12^3 grid (most cells empty, so many owners
    own nothing and many partner slots do not exist), plus outliers clamped into the boundary
    cells."""
    import oracle

    rng = np.random.default_rng(3)
    parts = [rng.normal(c, 0.05, size=(600, 3)) for c in ((-0.5, -0.5, -0.5), (0.3, 0.2, -0.1),
                                                            (0.7, -0.6, 0.6))]
    parts.append(rng.uniform(-3.0, 3.0, size=(40, 3)))
    x = np.concatenate(parts)
    pos = np.zeros((x.shape[0], 4), np.float32)
    pos[:, :3] = x
    pos[:, 3] = rng.uniform(0.5, 1.5, x.shape[0]) / x.shape[0]
    args = ((-1.0, -1.0, -1.0), 2.0 / 12, (12, 12, 12))
    print(f"[near pairs] clusters N={pos.shape[0]}", flush=True)
    acc, pot = near(nb, pos, 1e-4, *args, nb.NEAR_PAIRS)
    assert_accel_parity(acc, pot, oracle.near_grid(pos, np.float32(1e-4), *args),
                        what="clusters and outliers")


def test_pairs_and_one_sided_agree_and_auto(nb):
    """N = 2^20 on a 16^3 grid (256 bodies per cell, where the automatic choice is the pair
    kernel): sampled targets against the definition; the automatic call equals the forced pair
    kernel bit for bit; the one-sided kernel agrees within the bound; repeated calls identical."""
    import oracle

    w = workloads.make("cube1m")
    args = ((-1.0, -1.0, -1.0), 0.125, (16, 16, 16))
    print("[near pairs] cube1m 16^3", flush=True)
    a2, p2 = near(nb, w.pos, w.eps2, *args, nb.NEAR_PAIRS)
    a0, p0 = near(nb, w.pos, w.eps2, *args, nb.NEAR_AUTO)
    a1, p1 = near(nb, w.pos, w.eps2, *args, nb.NEAR_ONE_SIDED)
    assert np.array_equal(a0, a2) and np.array_equal(p0, p2)
    idx = np.unique(np.concatenate([np.random.default_rng(17).integers(0, w.n, 1500),
                                    [0, w.n - 1]]))
    ref = oracle.near_grid(w.pos, w.eps2, *args, targets=idx)
    assert_accel_parity(a2, p2, ref, idx=idx, what="pairs 16^3")
    assert_accel_parity(a1, p1, ref, idx=idx, what="one-sided 16^3")
    a3, p3 = near(nb, w.pos, w.eps2, *args, nb.NEAR_PAIRS)
    assert np.array_equal(a3, a2) and np.array_equal(p3, p2)


@pytest.mark.parametrize("bad", ["nan", "inf"])
def test_pairs_non_finite_body(nb, bad):
    """A non-finite coordinate gives unspecified values but a normal call through the pair
    kernel: every row is written (w = 0, no canary left); with a NaN coordinate (binned to the
    grid's low face on its axis) the bodies in the octant away from that corner stay finite; the
    next call on finite bodies is unaffected."""
    import torch

    import oracle

    n = 8000
    pos, _ = workloads.random_bodies(n, seed=19)
    bad_pos = pos.copy()
    bad_pos[5, 0] = np.nan if bad == "nan" else np.inf
    args = ((-1.0, -1.0, -1.0), 0.25, (8, 8, 8))
    print(f"[near pairs] non-finite {bad}", flush=True)
    pd = to_dev(bad_pos)
    acc = torch.full((n, 4), 7.0, device="cuda")
    pot = torch.full((n,), 7.0, device="cuda")
    nb.nbody_near_grid_kernel(pd, n, 1e-4, *args, nb.NEAR_PAIRS, acc, pot)
    torch.cuda.synchronize()
    a, p = acc.cpu().numpy(), pot.cpu().numpy()
    assert np.all(a[:, 3] == 0.0) and not np.any(p == 7.0)
    if bad == "nan":
        far = np.all(bad_pos[:, :3] > 0.0, axis=1)
        assert far.sum() > 500 and np.all(np.isfinite(a[far])) and np.all(np.isfinite(p[far]))
    a2, p2 = near(nb, pos, 1e-4, *args, nb.NEAR_PAIRS)
    assert_accel_parity(a2, p2, oracle.near_grid(pos, np.float32(1e-4), *args),
                        what="pairs after a non-finite call")


def test_pairs_plummer_dense_core(nb):
    """The Plummer sphere of 65,536 bodies on a 16^3 grid of side 0.25 (outliers clamped into
    the boundary cells): the core cells hold thousands of bodies (several 512-body i-sets whose
    forward bodies' sums are added to in place), most outer cells a few; sampled targets in the
    core, the outliers and at random against the grid definition."""
    import oracle

    w = workloads.make("plummer65536")
    args = ((-2.0, -2.0, -2.0), 0.25, (16, 16, 16))
    print("[near pairs] plummer65536 16^3", flush=True)
    acc, pot = near(nb, w.pos, w.eps2, *args, nb.NEAR_PAIRS)
    r = np.linalg.norm(w.pos[:, :3], axis=1)
    idx = np.unique(np.concatenate([np.argsort(r)[:300], np.argsort(r)[-200:],
                                    np.random.default_rng(5).integers(0, w.n, 600)]))
    ref = oracle.near_grid(w.pos, w.eps2, *args, targets=idx)
    assert_accel_parity(acc, pot, ref, idx=idx, what="pairs plummer near grid")
