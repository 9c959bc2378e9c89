"""GPU parity of the near-field entry points (nbody_p2p, nbody_near_grid) against the oracle's
list and grid definitions, through the C ABI."""

from __future__ import annotations

import numpy as np
import pytest

import workloads
from gpu_util import TOL, assert_accel_parity, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nb():
    import direct_all_pairs_amd

    return direct_all_pairs_amd


def _dev_i32(a):
    import torch

    a = np.ascontiguousarray(a, dtype=np.int32)
    if a.size == 0:
        a = np.zeros(1, np.int32)
    return torch.from_numpy(a).cuda()


def _csr(lists):
    off = np.zeros(len(lists) + 1, np.int32)
    off[1:] = np.cumsum([len(x) for x in lists])
    flat = np.array([c for x in lists for c in x], np.int32)
    return off, flat


def gpu_p2p(nb, pos, eps2, start, off, flat, pot=True, canary=None):
    import torch

    n = pos.shape[0]
    pd = to_dev(pos)
    acc = torch.full((n, 4), np.nan if canary is None else canary, device="cuda")
    p = torch.full((n,), np.nan if canary is None else canary, device="cuda") if pot else None
    nb.nbody_p2p(pd, n, float(eps2), _dev_i32(start), len(start) - 1, _dev_i32(off),
                 _dev_i32(flat), len(flat), acc, p)
    torch.cuda.synchronize()
    return acc.cpu().numpy(), (p.cpu().numpy() if pot else None)


def _cells(n, ncell, seed):
    rng = np.random.default_rng(seed)
    cuts = np.sort(rng.integers(0, n + 1, ncell - 1))
    return np.concatenate([[0], cuts, [n]]).astype(np.int32)


@pytest.mark.parametrize("n,ncell", [(1, 1), (70, 3), (1000, 17), (3001, 40), (3001, 10),
                                     (5000, 4), (3001, 150), (12000, 150), (40000, 200)])
def test_p2p_full_lists_equal_direct_sum(nb, n, ncell):
    """Every cell listing every cell: the near field is the whole direct sum (one wave per
    cell below 64 bodies per cell on average, four-wave workgroups above, up to 22 of them per
    cell at ~1250 bodies; lists of 150 and 200 entries are walked in segments of 64 entries:
    one wave per cell at ~20 bodies, four waves at ~80, four workgroups per cell at ~200)."""
    import oracle

    pos, _ = workloads.random_bodies(n, seed=1000 + n)
    start = _cells(n, ncell, n)
    off, flat = _csr([list(range(ncell))] * ncell)
    acc, pot = gpu_p2p(nb, pos, 1e-4, start, off, flat)
    assert_accel_parity(acc, pot, oracle.accel(pos, np.float32(1e-4)), what=f"p2p full N={n}")


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_p2p_random_lists(nb, seed):
    """Random lists with repeats, empty lists, empty cells, invalid entries and cells of
    more than 64 bodies (several target and source tiles), against the oracle's lists."""
    import oracle

    rng = np.random.default_rng(seed)
    n, ncell = 2500, 23
    pos, _ = workloads.random_bodies(n, seed=2000 + seed)
    start = _cells(n, ncell, 50 + seed)
    lists = []
    for c in range(ncell):
        k = int(rng.integers(0, 9))
        lst = list(rng.integers(0, ncell, k))
        if rng.random() < 0.3:
            lst += [-1, ncell, 10**6]
        if rng.random() < 0.5:
            lst.append(c)
        lists.append(lst)
    lists[3] = []
    off, flat = _csr(lists)
    acc, pot = gpu_p2p(nb, pos, 1e-4, start, off, flat)
    ref = oracle.p2p(pos, 1e-4, start, off, flat)
    assert_accel_parity(acc, pot, ref, what=f"p2p random lists seed={seed}")
    i0, i1 = start[3], start[4]
    assert np.all(acc[i0:i1, :3] == 0) and np.all(pot[i0:i1] == 0)


def test_p2p_bodies_outside_cells_untouched(nb):
    """Cell ranges covering only part of the bodies: the rest keep the canary."""
    import oracle

    n = 600
    pos, _ = workloads.random_bodies(n, seed=77)
    start = np.array([100, 180, 180, 420], np.int32)  # bodies 0..99 and 420..599 in no cell
    off, flat = _csr([[0, 2], [1], [2, 0]])
    acc, pot = gpu_p2p(nb, pos, 1e-4, start, off, flat, canary=7.25)
    assert np.all(acc[:100] == 7.25) and np.all(acc[420:] == 7.25)
    assert np.all(pot[:100] == 7.25) and np.all(pot[420:] == 7.25)
    ref = oracle.p2p(pos, 1e-4, start, off, flat)
    idx = np.arange(100, 420)
    sub = {k: v[idx] for k, v in ref.items()}
    assert_accel_parity(acc, pot, sub, idx=idx, what="p2p partial cover")


def test_p2p_no_potential_same_acceleration(nb):
    pos, _ = workloads.random_bodies(900, seed=78)
    start = _cells(900, 9, 4)
    off, flat = _csr([[c, (c + 1) % 9, (c + 5) % 9] for c in range(9)])
    a1, _ = gpu_p2p(nb, pos, 1e-4, start, off, flat, pot=True)
    a0, _ = gpu_p2p(nb, pos, 1e-4, start, off, flat, pot=False)
    assert np.array_equal(a0, a1)


def gpu_near_grid(nb, pos, eps2, lo, h, dims, pot=True):
    import torch

    n = pos.shape[0]
    pd = to_dev(pos)
    acc = torch.full((n, 4), np.nan, device="cuda")
    p = torch.full((n,), np.nan, device="cuda") if pot else None
    nb.nbody_near_grid(pd, n, float(eps2), lo, h, dims, acc, p)
    torch.cuda.synchronize()
    return acc.cpu().numpy(), (p.cpu().numpy() if pot else None)


@pytest.mark.parametrize("n,dims,h", [(1, (1, 1, 1), 4.0), (500, (2, 2, 2), 1.0),
                                      (3000, (5, 5, 5), 0.4), (20000, (8, 8, 8), 0.25),
                                      (20000, (13, 3, 7), 0.2), (3000, (1, 6, 5), 0.4),
                                      (3000, (7, 1, 1), 0.3), (3000, (2, 9, 1), 0.25),
                                      # 256 cells: one sort pass over all 8 digit bits;
                                      # 64^3 cells: keys of 18 bits, three sort passes
                                      (20000, (16, 16, 1), 0.125),
                                      (200000, (64, 64, 64), 2.0 / 64)])
def test_near_grid_uniform(nb, n, dims, h):
    """Uniform cube [-1, 1]^3 on grids of several shapes (bodies beyond the last cell join
    the boundary cells; one- and two-cell x extents, where a neighbourhood run holds one or
    two cells) against the grid definition."""
    import oracle

    pos, _ = workloads.random_bodies(n, seed=3000 + n)
    lo = (-1.0, -1.0, -1.0)
    acc, pot = gpu_near_grid(nb, pos, 1e-4, lo, h, dims)
    ref = oracle.near_grid(pos, 1e-4, lo, h, dims)
    assert_accel_parity(acc, pot, ref, what=f"near grid N={n} dims={dims}")


def test_near_grid_two_grids_equal_direct_sum(nb):
    """Two cells per axis: every cell neighbours every other, so the near field is the whole
    direct sum."""
    import oracle

    pos, _ = workloads.random_bodies(4000, seed=31)
    acc, pot = gpu_near_grid(nb, pos, 1e-4, (-1.0, -1.0, -1.0), 1.0, (2, 2, 2))
    assert_accel_parity(acc, pot, oracle.accel(pos, np.float32(1e-4)), what="2x2x2 grid")


def test_near_grid_plummer_clamped(nb):
    """A Plummer sphere (dense centre, far outliers) on a box smaller than the system: the
    outliers are clamped into the boundary cells; sampled targets against the definition."""
    import oracle

    w = workloads.make("plummer65536")
    lo, h, dims = (-2.0, -2.0, -2.0), 0.25, (16, 16, 16)
    acc, pot = gpu_near_grid(nb, w.pos, w.eps2, lo, h, dims)
    r = np.linalg.norm(w.pos[:, :3], axis=1)
    idx = np.unique(np.concatenate([np.argsort(r)[:200], np.argsort(r)[-200:],
                                    np.random.default_rng(4).integers(0, w.n, 600)]))
    ref = oracle.near_grid(w.pos, w.eps2, lo, h, dims, targets=idx)
    assert_accel_parity(acc, pot, ref, idx=idx, what="plummer near grid")


def test_near_grid_deterministic_and_order_free(nb):
    """Repeated calls give the same bits; permuting the input bodies permutes the output
    rows only up to rounding order (each cell keeps its bodies in input order)."""
    import oracle

    pos, _ = workloads.random_bodies(5000, seed=41)
    args = ((-1.0, -1.0, -1.0), 0.3, (7, 7, 7))
    a1, p1 = gpu_near_grid(nb, pos, 1e-4, *args)
    a2, p2 = gpu_near_grid(nb, pos, 1e-4, *args)
    assert np.array_equal(a1, a2) and np.array_equal(p1, p2)
    perm = np.random.default_rng(5).permutation(5000)
    a3, p3 = gpu_near_grid(nb, pos[perm], 1e-4, *args)
    ref = oracle.near_grid(pos, 1e-4, *args)
    inv = np.empty_like(perm)
    inv[perm] = np.arange(5000)
    assert_accel_parity(a3[inv], p3[inv], ref, what="permuted input")


def test_near_grid_few_large_cells(nb):
    """64 cells of ~780 bodies: 15 four-wave workgroups per cell, each taking every 15th
    64-target chunk, many source tiles per chunk; sampled targets against the grid
    definition."""
    import oracle

    pos, _ = workloads.random_bodies(50000, seed=51)
    args = ((-1.0, -1.0, -1.0), 0.5, (4, 4, 4))
    acc, pot = gpu_near_grid(nb, pos, 1e-4, *args)
    idx = np.unique(np.random.default_rng(6).integers(0, 50000, 1500))
    ref = oracle.near_grid(pos, 1e-4, *args, targets=idx)
    assert_accel_parity(acc, pot, ref, idx=idx, what="few large cells")


def test_near_grid_huge_cells(nb):
    """Eight cells of ~7500 bodies (2 x 2 x 2: the near field is the whole direct sum): ~118
    64-target chunks per cell over 122 workgroups per cell, so the larger cells' chunks fill
    them all and the others leave some workgroups without a chunk; sampled targets (both ends
    of the body range included) against the direct sum."""
    import oracle

    n = 60000
    pos, _ = workloads.random_bodies(n, seed=61)
    acc, pot = gpu_near_grid(nb, pos, 1e-4, (-1.0, -1.0, -1.0), 1.0, (2, 2, 2))
    rng = np.random.default_rng(8)
    idx = np.unique(np.concatenate([rng.integers(0, n, 800), [0, n - 1]]))
    ref = oracle.accel(pos, np.float32(1e-4), targets=idx)
    assert_accel_parity(acc, pot, ref, idx=idx, what="2x2x2 grid of 7500-body cells")
    assert np.all(np.isfinite(acc)) and np.all(np.isfinite(pot))  # every body written


def test_near_grid_one_cell_workgroup_cap(nb):
    """All 70,000 bodies in one cell (a 1 x 1 x 1 grid: the near field is the direct sum):
    1095 target chunks (1093 of 64 targets, then 32 and 16) over the most workgroups a cell
    gets (1024, below the 1107 its size asks for), so 71 of them take two chunks; sampled
    targets, both ends included, against the direct sum."""
    import oracle

    n = 70000
    pos, _ = workloads.random_bodies(n, seed=71)
    acc, pot = gpu_near_grid(nb, pos, 1e-4, (-1.0, -1.0, -1.0), 2.0, (1, 1, 1))
    rng = np.random.default_rng(9)
    idx = np.unique(np.concatenate([rng.integers(0, n, 600), [0, 63, 64, n - 1]]))
    ref = oracle.accel(pos, np.float32(1e-4), targets=idx)
    assert_accel_parity(acc, pot, ref, idx=idx, what="one cell of 70000 bodies")
    assert np.all(np.isfinite(acc)) and np.all(np.isfinite(pot))  # every body written


def test_near_grid_many_large_cells(nb):
    """N = 2^20 on a 16^3 grid (4096 cells of ~256 bodies: four workgroups of four waves per
    cell, 64-target chunks and a smaller rest, interior cells launched first); sampled targets
    against the grid definition, including cells below and above 256 bodies."""
    import oracle

    w = workloads.make("cube1m")
    args = ((-1.0, -1.0, -1.0), 0.125, (16, 16, 16))
    acc, pot = gpu_near_grid(nb, w.pos, w.eps2, *args)
    idx = np.unique(np.concatenate([np.random.default_rng(7).integers(0, w.n, 1500),
                                    [0, w.n - 1]]))
    ref = oracle.near_grid(w.pos, w.eps2, *args, targets=idx)
    assert_accel_parity(acc, pot, ref, idx=idx, what="16^3 grid, N = 2^20")
    a0, p0 = gpu_near_grid(nb, w.pos, w.eps2, *args, pot=False)
    assert p0 is None and np.array_equal(a0, acc)
