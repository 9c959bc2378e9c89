"""GPU parity of nbody_near_tree (near field over the leaves of the Morton-order octree)
against the oracle's definition of the same tree, through the C ABI."""

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


def gpu_near_tree(nb, pos, eps2, leaf_size, pot=True):
    import torch

    n = pos.shape[0]
    print(f"[tree] N={n} leaf_size={leaf_size} pot={pot}", flush=True)
    pd = to_dev(pos)
    acc = torch.full((n, 4), np.nan, device="cuda")
    p = torch.full((n,), np.nan, device="cuda") if pot else None
    st = nb.nbody_tree_stats()
    nb.nbody_near_tree(pd, n, float(eps2), int(leaf_size), acc, p, st)
    torch.cuda.synchronize()
    return acc.cpu().numpy(), (p.cpu().numpy() if pot else None), st.as_dict()


@pytest.mark.parametrize("n,leaf", [(1, 1), (2, 1), (100, 1), (100, 8), (3001, 16), (3001, 64),
                                    (3001, 300), (5000, 2)])
def test_near_tree_uniform(nb, n, leaf):
    """Uniform cube, every target against the tree definition (leaf sizes from one body,
    where every body is a leaf, to a tenth of the bodies)."""
    import oracle

    pos, _ = workloads.random_bodies(n, seed=4000 + n + leaf)
    acc, pot, st = gpu_near_tree(nb, pos, 1e-4, leaf)
    assert_accel_parity(acc, pot, oracle.near_tree(pos, 1e-4, leaf),
                        what=f"near tree N={n} leaf_size={leaf}")
    assert 1 <= st["leaves"] <= n and st["list_entries"] >= st["leaves"]
    assert n <= st["pair_terms"] <= n * n


@pytest.mark.parametrize("n,leaf", [(1, 1), (700, 700), (3000, 5000)])
def test_near_tree_one_leaf_is_the_direct_sum(nb, n, leaf):
    """leaf_size >= N: the root is the only leaf and the near field is the whole sum."""
    import oracle

    pos, _ = workloads.random_bodies(n, seed=4100 + n)
    acc, pot, st = gpu_near_tree(nb, pos, 1e-4, leaf)
    assert_accel_parity(acc, pot, oracle.accel(pos, np.float32(1e-4)), what=f"one leaf N={n}")
    assert st == {"leaves": 1, "list_entries": 1, "pair_terms": n * n}


def _lattice(cells, k, seed):
    """k bodies inside each cell of a cells^3 lattice on [0, 1]^3 plus bodies at the two
    corners, so that the root cube is [0, 1]^3."""
    rng = np.random.default_rng(seed)
    c = np.stack(np.meshgrid(*[np.arange(cells)] * 3, indexing="ij"), -1).reshape(-1, 3)
    c = np.repeat(c, k, axis=0)
    x = (c + rng.uniform(0.15, 0.85, size=c.shape)) / cells
    x = np.concatenate([x, [[0.0, 0.0, 0.0], [1.0, 1.0, 1.0]]])
    pos = np.zeros((x.shape[0], 4), np.float32)
    pos[:, :3] = x
    pos[:, 3] = rng.uniform(0.5, 1.5, size=x.shape[0]) / x.shape[0]
    return pos


def test_near_tree_full_octree_counts(nb):
    """Two bodies in every cell of a 16^3 lattice (three in the corner cells) with
    leaf_size = 3: the leaves are the lattice cells, each listing its 27-cell neighbourhood
    (clipped at the faces), so the counts have closed forms; results against the oracle."""
    import oracle

    cells = 16
    pos = _lattice(cells, 2, 5)
    acc, pot, st = gpu_near_tree(nb, pos, 1e-4, 3)
    per_axis = 2 * 2 + (cells - 2) * 3  # neighbours per axis: 2 at the faces, 3 inside
    assert st["leaves"] == cells ** 3
    assert st["list_entries"] == per_axis ** 3
    # pair terms: sum over cells A of |A| x bodies in A's neighbourhood
    cnt = np.full((cells,) * 3, 2, np.int64)
    cnt[0, 0, 0] += 1
    cnt[-1, -1, -1] += 1
    pad = np.pad(cnt, 1)
    hood = sum(pad[1 + dx:1 + dx + cells, 1 + dy:1 + dy + cells, 1 + dz:1 + dz + cells]
               for dx in (-1, 0, 1) for dy in (-1, 0, 1) for dz in (-1, 0, 1))
    assert st["pair_terms"] == int(np.sum(cnt * hood))
    assert_accel_parity(acc, pot, oracle.near_tree(pos, 1e-4, 3), what="16^3 lattice tree")


def test_near_tree_clustered_and_duplicates(nb):
    """A dense core inside a sparse halo (leaves at many levels, big leaves beside deep
    ones), 40 bodies at one point (a level-21 node holding more than leaf_size) and a plane
    of bodies (a flat root cube extent), against the definition."""
    import oracle

    rng = np.random.default_rng(11)
    core = rng.normal(0.0, 0.01, size=(3000, 3))
    halo = rng.uniform(-1.0, 1.0, size=(1500, 3))
    same = np.full((40, 3), 0.3)
    plane = np.column_stack([rng.uniform(-1, 1, 500), rng.uniform(-1, 1, 500), np.full(500, -0.5)])
    x = np.concatenate([core, halo, same, plane])
    pos = np.zeros((x.shape[0], 4), np.float32)
    pos[:, :3] = x
    pos[:, 3] = rng.uniform(0.5, 1.5, size=x.shape[0]) / x.shape[0]
    for leaf in (1, 8, 33):
        acc, pot, st = gpu_near_tree(nb, pos, 1e-5, leaf)
        assert_accel_parity(acc, pot, oracle.near_tree(pos, 1e-5, leaf),
                            what=f"clustered tree leaf_size={leaf}")


def test_near_tree_deep_leaves(nb):
    """Leaves 13 levels down: a 4^3 lattice of cells of side 2^-13 at the origin, two bodies
    per cell, and a body at (1, 1, 1) that sets the root cube; with leaf_size 3 the lattice
    cells are the leaves, so the lattice bodies get the grid near field of the lattice and
    the lone body only its self term."""
    import oracle

    rng = np.random.default_rng(14)
    h = 2.0 ** -13
    c = np.repeat(np.stack(np.meshgrid(*[np.arange(4)] * 3, indexing="ij"), -1).reshape(-1, 3),
                  2, axis=0)
    x = np.concatenate([(c + rng.uniform(0.15, 0.85, size=c.shape)) * h,
                        [[0.0, 0.0, 0.0], [1.0, 1.0, 1.0]]])
    pos = np.zeros((x.shape[0], 4), np.float32)
    pos[:, :3] = x
    pos[:, 3] = rng.uniform(0.5, 1.5, size=x.shape[0])
    acc, pot, st = gpu_near_tree(nb, pos, 1e-9, 3)
    assert st["leaves"] == 64 + 1 and st["list_entries"] == 10 ** 3 + 1  # 2 + 3 + 3 + 2 per axis
    assert_accel_parity(acc, pot, oracle.near_tree(pos, 1e-9, 3), what="deep leaves")
    g = oracle.near_grid(pos[:-1], 1e-9, (0.0, 0.0, 0.0), h, (4, 4, 4))
    assert_accel_parity(acc[:-1], pot[:-1], g, what="deep leaves vs lattice grid")


def test_near_tree_big_leaf_beside_fine_leaves(nb):
    """One leaf may list many smaller ones; only the total is bounded (53 per leaf). The octant
    [0, 1/2]^3 holds two bodies (one leaf at level 1); the octant beside it along x holds two
    bodies in each of its 8^3 cells of side 1/16 (512 leaves at level 4), and a body at (1, 1, 1)
    sets the root cube [0, 1]^3 (one more leaf). The big leaf's closed cube meets the 64 fine
    leaves on the shared face and the corner leaf: 66 entries with itself. Leaf, list-entry and
    pair-term counts against a brute-force count over the known leaf cubes; results against the
    oracle."""
    import oracle

    rng = np.random.default_rng(21)
    fine = np.stack(np.meshgrid(*[np.arange(8)] * 3, indexing="ij"), -1).reshape(-1, 3)
    fine = np.repeat(fine, 2, axis=0)
    xf = (fine + rng.uniform(0.15, 0.85, size=fine.shape)) / 16.0
    xf[:, 0] += 0.5
    x = np.concatenate([[[0.0, 0.0, 0.0], [0.25, 0.25, 0.25]], xf, [[1.0, 1.0, 1.0]]])
    pos = np.zeros((x.shape[0], 4), np.float32)
    pos[:, :3] = x
    pos[:, 3] = rng.uniform(0.5, 1.5, size=x.shape[0]) / x.shape[0]
    # leaves as (lo corner, side, bodies)
    leaves = [((0.0, 0.0, 0.0), 0.5, 2), ((0.5, 0.5, 0.5), 0.5, 1)]
    leaves += [((0.5 + i / 16, j / 16, k / 16), 1 / 16, 2)
               for i in range(8) for j in range(8) for k in range(8)]
    lo = np.array([l[0] for l in leaves])
    side = np.array([l[1] for l in leaves])
    cnt = np.array([l[2] for l in leaves], np.int64)
    hi = lo + side[:, None]
    meet = np.all((np.maximum(lo[:, None, :], lo[None, :, :])
                   <= np.minimum(hi[:, None, :], hi[None, :, :])), axis=2)
    assert meet[0].sum() == 66  # the big leaf's list
    acc, pot, st = gpu_near_tree(nb, pos, 1e-6, 2)
    assert st["leaves"] == len(leaves)
    assert st["list_entries"] == int(meet.sum()) <= 53 * len(leaves)
    assert st["pair_terms"] == int((meet * np.outer(cnt, cnt)).sum())
    assert_accel_parity(acc, pot, oracle.near_tree(pos, 1e-6, 2), what="big leaf beside fine leaves")


@pytest.mark.parametrize("bad", ["nan", "inf"])
def test_near_tree_non_finite_body(nb, bad):
    """A non-finite coordinate gives unspecified values but a normal call: a NaN coordinate is
    left out of the bounding cube and binned to the cube's low face on its axis; an infinite
    one makes the cube infinite, so every body lands in one cell. The call succeeds and
    writes every row (w = 0); with a NaN body the rows of bodies far from that face stay
    finite; the next call on finite bodies is unaffected. The same for the grid near field."""
    import oracle

    pos, _ = workloads.random_bodies(3000, seed=17)
    bad_pos = pos.copy()
    bad_pos[5, 0] = np.nan if bad == "nan" else np.inf
    acc, pot, st = gpu_near_tree(nb, bad_pos, 1e-4, 16)
    assert st["leaves"] >= 1 and np.all(acc[:, 3] == 0.0)
    if bad == "nan":
        far = np.all(bad_pos[:, :3] > 0.0, axis=1)  # the octant away from the corner cell
        assert far.sum() > 100 and np.all(np.isfinite(acc[far])) and np.all(np.isfinite(pot[far]))
    acc2, pot2, _ = gpu_near_tree(nb, pos, 1e-4, 16)
    assert_accel_parity(acc2, pot2, oracle.near_tree(pos, 1e-4, 16), what="after a non-finite call")
    import torch

    pd = to_dev(bad_pos)
    acc_g = torch.full((3000, 4), 7.0, device="cuda")
    pot_g = torch.full((3000,), 7.0, device="cuda")
    nb.nbody_near_grid(pd, 3000, 1e-4, (-1.0, -1.0, -1.0), 0.25, (8, 8, 8), acc_g, pot_g)
    torch.cuda.synchronize()
    ag = acc_g.cpu().numpy()
    assert np.all(ag[:, 3] == 0.0)
    if bad == "nan":
        assert np.all(np.isfinite(ag[far]))


def test_near_tree_coincident_bodies(nb):
    """All bodies at one point: one leaf (root cube side 1), the whole direct sum."""
    import oracle

    pos = np.zeros((37, 4), np.float32)
    pos[:, :3] = 2.5
    pos[:, 3] = np.linspace(0.5, 1.5, 37) / 37
    acc, pot, st = gpu_near_tree(nb, pos, 1e-3, 1)
    assert st["leaves"] == 1
    assert_accel_parity(acc, pot, oracle.accel(pos, np.float32(1e-3)), what="coincident")


def test_near_tree_plummer_sampled(nb):
    """Plummer sphere, N = 65536, leaf_size 64: sampled targets (centre, outliers, random)
    against the definition; repeated calls give the same bits; no potential, same
    accelerations."""
    import oracle

    w = workloads.make("plummer65536")
    acc, pot, st = gpu_near_tree(nb, w.pos, w.eps2, 64)
    r = np.linalg.norm(w.pos[:, :3], axis=1)
    idx = np.unique(np.concatenate([np.argsort(r)[:300], np.argsort(r)[-300:],
                                    np.random.default_rng(9).integers(0, w.n, 1000)]))
    ref = oracle.near_tree(w.pos, w.eps2, 64, targets=idx)
    assert_accel_parity(acc, pot, ref, idx=idx, what="plummer tree")
    # the core splits into leaves of at most 64 bodies despite outliers at r ~ 500
    assert st["pair_terms"] < 64 * 27 * w.n
    a2, p2, st2 = gpu_near_tree(nb, w.pos, w.eps2, 64)
    assert np.array_equal(acc, a2) and np.array_equal(pot, p2) and st == st2
    a0, p0, _ = gpu_near_tree(nb, w.pos, w.eps2, 64, pot=False)
    assert p0 is None and np.array_equal(a0, acc)


def test_near_tree_cube1m_sampled(nb):
    """N = 2^20 uniform cube, leaf_size 64 (the benchmarked configuration): sampled targets,
    both ends included, against the definition; every body written."""
    import oracle

    w = workloads.make("cube1m")
    acc, pot, st = gpu_near_tree(nb, w.pos, w.eps2, 64)
    idx = np.unique(np.concatenate([np.random.default_rng(10).integers(0, w.n, 1500),
                                    [0, w.n - 1]]))
    ref = oracle.near_tree(w.pos, w.eps2, 64, targets=idx)
    assert_accel_parity(acc, pot, ref, idx=idx, what="cube1m tree")
    assert np.all(np.isfinite(acc)) and np.all(np.isfinite(pot))
    print(f"[tree] cube1m stats {st}", flush=True)


@pytest.mark.parametrize("n,leaf", [(60000, 200), (60000, 1000), (1 << 20, 1024)])
def test_near_tree_large_leaves(nb, n, leaf):
    """Large leaves, uniform cubes: 512 leaves of ~117 bodies (two four-wave workgroups per
    leaf), 64 of ~940 (16 per leaf) and 4096 of ~256 at N = 2^20 (four per leaf) over the
    packed leaf lists; sampled targets, both ends included, against the definition."""
    import oracle

    pos, _ = workloads.random_bodies(n, seed=15 + leaf)
    acc, pot, st = gpu_near_tree(nb, pos, 1e-4, leaf)
    idx = np.unique(np.concatenate([np.random.default_rng(leaf).integers(0, n, 1500),
                                    [0, n - 1]]))
    assert_accel_parity(acc, pot, oracle.near_tree(pos, 1e-4, leaf, targets=idx), idx=idx,
                        what=f"large leaves leaf_size={leaf}")
    assert np.all(np.isfinite(acc)) and np.all(np.isfinite(pot))
    print(f"[tree] leaf_size={leaf}: {st}, {n / st['leaves']:.1f} bodies per leaf", flush=True)


def test_near_tree_permuted_input(nb):
    """Permuting the input bodies permutes the rows (up to rounding order)."""
    import oracle

    pos, _ = workloads.random_bodies(4000, seed=12)
    perm = np.random.default_rng(13).permutation(4000)
    acc, pot, _ = gpu_near_tree(nb, pos[perm], 1e-4, 16)
    inv = np.empty_like(perm)
    inv[perm] = np.arange(4000)
    assert_accel_parity(acc[inv], pot[inv], oracle.near_tree(pos, 1e-4, 16), what="permuted")


@pytest.mark.parametrize("with_stats", [False, True])
def test_near_tree_graph_replays_equal_the_first_call(nb, with_stats):
    """Repeated calls with the same buffers: the first launches the build and list passes
    directly, the second captures them into graphs, later ones replay them. Five calls, with
    other library work (a grid near field, an all-pairs evaluation) and a synchronization
    between them, all equal the first bit for bit, and it agrees with the oracle; new positions
    written into the same buffer replay to the same bits as a first call on another buffer
    (the graphs read the buffers' current contents)."""
    import torch

    import oracle

    n, leaf, eps2 = 20000, 32, np.float32(1e-4)
    pos, _ = workloads.random_bodies(n, seed=77)
    other, _ = workloads.random_bodies(4000, seed=78)
    pd, od = to_dev(pos), to_dev(other)
    acc = torch.empty((n, 4), device="cuda")
    pot = torch.empty((n,), device="cuda")
    oa = torch.empty((4000, 4), device="cuda")
    op = torch.empty((4000,), device="cuda")
    nb.nbody_release_workspace()
    print(f"[tree] graph replays, stats={with_stats}", flush=True)
    runs = []
    for k in range(5):
        acc.fill_(np.nan)
        pot.fill_(np.nan)
        st = nb.nbody_tree_stats() if with_stats else None
        nb.nbody_near_tree(pd, n, float(eps2), leaf, acc, pot, st)
        torch.cuda.synchronize()
        runs.append((acc.cpu().numpy().copy(), pot.cpu().numpy().copy(),
                     st.as_dict() if st is not None else None))
        nb.nbody_near_grid(od, 4000, float(eps2), (-1.0, -1.0, -1.0), 0.5, (4, 4, 4), oa, op)
        nb.nbody_accel(od, 4000, float(eps2), oa, op)
        torch.cuda.synchronize()
    for a, p, st in runs[1:]:
        assert np.array_equal(a, runs[0][0]) and np.array_equal(p, runs[0][1])
        assert st == runs[0][2]
    idx = np.unique(np.random.default_rng(9).integers(0, n, 500))
    assert_accel_parity(runs[0][0], runs[0][1], oracle.near_tree(pos, eps2, leaf, targets=idx),
                        idx=idx, what="tree, first call")
    # new contents, same buffer (a replay) against a first call on a fresh buffer
    pos2, _ = workloads.random_bodies(n, seed=79)
    pd.copy_(torch.from_numpy(pos2).cuda())
    nb.nbody_near_tree(pd, n, float(eps2), leaf, acc, pot, None)
    fresh = to_dev(pos2)
    acc2 = torch.empty((n, 4), device="cuda")
    pot2 = torch.empty((n,), device="cuda")
    nb.nbody_near_tree(fresh, n, float(eps2), leaf, acc2, pot2, None)
    torch.cuda.synchronize()
    assert np.array_equal(acc.cpu().numpy(), acc2.cpu().numpy())
    assert np.array_equal(pot.cpu().numpy(), pot2.cpu().numpy())
    assert_accel_parity(acc.cpu().numpy(), pot.cpu().numpy(),
                        oracle.near_tree(pos2, eps2, leaf, targets=idx), idx=idx,
                        what="tree, replay on new positions")
