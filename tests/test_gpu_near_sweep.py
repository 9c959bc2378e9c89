"""Seeded sweep of the near fields (grid and octree leaves) over mixed inputs: uniform,
clustered, flat and duplicate-heavy bodies, grid shapes from one cell per axis to 20, leaf
sizes from 1 to 500, with and without the potential; every target against the oracle's
definition, through the C ABI. The cases are drawn once from a fixed seed, so a failure names
a reproducible case."""

from __future__ import annotations

import numpy as np
import pytest

from gpu_util import assert_accel_parity, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nb():
    import direct_all_pairs_amd

    return direct_all_pairs_amd


def _bodies(kind: str, n: int, rng) -> np.ndarray:
    if kind == "uniform":
        x = rng.uniform(-1.0, 1.0, size=(n, 3))
    elif kind == "clustered":
        k = n // 3
        x = np.concatenate([rng.normal(0.3, 0.02, size=(k, 3)), rng.normal(-0.5, 0.1, size=(k, 3)),
                            rng.uniform(-1.0, 1.0, size=(n - 2 * k, 3))])
    elif kind == "flat":
        x = np.column_stack([rng.uniform(-1, 1, n), rng.uniform(-1, 1, n), np.full(n, 0.25)])
    else:  # duplicates: a few hundred distinct points, each repeated
        pts = rng.uniform(-1.0, 1.0, size=(max(n // 8, 1), 3))
        x = pts[rng.integers(0, pts.shape[0], n)]
    pos = np.zeros((n, 4), np.float32)
    pos[:, :3] = x
    pos[:, 3] = rng.uniform(0.5, 1.5, size=n) / n
    return pos


def _cases():
    rng = np.random.default_rng(20261202)
    kinds = ["uniform", "clustered", "flat", "duplicates"]
    out = []
    for i in range(24):
        kind = kinds[i % 4]
        n = int(rng.integers(1, 6000))
        dims = tuple(int(v) for v in rng.integers(1, 21, size=3))
        leaf = int(rng.choice([1, 2, 5, 16, 33, 64, 100, 500]))
        pot = bool(i % 5 != 4)
        out.append((i, kind, n, dims, leaf, pot))
    return out


@pytest.mark.parametrize("case", _cases(), ids=lambda c: f"{c[0]}-{c[1]}-n{c[2]}")
def test_near_fields_random_case(nb, case):
    import torch

    import oracle

    i, kind, n, dims, leaf, pot = case
    rng = np.random.default_rng(1000 + i)
    pos = _bodies(kind, n, rng)
    eps2 = float(10.0 ** rng.uniform(-6, -3))
    print(f"[sweep] case {i}: {kind} N={n} dims={dims} leaf={leaf} pot={pot} eps2={eps2:.2e}",
          flush=True)
    pd = to_dev(pos)
    # grid: the cube [-1.1, 1.1]^3 cut into dims cells of side h along the longest axis
    h = 2.2 / max(dims)
    lo = (-1.1, -1.1, -1.1)
    acc = torch.full((n, 4), np.nan, device="cuda")
    p = torch.full((n,), np.nan, device="cuda") if pot else None
    nb.nbody_near_grid(pd, n, eps2, lo, h, dims, acc, p)
    acc_t = torch.full((n, 4), np.nan, device="cuda")
    p_t = torch.full((n,), np.nan, device="cuda") if pot else None
    st = nb.nbody_tree_stats()
    nb.nbody_near_tree(pd, n, eps2, leaf, acc_t, p_t, st)
    torch.cuda.synchronize()
    ref_g = oracle.near_grid(pos, eps2, lo, h, dims)
    ref_t = oracle.near_tree(pos, eps2, leaf)
    if pot:
        assert_accel_parity(acc.cpu().numpy(), p.cpu().numpy(), ref_g, what=f"grid case {i}")
        assert_accel_parity(acc_t.cpu().numpy(), p_t.cpu().numpy(), ref_t, what=f"tree case {i}")
    else:
        # accelerations only: the potential columns of the reference are not compared
        a = acc.cpu().numpy()
        a_t = acc_t.cpu().numpy()
        assert np.all(a[:, 3] == 0.0) and np.all(a_t[:, 3] == 0.0)
        acc2 = torch.full((n, 4), np.nan, device="cuda")
        p2 = torch.full((n,), np.nan, device="cuda")
        nb.nbody_near_grid(pd, n, eps2, lo, h, dims, acc2, p2)
        acc3 = torch.full((n, 4), np.nan, device="cuda")
        p3 = torch.full((n,), np.nan, device="cuda")
        nb.nbody_near_tree(pd, n, eps2, leaf, acc3, p3, None)
        torch.cuda.synchronize()
        # the acceleration bits do not depend on whether the potential is computed
        assert np.array_equal(a, acc2.cpu().numpy()) and np.array_equal(a_t, acc3.cpu().numpy())
        assert_accel_parity(acc2.cpu().numpy(), p2.cpu().numpy(), ref_g, what=f"grid case {i}")
        assert_accel_parity(acc3.cpu().numpy(), p3.cpu().numpy(), ref_t, what=f"tree case {i}")
    assert 1 <= st.as_dict()["leaves"] <= n


@pytest.mark.parametrize("case", _cases(), ids=lambda c: f"{c[0]}-{c[1]}-n{c[2]}")
def test_near_grid_pairs_random_case(nb, case):
    """The same cases through the pair-symmetric near-grid kernel (forced, whatever the cell
    sizes): every target against the grid definition; the acceleration bits do not depend on
    the potential."""
    import torch

    import oracle

    i, kind, n, dims, _, pot = case
    rng = np.random.default_rng(1000 + i)
    pos = _bodies(kind, n, rng)
    eps2 = float(10.0 ** rng.uniform(-6, -3))
    print(f"[sweep] pairs case {i}: {kind} N={n} dims={dims} eps2={eps2:.2e}", flush=True)
    pd = to_dev(pos)
    h = 2.2 / max(dims)
    lo = (-1.1, -1.1, -1.1)
    acc = torch.full((n, 4), np.nan, device="cuda")
    p = torch.full((n,), np.nan, device="cuda")
    nb.nbody_near_grid_kernel(pd, n, eps2, lo, h, dims, nb.NEAR_PAIRS, acc, p)
    acc0 = torch.full((n, 4), np.nan, device="cuda")
    nb.nbody_near_grid_kernel(pd, n, eps2, lo, h, dims, nb.NEAR_PAIRS, acc0, None)
    torch.cuda.synchronize()
    ref = oracle.near_grid(pos, eps2, lo, h, dims)
    a = acc.cpu().numpy()
    assert_accel_parity(a, p.cpu().numpy(), ref, what=f"grid pairs case {i}")
    assert np.array_equal(acc0.cpu().numpy(), a)
