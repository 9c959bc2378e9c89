"""Race probe (GPU): the test build of the library refills every LDS slot that a barrier
hands back only after first writing NaN into it, so a missing or misplaced barrier shows up
as NaN or changed outputs. With the barriers in place its results must equal the library's
bit for bit, with no NaN, for tile counts and sizes at tile boundaries +- 1 in every mode that
shares LDS between waves (tiles, small N, pair bands and runs of band pairs, the near-field
kernels)."""

from __future__ import annotations

import ctypes

import numpy as np
import pytest

import workloads
from gpu_util import to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nb():
    import direct_all_pairs_amd

    return direct_all_pairs_amd


@pytest.fixture(scope="module")
def probe(nb):
    from direct_all_pairs_amd import build

    if not build.PROBE_LIB.exists():
        pytest.fail(f"{build.PROBE_LIB} is not built (run __graft_entry__.build())")
    lib = ctypes.CDLL(str(build.PROBE_LIB))
    vp, i64, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float
    lib.nbody_accel_plan.argtypes = [vp, i64, f32, vp, vp, ctypes.POINTER(nb.nbody_plan), vp]
    lib.nbody_step_plan.argtypes = [vp, vp, i64, f32, f32, i64, ctypes.POINTER(nb.nbody_plan), vp]
    lib.nbody_near_grid.argtypes = [vp, i64, f32, ctypes.POINTER(ctypes.c_float), f32,
                                    ctypes.POINTER(ctypes.c_int32), vp, vp, vp]
    lib.nbody_near_grid_kernel.argtypes = [vp, i64, f32, ctypes.POINTER(ctypes.c_float), f32,
                                           ctypes.POINTER(ctypes.c_int32), ctypes.c_int32, vp,
                                           vp, vp]
    lib.nbody_p2p.argtypes = [vp, i64, f32, vp, ctypes.c_int32, vp, vp, i64, vp, vp, vp]
    lib.nbody_last_error.restype = ctypes.c_char_p
    return lib


def _stream():
    import torch

    return torch.cuda.current_stream().cuda_stream


def _accel_both(nb, probe, pos_h, eps2, plan):
    import torch

    n = pos_h.shape[0]
    pd = to_dev(pos_h)
    outs = []
    for which in ("library", "probe"):
        acc = torch.full((n, 4), 7.0, device="cuda")
        pot = torch.full((n,), 7.0, device="cuda")
        p = nb.make_plan(**plan)
        if which == "library":
            nb.nbody_accel_plan(pd, n, eps2, acc, pot, p)
        else:
            rc = probe.nbody_accel_plan(pd.data_ptr(), n, eps2, acc.data_ptr(), pot.data_ptr(),
                                        ctypes.byref(p), _stream())
            assert rc == 0, probe.nbody_last_error()
        torch.cuda.synchronize()
        outs.append((acc.cpu().numpy(), pot.cpu().numpy()))
    return outs


def _assert_same(outs, what):
    (a0, p0), (a1, p1) = outs
    assert not np.isnan(a1).any() and not np.isnan(p1).any(), f"{what}: NaN from the probe build"
    assert np.array_equal(a0, a1) and np.array_equal(p0, p1), f"{what}: probe build differs"


PROBE_CASES = (
    [dict(bcast="lds", tpl=1, wg=wg, splits=s) for wg in (64, 128, 256, 512) for s in (1, 3)]
    + [dict(mode="small", tpl=tw) for tw in (4, 8, 16, 32)]
    + [dict(mode="pairs", band=b, tpl=t)
       for b, t in ((256, 4), (512, 4), (512, 8), (1024, 4), (1024, 8), (2048, 8), (4096, 8))]
    # runs of several band pairs that keep the walked band's sums in LDS (or, with 4096-body
    # bands, in its global slot) across their items; run 16 with a split tail on 40 bands
    + [dict(mode="pairs", band=b, tpl=t, run=r)
       for b, t, r in ((256, 4, 2), (512, 8, 2), (2048, 8, 2), (4096, 8, 2), (256, 4, 16))]
)


def _sizes(plan):
    if plan.get("mode") == "small":
        return (2047, 2049, 3073)
    tile = plan.get("band") or plan["wg"]
    k = 4 if plan.get("mode") == "pairs" else 6
    if plan.get("run", 0) >= 16:
        k = 40  # 20 band pairs per owner band: one run of 4, then the last 16 split into four
    return (k * tile - 1, k * tile + 1)


@pytest.mark.parametrize("plan", PROBE_CASES, ids=lambda p: "-".join(f"{k}{v}" for k, v in p.items()))
def test_probe_build_matches_library(nb, probe, plan):
    for n in _sizes(plan):
        pos, _ = workloads.random_bodies(n, seed=70 + n)
        _assert_same(_accel_both(nb, probe, pos, 1e-4, plan), f"N={n} {plan}")


def test_probe_build_small_steps(nb, probe):
    """Small-mode steps (alternating position buffers) agree bit for bit over three steps."""
    import torch

    n = 3073
    pos_h, vel_h = workloads.random_bodies(n, seed=9)
    res = []
    for which in ("library", "probe"):
        pos, vel = to_dev(pos_h), to_dev(vel_h)
        p = nb.make_plan(mode="small", tpl=8)
        if which == "library":
            nb.nbody_step_plan(pos, vel, n, 1e-3, 1e-4, 3, p)
        else:
            rc = probe.nbody_step_plan(pos.data_ptr(), vel.data_ptr(), n, 1e-3, 1e-4, 3,
                                       ctypes.byref(p), _stream())
            assert rc == 0, probe.nbody_last_error()
        torch.cuda.synchronize()
        res.append((pos.cpu().numpy(), vel.cpu().numpy()))
    assert np.array_equal(res[0][0], res[1][0]) and np.array_equal(res[0][1], res[1][1])


@pytest.mark.parametrize("kernel", [1, 2])
@pytest.mark.parametrize("n,h,dims", [(20000, 1.0, (2, 2, 2)),
                                      (800000, 0.125, (16, 16, 16)),
                                      (100000, 0.125, (16, 16, 16))])
def test_probe_build_chunk_near_field(nb, probe, n, h, dims, kernel):
    """The near-field kernels whose four waves add their sums through a shared buffer. The
    one-sided chunk kernel (kernel 1): eight large cells (2 x 2 x 2 grid, ~2500 bodies each:
    42 workgroups per cell, each with one or two 64-target chunks and many source tiles), 4096
    cells of ~195 and of ~24 bodies (64-target chunks, and source groups for small chunks). The
    pair-symmetric kernel (kernel 2): the same grids, i.e. five 512-body i-sets per large cell
    with the block and sum rows reused between them, and one i-set of 1 to 5 rows per cell."""
    import torch

    pos_h, _ = workloads.random_bodies(n, seed=12)
    pd = to_dev(pos_h)
    lo = (-1.0, -1.0, -1.0)
    outs = []
    for which in ("library", "probe"):
        acc = torch.full((n, 4), 7.0, device="cuda")
        pot = torch.full((n,), 7.0, device="cuda")
        if which == "library":
            nb.nbody_near_grid_kernel(pd, n, 1e-4, lo, h, dims, kernel, acc, pot)
        else:
            rc = probe.nbody_near_grid_kernel(pd.data_ptr(), n, 1e-4, (ctypes.c_float * 3)(*lo),
                                              h, (ctypes.c_int32 * 3)(*dims), kernel,
                                              acc.data_ptr(), pot.data_ptr(), _stream())
            assert rc == 0, probe.nbody_last_error()
        torch.cuda.synchronize()
        outs.append((acc.cpu().numpy(), pot.cpu().numpy()))
    _assert_same(outs, f"near grid kernel {kernel}, {dims} cells")


@pytest.mark.parametrize("n,ncell,per_list", [(3000, 150, 172), (12000, 150, 172),
                                               (600000, 3100, 70)])
def test_probe_build_list_segments(nb, probe, n, ncell, per_list):
    """CSR lists of more than 64 entries: the near-field kernel walks them in segments whose
    table wave 0 rewrites in LDS between two workgroup barriers: one wave per cell at ~20
    bodies per cell, four waves at ~80, four workgroups of four waves per cell at ~190."""
    import torch

    pos_h, _ = workloads.random_bodies(n, seed=13)
    rng = np.random.default_rng(ncell)
    cuts = np.sort(rng.integers(0, n + 1, ncell - 1))
    start = np.concatenate([[0], cuts, [n]]).astype(np.int32)
    lists = [list(rng.integers(0, ncell, per_list)) for _ in range(ncell)]
    off = np.zeros(ncell + 1, np.int32)
    off[1:] = np.cumsum([len(x) for x in lists])
    flat = np.array([c for x in lists for c in x], np.int32)
    pd = to_dev(pos_h)
    st, of, fl = (torch.from_numpy(a).cuda() for a in (start, off, flat))
    outs = []
    for which in ("library", "probe"):
        acc = torch.full((n, 4), 7.0, device="cuda")
        pot = torch.full((n,), 7.0, device="cuda")
        if which == "library":
            nb.nbody_p2p(pd, n, 1e-4, st, ncell, of, fl, len(flat), acc, pot)
        else:
            rc = probe.nbody_p2p(pd.data_ptr(), n, 1e-4, st.data_ptr(), ncell, of.data_ptr(),
                                 fl.data_ptr(), len(flat), acc.data_ptr(), pot.data_ptr(),
                                 _stream())
            assert rc == 0, probe.nbody_last_error()
        torch.cuda.synchronize()
        outs.append((acc.cpu().numpy(), pot.cpu().numpy()))
    _assert_same(outs, f"p2p lists of {per_list} entries, {ncell} cells")
