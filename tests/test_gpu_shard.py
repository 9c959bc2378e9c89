"""GPU parity of the split evaluation (nbody_accel_shard, nbody_shard_finish) through the C
ABI: every shard's part against the oracle's shard definition, the merged parts against the
direct sum, one shard against nbody_accel bit for bit, and shards of the N = 2^20 cube."""

from __future__ import annotations

import numpy as np
import pytest

import workloads
from gpu_util import TOL, accel_errors, assert_accel_parity, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nb():
    import direct_all_pairs_amd

    return direct_all_pairs_amd


def run_shard(nb, pd, n, eps2, s, S, band, tpl=0, want_pot=True, run=0):
    import torch

    out = torch.full((n, 4), float("nan"), device="cuda")
    nb.nbody_accel_shard(pd, n, float(eps2), s, S, out, want_pot=want_pot,
                         plan=dict(mode="pairs", band=band, tpl=tpl, run=run))
    torch.cuda.synchronize()
    return out


def finish(nb, partials, n, S, t0, t1, pot=True):
    import torch

    acc = torch.full((t1 - t0, 4), float("nan"), device="cuda")
    p = torch.full((t1 - t0,), float("nan"), device="cuda") if pot else None
    nb.nbody_shard_finish(partials, n, S, t0, t1, acc, p)
    torch.cuda.synchronize()
    return acc.cpu().numpy(), (p.cpu().numpy() if p is not None else None)


def assert_part_parity(part, ref, what):
    """A shard's part: (ax, ay, az) within 1e-5 of the shard's own B_i, w = its sum of m/r
    within 1e-5 of its own P_i (a body the shard never pairs must get exact zeros)."""
    e_a, e_p = accel_errors(np.concatenate([part[:, :3], np.zeros((len(part), 1), np.float32)],
                                           axis=1), -part[:, 3], ref)
    assert np.all(np.isfinite(e_a)) and e_a.max() <= TOL, f"{what}: err/B {e_a.max():.3e}"
    assert e_p.max() <= TOL, f"{what}: err/P {e_p.max():.3e}"


# N, band, shard counts: even and odd band counts, a one-body last band, S = nb
SHARD_CASES = [(1, 512, (1,)), (2049, 512, (1, 2, 5)), (3000, 512, (2, 3, 6)),
               (5000, 1024, (2, 5)), (20011, 512, (8, 40))]


@pytest.mark.parametrize("n,band,shards", SHARD_CASES)
@pytest.mark.parametrize("tpl,run", [(4, 0), (8, 0), (8, 3)])
def test_shard_parts_and_merge(nb, n, band, shards, tpl, run):
    import torch

    import oracle

    eps2 = np.float32(1e-4)
    pos, _ = workloads.random_bodies(n, seed=900 + n)
    pd = to_dev(pos)
    rng = np.random.default_rng(n)
    idx = None if n <= 5000 else np.unique(np.concatenate(
        [rng.integers(0, n, 96), np.arange(0, n, band), [n - 1]]))
    full = oracle.accel(pos, eps2, targets=idx)
    for S in shards:
        parts = []
        for s in range(S):
            out = run_shard(nb, pd, n, eps2, s, S, band, tpl, run=run)
            part = out.cpu().numpy()
            ref = oracle.shard(pos, eps2, band, s, S, targets=idx)
            assert_part_parity(part if idx is None else part[idx], ref,
                               f"N={n} band={band} tpl={tpl} run={run} shard {s}/{S}")
            parts.append(out)
        stacked = torch.stack(parts).contiguous()
        acc, pot = finish(nb, stacked, n, S, 0, n)
        assert_accel_parity(acc, pot, full, idx=idx, what=f"N={n} merged S={S}")
        t0, t1 = n // 3, n // 3 + max(1, n // 4)
        a2, p2 = finish(nb, stacked, n, S, t0, t1)
        assert np.array_equal(a2, acc[t0:t1]) and np.array_equal(p2, pot[t0:t1])
        a3, p3 = finish(nb, stacked, n, S, t0, t1, pot=False)
        assert p3 is None and np.array_equal(a3, a2)


@pytest.mark.parametrize("n,band,run", [(3000, 512, 0), (3000, 512, 2), (70000, 2048, 0),
                                        (70000, 2048, 5), (70000, 4096, 0), (70000, 4096, 4)])
def test_one_shard_equals_accel(nb, n, band, run):
    """A single shard finished is nbody_accel_plan with the same pairs plan, bit for bit."""
    import torch

    pos, _ = workloads.random_bodies(n, seed=31)
    pd = to_dev(pos)
    plan = dict(mode="pairs", band=band, tpl=8, run=run)
    out = run_shard(nb, pd, n, 1e-4, 0, 1, band, 8, run=run)
    acc, pot = finish(nb, out.unsqueeze(0).contiguous(), n, 1, 0, n)
    a_ref = torch.empty((n, 4), device="cuda")
    p_ref = torch.empty((n,), device="cuda")
    nb.nbody_accel_plan(pd, n, 1e-4, a_ref, p_ref, plan)
    torch.cuda.synchronize()
    assert np.array_equal(acc, a_ref.cpu().numpy()) and np.array_equal(pot, p_ref.cpu().numpy())


def test_shard_without_potential_and_determinism(nb):
    pos, _ = workloads.random_bodies(4100, seed=5)
    pd = to_dev(pos)
    a = run_shard(nb, pd, 4100, 1e-4, 1, 3, 512).cpu().numpy()
    b = run_shard(nb, pd, 4100, 1e-4, 1, 3, 512).cpu().numpy()
    c = run_shard(nb, pd, 4100, 1e-4, 1, 3, 512, want_pot=False).cpu().numpy()
    assert np.array_equal(a, b)
    assert np.array_equal(c[:, :3], a[:, :3]) and np.all(c[:, 3] == 0.0)


def test_shards_of_cube1m_sampled(nb):
    """N = 2^20 in eight shards (one GPU's share each, at its real shape): the first and the
    last shard against the oracle's shard sums, and the merged result against the direct sum,
    on sampled targets (each shard's band boundaries and random bodies)."""
    import torch

    import oracle

    w = workloads.make("cube1m")
    n, S = w.n, 8
    pd = to_dev(w.pos)
    band = nb.nbody_plan_for(n).band
    rng = np.random.default_rng(8)
    idx = np.unique(np.concatenate([rng.integers(0, n, 48), np.arange(0, n, n // S),
                                    np.arange(n // S - 1, n, n // S)]))
    parts = []
    for s in range(S):
        out = run_shard(nb, pd, n, w.eps2, s, S, band)
        if s in (0, S - 1):
            ref = oracle.shard(w.pos, w.eps2, band, s, S, targets=idx)
            assert_part_parity(out.cpu().numpy()[idx], ref, f"cube1m shard {s}/{S}")
        parts.append(out)
    acc, pot = finish(nb, torch.stack(parts).contiguous(), n, S, 0, n)
    assert_accel_parity(acc, pot, oracle.accel(w.pos, w.eps2, targets=idx), idx=idx,
                        what="cube1m merged")
