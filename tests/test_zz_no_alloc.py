"""nbody_step_noalloc, the step entry point for callers that cannot allocate
device memory: its scratch comes from the library's static array, and its
results equal nbody_step's bit for bit (same plan, same kernels). Checked on
two calls in a row, the second with a smaller input, plus the first step of
each against the fp64 oracle under the one-step bound, the size limit, and
that a call takes no device memory.
"""

from __future__ import annotations

import numpy as np
import pytest

import workloads
from gpu_util import assert_step_parity, to_dev

pytestmark = pytest.mark.gpu

DT, EPS2 = np.float32(1e-3), np.float32(1e-4)


@pytest.fixture(scope="module")
def nb():
    import direct_all_pairs_amd

    return direct_all_pairs_amd


def _both(nb, n, nsteps, seed):
    """The same state stepped by nbody_step and by nbody_step_noalloc."""
    import torch

    pos_h, vel_h = workloads.random_bodies(n, seed=seed)
    vel_h = vel_h.copy()
    vel_h[:, :3] = np.random.default_rng(seed).uniform(-0.5, 0.5, (n, 3)).astype(np.float32)
    p_ref, v_ref = to_dev(pos_h), to_dev(vel_h)
    p_new, v_new = to_dev(pos_h), to_dev(vel_h)
    print(f"[no_alloc] N={n} nsteps={nsteps} plan={nb.nbody_plan_for(n).as_dict()}", flush=True)
    nb.nbody_step(p_ref, v_ref, n, float(DT), float(EPS2), nsteps)
    nb.nbody_step_noalloc(p_new, v_new, n, float(DT), float(EPS2), nsteps)
    torch.cuda.synchronize()
    return pos_h, vel_h, (p_ref, v_ref), (p_new, v_new)


def test_noalloc_equals_step_two_calls_second_smaller(nb):
    """A pair-band plan (N = 20011, 3 steps) and then a small-N plan (N = 3001, 5 steps: an
    odd count, whose final positions are copied back from the second buffer) in a row; each
    equal to nbody_step bit for bit, and one noalloc step of each within the oracle's bound."""
    import oracle
    import torch

    for n, nsteps, mode in ((20011, 3, nb.MODE_PAIRS), (3001, 5, nb.MODE_SMALL)):
        assert nb.nbody_plan_for(n).mode == mode
        _, _, (p_ref, v_ref), (p_new, v_new) = _both(nb, n, nsteps, seed=n)
        assert torch.equal(p_ref, p_new) and torch.equal(v_ref, v_new), f"N={n}: bits differ"
        # one step of the static-scratch path against the oracle
        pos_h, vel_h = workloads.random_bodies(n, seed=n + 1)
        pos, vel = to_dev(pos_h), to_dev(vel_h)
        nb.nbody_step_noalloc(pos, vel, n, float(DT), float(EPS2), 1)
        torch.cuda.synchronize()
        ref = oracle.accel(pos_h, EPS2)
        assert_step_parity(pos_h, vel_h, pos.cpu().numpy(), vel.cpu().numpy(), DT, ref,
                           what=f"noalloc N={n}")


def test_noalloc_rejects_beyond_static_scratch(nb):
    """N = 70000 needs 137 x N x 16 bytes of pair slots (> 128 MiB): NBODY_EINVAL, nothing
    enqueued, inputs untouched (real buffers of that size, so no launch could misbehave)."""
    import torch

    n = 70000
    pos_h, vel_h = workloads.random_bodies(n, seed=7)
    pos, vel = to_dev(pos_h), to_dev(vel_h)
    rc = nb.nbody_step_noalloc(pos, vel, n, float(DT), float(EPS2), 1, check=False)
    assert rc == nb.NBODY_EINVAL and "static" in nb.nbody_last_error()
    torch.cuda.synchronize()
    assert np.array_equal(pos.cpu().numpy(), pos_h) and np.array_equal(vel.cpu().numpy(), vel_h)


def _pair_step_bytes(nb, n):
    """Scratch of the automatic plan's pair step: 1 + R + D slots of N records (D = nb/2, R runs
    of the plan's length, the last run of 16 or more split into four)."""
    p = nb.nbody_plan_for(n)
    assert p.mode == nb.MODE_PAIRS and p.passes == 1, p.as_dict()
    d, k = p.splits // 2, p.run
    r = (-(-(d - k) // k) + 4) if (k >= 16 and d > k) else -(-d // k)
    return (1 + r + d) * n * 16


@pytest.mark.parametrize("n", [65027, 65028])
def test_noalloc_limit_at_the_boundary(nb, n):
    """Just below and just above the 128 MiB array (N = 65027: 129 slots of N records take
    134,215,728 of its 134,217,728 bytes; N = 65028 needs 64 bytes more): the first runs a step
    equal to nbody_step bit for bit, the second is rejected before anything is enqueued."""
    import torch

    need = _pair_step_bytes(nb, n)
    fits = need <= 128 * 1024 * 1024
    assert fits == (n == 65027), need
    pos_h, vel_h = workloads.random_bodies(n, seed=13)
    pos, vel = to_dev(pos_h), to_dev(vel_h)
    rc = nb.nbody_step_noalloc(pos, vel, n, float(DT), float(EPS2), 1, check=False)
    torch.cuda.synchronize()
    if not fits:
        assert rc == nb.NBODY_EINVAL and "static" in nb.nbody_last_error()
        assert np.array_equal(pos.cpu().numpy(), pos_h) and np.array_equal(vel.cpu().numpy(), vel_h)
        return
    assert rc == 0, nb.nbody_last_error()
    p2, v2 = to_dev(pos_h), to_dev(vel_h)
    nb.nbody_step(p2, v2, n, float(DT), float(EPS2), 1)
    torch.cuda.synchronize()
    assert np.array_equal(pos.cpu().numpy(), p2.cpu().numpy())
    assert np.array_equal(vel.cpu().numpy(), v2.cpu().numpy())


def test_noalloc_takes_no_device_memory(nb):
    """After the library's cached scratch is released, a noalloc call leaves the device's
    free memory where it was, while nbody_step of the same size takes its slot array."""
    import torch

    n, nsteps = 20011, 2
    pos_h, vel_h = workloads.random_bodies(n, seed=11)
    pos, vel = to_dev(pos_h), to_dev(vel_h)
    nb.nbody_step_noalloc(pos, vel, 64, float(DT), float(EPS2), 1)  # static array in place
    torch.cuda.synchronize()
    nb.nbody_release_workspace()
    free0 = torch.cuda.mem_get_info()[0]
    nb.nbody_step_noalloc(pos, vel, n, float(DT), float(EPS2), nsteps)
    torch.cuda.synchronize()
    free1 = torch.cuda.mem_get_info()[0]
    nb.nbody_step(pos, vel, n, float(DT), float(EPS2), nsteps)
    torch.cuda.synchronize()
    free2 = torch.cuda.mem_get_info()[0]
    slots = nb.nbody_plan_for(n).splits * n * 16
    assert free0 - free1 < (4 << 20), f"noalloc took {free0 - free1} bytes"
    assert free1 - free2 >= slots, f"nbody_step took {free1 - free2} < {slots} bytes"
    nb.nbody_release_workspace()
