"""nbody_time_kernel, the measurement hook bench.py times the pair-term kernel with: the
events the library records around the first pair-term kernel launch of a call bracket a
positive interval inside the call, the results do not depend on the hook, and once it is
switched off later calls leave the events alone."""

from __future__ import annotations

import numpy as np
import pytest

import workloads
from gpu_util import to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nb():
    import direct_all_pairs_amd

    return direct_all_pairs_amd


def _events(k):
    import torch

    ev = [torch.cuda.Event(enable_timing=True) for _ in range(k)]
    for e in ev:
        e.record()
    return ev


@pytest.mark.parametrize("n", [3000, 20011])  # small-N kernel; pair bands and their combine
def test_time_kernel_brackets_the_first_pair_term_launch(nb, n):
    import torch

    print(f"[timing] N={n} plan={nb.nbody_plan_for(n).as_dict()}", flush=True)
    pos_h, vel_h = workloads.random_bodies(n, seed=n)
    pos, vel = to_dev(pos_h), to_dev(vel_h)
    acc0, pot0 = torch.empty_like(pos), torch.empty(n, device=pos.device)
    nb.nbody_accel(pos, n, 1e-4, acc0, pot0)
    ka, kb, ca, cb = _events(4)
    acc, pot = torch.empty_like(pos), torch.empty(n, device=pos.device)
    nb.nbody_time_kernel(ka, kb)
    ca.record()
    nb.nbody_accel(pos, n, 1e-4, acc, pot)
    cb.record()
    torch.cuda.synchronize()
    nb.nbody_time_kernel(None, None)
    k, c = ka.elapsed_time(kb), ca.elapsed_time(cb)
    assert 0.0 < k <= c, (k, c)
    assert torch.equal(acc, acc0) and torch.equal(pot, pot0)  # the hook changes nothing
    # switched off: another call does not record the events again
    nb.nbody_accel(pos, n, 1e-4, acc, pot)
    torch.cuda.synchronize()
    assert ka.elapsed_time(kb) == k
    # a step call: the first step's launch is bracketed, the rest are not
    ka2, kb2, ca2, cb2 = _events(4)
    nb.nbody_time_kernel(ka2, kb2)
    ca2.record()
    nb.nbody_step(pos, vel, n, 1e-3, 1e-4, 5)
    cb2.record()
    torch.cuda.synchronize()
    nb.nbody_time_kernel(None, None)
    k2, c2 = ka2.elapsed_time(kb2), ca2.elapsed_time(cb2)
    assert 0.0 < k2 < c2, (k2, c2)
    assert np.all(np.isfinite(pos.cpu().numpy()))
