"""The parity checker used by the GPU tests, exercised on the CPU with oracle
results rounded to float32 (must pass) and with planted errors (must fail)."""

import numpy as np
import pytest

import workloads
from gpu_util import assert_accel_parity, assert_step_parity


def _as_gpu(ref):
    n = ref["acc"].shape[0]
    acc = np.zeros((n, 4), np.float32)
    acc[:, :3] = ref["acc"]
    return acc, ref["pot"].astype(np.float32)


def test_checker_accepts_rounded_oracle(orc):
    pos, _ = workloads.random_bodies(500, seed=1)
    ref = orc.accel(pos, 1e-4)
    acc, pot = _as_gpu(ref)
    assert_accel_parity(acc, pot, ref)


def test_checker_single_body_zero_scale(orc):
    pos = np.array([[0.1, 0.2, 0.3, 1.0]], np.float32)
    ref = orc.accel(pos, 1e-4)
    acc, pot = _as_gpu(ref)
    assert_accel_parity(acc, pot, ref)
    acc[0, 0] = 1e-30
    with pytest.raises(AssertionError):
        assert_accel_parity(acc, pot, ref)


@pytest.mark.parametrize("what", ["acc", "pot", "w"])
def test_checker_rejects_planted_error(orc, what):
    pos, _ = workloads.random_bodies(500, seed=2)
    ref = orc.accel(pos, 1e-4)
    acc, pot = _as_gpu(ref)
    if what == "acc":
        acc[17, 1] += np.float32(3e-5 * ref["bound_a"][17])
    elif what == "pot":
        pot[3] *= np.float32(1 + 3e-5)
    else:
        acc[5, 3] = 1.0
    with pytest.raises(AssertionError):
        assert_accel_parity(acc, pot, ref)


def test_step_checker(orc):
    pos, vel = workloads.random_bodies(300, seed=3)
    dt = np.float32(1e-3)
    ref = orc.accel(pos, 1e-4)
    p64, v64 = orc.euler(pos, vel, dt, 1e-4, 1)
    p1, v1 = p64.astype(np.float32), v64.astype(np.float32)
    p1[:, 3], v1[:, 3] = pos[:, 3], vel[:, 3]
    assert_step_parity(pos, vel, p1, v1, dt, ref)
    bad = v1.copy()
    bad[7, 0] += np.float32(1e-3)
    with pytest.raises(AssertionError):
        assert_step_parity(pos, vel, p1, bad, dt, ref)
    bad = p1.copy()
    bad[9, 2] = np.nextafter(np.nextafter(bad[9, 2], np.float32(9)), np.float32(9))
    bad[9, 2] = np.nextafter(bad[9, 2], np.float32(9))
    with pytest.raises(AssertionError):
        assert_step_parity(pos, vel, bad, v1, dt, ref)
