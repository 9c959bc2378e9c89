"""The fp64 oracle against its pins (closed forms, invariants, brute force). CPU only."""

import numpy as np
import pytest

import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)


def test_targets_subset_matches_full(orc):
    """The subset entry used for large-N sampling returns exactly the full run's rows."""
    import workloads

    pos, _ = workloads.random_bodies(300, seed=11)
    full = orc.accel(pos, 1e-4)
    idx = np.array([0, 299, 17, 150, 17])
    sub = orc.accel(pos, 1e-4, targets=idx)
    for k in ("acc", "pot", "bound_a", "bound_p"):
        assert np.array_equal(sub[k], full[k][idx])


def test_thread_count_independent(orc, monkeypatch):
    """Each target's sum is sequential, so the result is the same for any thread split."""
    import workloads

    pos, _ = workloads.random_bodies(257, seed=12)
    a = orc.accel(pos, 1e-4)
    b = orc.accel(pos, 1e-4, targets=np.arange(257)[::-1].copy())
    assert np.array_equal(a["acc"][::-1], b["acc"])


def test_float32_widening(orc):
    """float32 records are widened exactly; eps2 is the float32 value, widened."""
    pos = np.array([[0.1, 0.2, 0.3, 1.0], [0.4, 0.5, 0.6, 2.0]], dtype=np.float32)
    r32 = orc.accel(pos, 1e-4)
    r64 = orc.accel_exact(pos.astype(np.float64), float(np.float32(1e-4)))
    assert np.array_equal(r32["acc"], r64["acc"])


def test_rejects_bad_targets(orc):
    pos = np.zeros((3, 4))
    with pytest.raises(ValueError):
        orc.accel_exact(pos, 1.0, targets=[0, 3])
