"""Seeded input generators: reproducibility, shapes, bounds and distribution checks. CPU only."""

import numpy as np
import pytest
from scipy import stats

import workloads


def test_seed_reproducible():
    a = workloads.uniform_cube(1000)
    b = workloads.uniform_cube(1000)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    c = workloads.uniform_cube(1000, seed=1)
    assert not np.array_equal(a[0], c[0])


def test_disk():
    w = workloads.make("disk4096")
    assert w.pos.dtype == np.float32 and w.pos.shape == (4096, 4)
    assert np.all(w.pos[:, 2] == 0) and np.all(w.vel[:, 2] == 0) and np.all(w.pos[:, 3] == 1)
    assert np.all(np.abs(w.pos[:, :2]) <= 1) and np.all(np.abs(w.vel[:, :2]) <= 1)
    assert w.eps2 == np.float32(1e-6) and w.dt == np.float32(1e-3) and w.nsteps == 1
    # uniform: mean ~ 0, variance ~ 1/3
    assert abs(w.pos[:, 0].mean()) < 0.05 and abs(w.pos[:, 0].var() - 1 / 3) < 0.02


@pytest.mark.parametrize("name,n", [("cube2048_steps", 2048), ("cube1m", 1 << 20)])
def test_cube(name, n):
    w = workloads.make(name)
    assert w.n == n
    assert np.all(np.abs(w.pos[:, :3]) <= 1)
    m = w.pos[:, 3].astype(np.float64) * n
    assert m.min() >= 0.5 * (1 - 1e-6) and m.max() <= 1.5 * (1 + 1e-6)
    assert np.all(w.vel == 0)
    assert w.eps2 == np.float32(1e-4)


def _plummer_cdf(r):
    return r ** 3 / (r * r + 1.0) ** 1.5


def test_plummer_radial_profile():
    """Kolmogorov-Smirnov test of radii against M(<r)/M = r^3/(r^2+1)^(3/2)."""
    w = workloads.make("plummer65536")
    r = np.linalg.norm(w.pos[:, :3].astype(np.float64), axis=1)
    ks = stats.kstest(r, _plummer_cdf)
    assert ks.pvalue > 1e-3, ks
    assert np.all(w.pos[:, 3] == np.float32(2.0 ** -16))
    assert w.eps2 == np.float32(1e-4) and w.want_pot


def test_plummer_velocity_scale():
    """Mean square speed of a Plummer sphere (M = a = G = 1) is 3 pi / 32."""
    w = workloads.make("plummer65536")
    v2 = (w.vel[:, :3].astype(np.float64) ** 2).sum(axis=1)
    assert abs(v2.mean() / (3 * np.pi / 32) - 1) < 0.03
    # speeds never exceed the local escape speed
    r = np.linalg.norm(w.pos[:, :3].astype(np.float64), axis=1)
    vesc = np.sqrt(2.0) * (r * r + 1) ** -0.25
    assert np.all(np.sqrt(v2) <= vesc * (1 + 1e-6))


def test_plummer_virial_and_mean_field(orc):
    """2K/|W| ~ 1, W ~ -3 pi/32, and each body's potential ~ -1/sqrt(r^2+1) (Plummer, M = a = 1)."""
    pos, vel = workloads.plummer_bodies(4096, seed=5)
    E, K, W = orc.energy(pos, vel, 1e-4)
    assert abs(W / (-3 * np.pi / 32) - 1) < 0.05
    assert abs(2 * K / abs(W) - 1) < 0.08
    r = orc.accel(pos, 1e-4)
    m = pos[:, 3].astype(np.float64)
    p_excl = r["pot"] + m / np.sqrt(np.float64(np.float32(1e-4)))
    rad = np.linalg.norm(pos[:, :3].astype(np.float64), axis=1)
    phi = -(1 - 1 / 4096) / np.sqrt(rad * rad + 1)
    assert np.median(np.abs(p_excl / phi - 1)) < 0.03


def test_two_plummer():
    w = workloads.make("two_plummer300007")
    assert w.n == 300_007 and w.meta["n_a"] == 150_003
    m = w.pos[:, 3].astype(np.float64)
    assert abs(m.sum() - 1) < 1e-5 and np.all(m > 0)
    a, b = w.pos[:150_003, :3].astype(np.float64), w.pos[150_003:, :3].astype(np.float64)
    assert np.allclose(np.median(a, axis=0), [4, 0, 0], atol=0.03)
    assert np.allclose(np.median(b, axis=0), [-4, 0, 0], atol=0.03)
    va, vb = w.vel[:150_003, :3].astype(np.float64), w.vel[150_003:, :3].astype(np.float64)
    assert np.allclose(va.mean(axis=0), [-0.3, 0.1, 0], atol=0.01)
    assert np.allclose(vb.mean(axis=0), [0.3, 0.1, 0], atol=0.01)
    # log-normal masses: log m has standard deviation 1
    assert abs(np.log(m).std() - 1) < 0.01
    assert w.eps2 == np.float32(4e-4) and w.nsteps == 10 and w.dt == np.float32(1e-3)


def test_dyadic_grid():
    pos, _ = workloads.dyadic_grid_bodies(500, seed=1)
    k = pos[:, :3].astype(np.float64) * 1024
    assert np.array_equal(k, np.round(k))
    assert np.all(np.abs(pos[:, :3]) <= 0.5)
