"""Seeded synthetic inputs for the direct all-pairs softened-gravity path.

This module only draws initial conditions. It holds none of the arithmetic of
the method itself (no accelerations, potentials or integration): both the fp64
oracle and the GPU path receive the float32 arrays built here.

Conventions (shared by every generator):

* Bodies are packed as float32 ``(N, 4)`` arrays: ``pos[i] = (x, y, z, m)`` with
  the mass in the fourth slot, ``vel[i] = (vx, vy, vz, 0)``. This is the
  array-of-structures particle record of the ATI Stream slides (Nakasato,
  "スライド 1", No.5) and of the float4 body in GPU Gems 3 ch. 31 as retold on
  the CSDN "Cuda Nbody笔记" page.
* Every value is drawn in float64 and then rounded once to float32; the float32
  arrays are the canonical input.
* The random stream is ``numpy.random.Generator(PCG64(seed))`` and the default
  seed is N, echoing the lecture's CPU program that seeds its generator with
  the body count (Degawa, "N 体問題", slide 14). Draws happen in the order the
  code below makes them; changing that order changes the workload.
* "Uniform in [a, b]" means ``a + (b - a) * U`` with ``U = rng.random()``.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "Workload",
    "uniform_disk",
    "uniform_cube",
    "plummer_sphere",
    "two_plummer",
    "random_bodies",
    "dyadic_grid_bodies",
    "make",
    "CONFIGS",
]


@dataclass
class Workload:
    name: str
    pos: np.ndarray  # float32 (N, 4): x, y, z, m
    vel: np.ndarray  # float32 (N, 4): vx, vy, vz, 0
    eps2: np.float32
    dt: np.float32 | None = None
    nsteps: int = 0
    want_pot: bool = False
    meta: dict = field(default_factory=dict)

    @property
    def n(self) -> int:
        return int(self.pos.shape[0])


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(int(seed)))


def _pack(x, y, z, m, vx, vy, vz) -> tuple[np.ndarray, np.ndarray]:
    n = len(x)
    pos = np.empty((n, 4), dtype=np.float32)
    vel = np.zeros((n, 4), dtype=np.float32)
    pos[:, 0], pos[:, 1], pos[:, 2], pos[:, 3] = x, y, z, m
    vel[:, 0], vel[:, 1], vel[:, 2] = vx, vy, vz
    return pos, vel


def uniform_disk(n: int, seed: int | None = None) -> tuple[np.ndarray, np.ndarray]:
    """Planar disk of the lecture's CPU program (Degawa, "N 体問題", slide 14).

    x, y, vx, vy uniform in [-1, 1]; z = vz = 0; unit masses. Per body the draw
    order is x, y, vx, vy, as in that program's initial-value loop.
    """
    rng = _rng(n if seed is None else seed)
    u = rng.random((n, 4))  # row i: x, y, vx, vy of body i
    c = 2.0 * u - 1.0
    z = np.zeros(n)
    return _pack(c[:, 0], c[:, 1], z, np.ones(n), c[:, 2], c[:, 3], z)


def uniform_cube(n: int, seed: int | None = None) -> tuple[np.ndarray, np.ndarray]:
    """Uniform cube [-1, 1]^3, masses uniform in [0.5, 1.5]/N, zero velocities."""
    rng = _rng(n if seed is None else seed)
    xyz = 2.0 * rng.random((n, 3)) - 1.0
    m = (0.5 + rng.random(n)) / n
    z = np.zeros(n)
    return _pack(xyz[:, 0], xyz[:, 1], xyz[:, 2], m, z, z, z)


def _isotropic(rng: np.random.Generator, r: np.ndarray) -> np.ndarray:
    """Points at radius r with isotropic directions: cos(theta) and phi uniform."""
    n = len(r)
    u = rng.random((n, 2))
    cth = 2.0 * u[:, 0] - 1.0
    sth = np.sqrt(np.maximum(0.0, 1.0 - cth * cth))
    phi = 2.0 * np.pi * u[:, 1]
    return np.stack([r * sth * np.cos(phi), r * sth * np.sin(phi), r * cth], axis=1)


def _plummer_q(rng: np.random.Generator, n: int) -> np.ndarray:
    """Speed fraction q = v / v_esc by rejection from g(q) = q^2 (1 - q^2)^(7/2).

    max g is about 0.0920 (at q^2 = 2/9), so a box of height 0.1 covers it and
    about 43 % of the draws are accepted. Batches are drawn until n samples
    are accepted; accepted samples keep their draw order.
    """
    out = np.empty(0)
    while out.size < n:
        k = 64 + 3 * (n - out.size)
        q = rng.random(k)
        y = 0.1 * rng.random(k)
        ok = y < q * q * (1.0 - q * q) ** 3.5
        out = np.concatenate([out, q[ok]])
    return out[:n]


def plummer_sphere(
    n: int,
    total_mass: float = 1.0,
    seed: int | None = None,
    rng: np.random.Generator | None = None,
) -> tuple[np.ndarray, np.ndarray]:
    """Plummer sphere, scale radius 1, G = 1, equal masses total_mass/n, fp64.

    Radius from the inverse of the cumulative mass M(<r)/M = r^3/(r^2+1)^(3/2):
    r = (X^(-2/3) - 1)^(-1/2), X uniform. Speeds q * v_esc(r) with
    v_esc = sqrt(2 M) (r^2 + 1)^(-1/4) and q from the Plummer distribution
    function (Aarseth, Henon & Wielen 1974 construction); isotropic directions
    for both. No truncation and no recentring. Returns fp64 arrays
    (xyz, vxyz) of shape (n, 3).
    """
    if rng is None:
        rng = _rng(n if seed is None else seed)
    x = rng.random(n)
    with np.errstate(divide="ignore"):
        r = 1.0 / np.sqrt(x ** (-2.0 / 3.0) - 1.0)
    xyz = _isotropic(rng, r)
    q = _plummer_q(rng, n)
    vesc = np.sqrt(2.0 * total_mass) * (r * r + 1.0) ** -0.25
    vxyz = _isotropic(rng, q * vesc)
    return xyz, vxyz


def plummer_bodies(n: int, seed: int | None = None) -> tuple[np.ndarray, np.ndarray]:
    """Single Plummer sphere with total mass 1 and equal masses 1/N, as float32 records."""
    xyz, v = plummer_sphere(n, 1.0, seed=seed)
    m = np.full(n, 1.0 / n)
    return _pack(xyz[:, 0], xyz[:, 1], xyz[:, 2], m, v[:, 0], v[:, 1], v[:, 2])


def two_plummer(
    n_a: int = 150_003, n_b: int = 150_004, seed: int | None = None
) -> tuple[np.ndarray, np.ndarray]:
    """Two Plummer spheres on a collision course with log-normal masses.

    Bodies [0, n_a) form sphere A centred at (+4, 0, 0) moving with (-0.3, 0.1, 0);
    bodies [n_a, n_a + n_b) form sphere B at (-4, 0, 0) moving with (+0.3, 0.1, 0).
    Masses are exp(Z), Z standard normal, normalised in fp64 to a total of 1
    over all bodies; each sphere's velocity scale uses its own mass M_s.
    Draw order: all n_a + n_b normals, then sphere A, then sphere B.
    """
    n = n_a + n_b
    rng = _rng(n if seed is None else seed)
    w = np.exp(rng.standard_normal(n))
    m = w / w.sum()
    ma, mb = m[:n_a].sum(), m[n_a:].sum()
    xa, va = plummer_sphere(n_a, ma, rng=rng)
    xb, vb = plummer_sphere(n_b, mb, rng=rng)
    xa += np.array([4.0, 0.0, 0.0])
    va += np.array([-0.3, 0.1, 0.0])
    xb += np.array([-4.0, 0.0, 0.0])
    vb += np.array([0.3, 0.1, 0.0])
    xyz = np.concatenate([xa, xb])
    v = np.concatenate([va, vb])
    return _pack(xyz[:, 0], xyz[:, 1], xyz[:, 2], m, v[:, 0], v[:, 1], v[:, 2])


def random_bodies(n: int, seed: int, spread: float = 1.0) -> tuple[np.ndarray, np.ndarray]:
    """Generic test bodies: positions in [-spread, spread]^3, masses in [0.5, 1.5]/max(n,1),
    velocities in [-1, 1]^3."""
    rng = _rng(seed)
    xyz = spread * (2.0 * rng.random((n, 3)) - 1.0)
    m = (0.5 + rng.random(n)) / max(n, 1)
    v = 2.0 * rng.random((n, 3)) - 1.0
    return _pack(xyz[:, 0], xyz[:, 1], xyz[:, 2], m, v[:, 0], v[:, 1], v[:, 2])


def dyadic_grid_bodies(n: int, seed: int, bits: int = 10) -> tuple[np.ndarray, np.ndarray]:
    """Positions on multiples of 2^-bits inside [-1/2, 1/2), masses multiples of 2^-12.

    Differences of such coordinates are exact in float32, and so are the same
    differences after a shift by any multiple of 2^-bits that keeps |x| < 1.
    """
    rng = _rng(seed)
    k = rng.integers(-(1 << (bits - 1)), 1 << (bits - 1), size=(n, 3))
    xyz = k.astype(np.float64) * 2.0 ** -bits
    m = rng.integers(1 << 11, 3 << 11, size=n).astype(np.float64) * 2.0 ** -12
    z = np.zeros(n)
    return _pack(xyz[:, 0], xyz[:, 1], xyz[:, 2], m, z, z, z)


def _f32(x: float) -> np.float32:
    return np.float32(x)


# The five workloads. "eps" values are squared in fp64 before the single
# rounding to float32; "eps^2" values are rounded directly.
CONFIGS = {
    "disk4096": dict(n=4096, desc="N=4096 planar disk, m=1, eps^2=1e-6; one accel + one Euler step dt=1e-3"),
    "plummer65536": dict(n=65536, desc="N=65536 Plummer sphere, m=1/N, eps=0.01; accel + potential"),
    "cube2048_steps": dict(n=2048, desc="N=2048 uniform cube, m in [0.5,1.5]/N, eps^2=1e-4; 1000 Euler steps dt=1e-4"),
    "cube1m": dict(n=1_048_576, desc="N=1,048,576 uniform cube, m in [0.5,1.5]/N, v=0, eps^2=1e-4; accel + potential"),
    "two_plummer300007": dict(n=300_007, desc="N=300,007 two Plummer spheres, log-normal masses, eps=0.02; 10 Euler steps dt=1e-3"),
}


def make(name: str, n: int | None = None) -> Workload:
    """Build one of the five named workloads.

    ``n`` overrides the body count for the shape-preserving workloads (disk,
    cube, Plummer); the two-sphere workload splits an override as
    (n // 2, n - n // 2).
    """
    if name == "disk4096":
        N = 4096 if n is None else n
        pos, vel = uniform_disk(N)
        return Workload(name, pos, vel, _f32(1e-6), _f32(1e-3), 1, False, {"N": N})
    if name == "plummer65536":
        N = 65536 if n is None else n
        pos, vel = plummer_bodies(N)
        return Workload(name, pos, vel, _f32(0.01 * 0.01), None, 0, True, {"N": N, "eps": 0.01})
    if name == "cube2048_steps":
        N = 2048 if n is None else n
        pos, vel = uniform_cube(N)
        return Workload(name, pos, vel, _f32(1e-4), _f32(1e-4), 1000, False, {"N": N})
    if name == "cube1m":
        N = 1_048_576 if n is None else n
        pos, vel = uniform_cube(N)
        return Workload(name, pos, vel, _f32(1e-4), None, 0, True, {"N": N})
    if name == "two_plummer300007":
        if n is None:
            na, nb = 150_003, 150_004
        else:
            na, nb = n // 2, n - n // 2
        pos, vel = two_plummer(na, nb)
        return Workload(name, pos, vel, _f32(0.02 * 0.02), _f32(1e-3), 10, False,
                        {"N": na + nb, "n_a": na, "n_b": nb, "eps": 0.02})
    raise KeyError(name)
