"""Pins for the fp64 oracle: checks against facts the pages and the mathematics fix.

Each ``pin_*`` takes a loaded oracle (``oracle.Oracle``) and raises
AssertionError when the oracle disagrees with a closed form, an invariant, a
special case or an independent 50-digit brute force. test_oracle.py runs them
on the real oracle; test_oracle_mutations.py runs them on copies of oracle.c
with planted mistakes and requires each mistake to trip at least one pin.

Sources for what is pinned:
- Degawa, "N 体問題", slide 4 (acceleration sum), slide 12 (softening replaces
  the j != i branch; the self term has a zero numerator), slides 5-6 and 15
  (explicit Euler, position first with the old velocity).
- Nakasato, "スライド 1", No.4 (acceleration and potential; minus sign of p).
- GPU Gems 3 ch. 31 study page, section 1 (r_ij = x_j - x_i).
"""

from __future__ import annotations

import math
from decimal import Decimal, getcontext

import numpy as np


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    err = np.abs(a - b)
    if not np.all(np.isfinite(a)) or np.any(err > tol):
        raise AssertionError(f"{what}: max err {np.nanmax(err) if err.size else 0:.3e} > tol\n"
                             f"got {a}\nwant {b}")


def _bodies(xyz, m):
    xyz = np.asarray(xyz, dtype=np.float64).reshape(-1, 3)
    p = np.zeros((xyz.shape[0], 4))
    p[:, :3] = xyz
    p[:, 3] = m
    return p


# ---------------------------------------------------------------- special cases

def pin_single_body(orc):
    """N = 1: the only term is the self term: a = 0 exactly and p = -m/eps."""
    for m, e2, x in [(1.0, 1e-6, (0.3, -0.2, 0.9)), (2.5, 0.25, (0, 0, 0)), (1e-3, 4e-4, (7, 1, 2))]:
        r = orc.accel_exact(_bodies([x], m), e2)
        if not np.all(r["acc"] == 0.0):
            raise AssertionError(f"N=1 acceleration not zero: {r['acc']}")
        _close(r["pot"], [-m / math.sqrt(e2)], 0.0, "N=1 potential")
        _close(r["bound_p"], [m / math.sqrt(e2)], 0.0, "N=1 P scale")
        _close(r["bound_a"], [0.0], 0.0, "N=1 B scale")


def pin_two_body_345(orc):
    """Hand-derived worked example: m0 = 1 at the origin, m1 = 2 at (3, 4, 0), eps2 = 11.

    |r|^2 + eps2 = 25 + 11 = 36, so (.)^(3/2) = 216 and (.)^(1/2) = 6:
      a0 = 2 (3, 4, 0)/216 = (1/36, 1/27, 0)      a1 = 1 (-3, -4, 0)/216 = (-1/72, -1/54, 0)
      p0 = -2/6 - 1/sqrt(11)                      p1 = -1/6 - 2/sqrt(11)
      B0 = 2*5/216, B1 = 5/216;  P0 = 2/6 + 1/sqrt(11), P1 = 1/6 + 2/sqrt(11)
    """
    pos = _bodies([[0, 0, 0], [3, 4, 0]], [1.0, 2.0])
    r = orc.accel_exact(pos, 11.0)
    tol = 4e-16
    _close(r["acc"], [[1 / 36, 1 / 27, 0], [-1 / 72, -1 / 54, 0]], tol, "3-4-5 accelerations")
    s11 = math.sqrt(11.0)
    _close(r["pot"], [-1 / 3 - 1 / s11, -1 / 6 - 2 / s11], 4 * tol, "3-4-5 potentials")
    _close(r["bound_a"], [10 / 216, 5 / 216], tol, "3-4-5 B scales")
    _close(r["bound_p"], [1 / 3 + 1 / s11, 1 / 6 + 2 / s11], 4 * tol, "3-4-5 P scales")


def pin_two_body_random(orc):
    """Random pairs: each body is pulled toward the other with m_other |r| / (r^2+eps2)^(3/2)."""
    rng = np.random.Generator(np.random.PCG64(2))
    for _ in range(20):
        x = rng.normal(size=(2, 3))
        m = rng.uniform(0.1, 3.0, size=2)
        e2 = 10.0 ** rng.uniform(-6, 0)
        r = orc.accel_exact(_bodies(x, m), e2)
        d = x[1] - x[0]
        dist = float(np.sqrt(d @ d))
        mag0 = m[1] * dist / (dist * dist + e2) ** 1.5
        mag1 = m[0] * dist / (dist * dist + e2) ** 1.5
        unit = d / dist
        _close(r["acc"][0], mag0 * unit, 1e-14 * mag0, "two-body a0 (toward body 1)")
        _close(r["acc"][1], -mag1 * unit, 1e-14 * mag1, "two-body a1 (toward body 0)")
        p0 = -m[1] / math.hypot(dist, math.sqrt(e2)) - m[0] / math.sqrt(e2)
        _close(r["pot"][0], p0, 1e-14 * abs(p0), "two-body p0")


# ------------------------------------------------------------ brute force

def _decimal_sums(pos: np.ndarray, eps2: float):
    getcontext().prec = 50
    n = pos.shape[0]
    P = [[Decimal(float(v)) for v in row] for row in pos]
    e2 = Decimal(float(eps2))
    out = []
    for i in range(n):
        ax = ay = az = p = B = Pp = Decimal(0)
        for j in range(n):
            dx = P[j][0] - P[i][0]
            dy = P[j][1] - P[i][1]
            dz = P[j][2] - P[i][2]
            r2 = dx * dx + dy * dy + dz * dz
            q = r2 + e2
            sq = q.sqrt()
            w = P[j][3] / (q * sq)
            ax += w * dx
            ay += w * dy
            az += w * dz
            p -= P[j][3] / sq
            B += w * r2.sqrt()
            Pp += P[j][3] / sq
        out.append((float(ax), float(ay), float(az), float(p), float(B), float(Pp)))
    return np.array(out)


def pin_decimal_bruteforce(orc):
    """Random small systems against 50-digit decimal arithmetic of the same sum."""
    rng = np.random.Generator(np.random.PCG64(3))
    for n in (3, 5, 8, 13, 16):
        x = rng.uniform(-1, 1, size=(n, 3))
        m = rng.uniform(0.5, 1.5, size=n)
        e2 = 10.0 ** rng.uniform(-5, -1)
        pos = _bodies(x, m)
        r = orc.accel_exact(pos, e2)
        d = _decimal_sums(pos, e2)
        B = d[:, 4]
        Pp = d[:, 5]
        err_a = np.linalg.norm(r["acc"] - d[:, :3], axis=1)
        if np.any(err_a > 1e-13 * B):
            raise AssertionError(f"decimal brute force, accel, N={n}: {err_a / B}")
        _close(r["pot"], d[:, 3], 1e-13 * Pp, f"decimal brute force, potential, N={n}")
        _close(r["bound_a"], B, 1e-13 * B, f"decimal brute force, B, N={n}")
        _close(r["bound_p"], Pp, 1e-13 * Pp, f"decimal brute force, P, N={n}")


# ---------------------------------------------------------------- symmetry

def pin_symmetric_centre(orc):
    """Equal masses on the cube's 8 vertices or the octahedron's 6 vertices plus a central body.

    By symmetry the central body feels no force, and every vertex is pulled
    straight toward the centre.
    """
    cube = np.array([[sx, sy, sz] for sx in (-1, 1) for sy in (-1, 1) for sz in (-1, 1)], float)
    octa = np.array([[1, 0, 0], [-1, 0, 0], [0, 1, 0], [0, -1, 0], [0, 0, 1], [0, 0, -1]], float)
    for verts, scale, e2 in [(cube, 0.5, 1e-2), (octa, 1.7, 1e-4), (cube, 3.0, 1.0)]:
        xyz = np.concatenate([np.zeros((1, 3)), scale * verts])
        m = np.concatenate([[2.0], np.full(len(verts), 0.75)])
        r = orc.accel_exact(_bodies(xyz, m), e2)
        B = r["bound_a"]
        if np.linalg.norm(r["acc"][0]) > 1e-15 * B[0]:
            raise AssertionError(f"force at the centre of a symmetric set: {r['acc'][0]}")
        for k in range(1, len(xyz)):
            a = r["acc"][k]
            x = xyz[k]
            if np.linalg.norm(np.cross(a, x)) > 1e-14 * B[k] * np.linalg.norm(x) or a @ x >= 0:
                raise AssertionError(f"vertex {k} not pulled toward the centre: a={a}, x={x}")
        # all vertices are equivalent: same |a| and same p
        mags = np.linalg.norm(r["acc"][1:], axis=1)
        _close(mags, np.full_like(mags, mags[0]), 1e-14 * mags[0], "vertex |a| equal")
        _close(r["pot"][1:], np.full(len(verts), r["pot"][1]), 1e-14 * abs(r["pot"][1]),
               "vertex p equal")


def pin_ring(orc):
    """n equal masses m on a circle of radius R (a regular polygon), plane z = 0.

    Body i at angle t_i; body j at t_i + 2 pi k/n. The chord has
    |r|^2 = 4 R^2 sin^2(pi k/n) and its component toward the centre is
    2 R sin^2(pi k/n); tangential parts cancel between k and n - k. So every
    body feels an inward pull of
        A = m sum_{k=1}^{n-1} 2 R sin^2(pi k/n) / (4 R^2 sin^2(pi k/n) + eps2)^(3/2)
    and has potential
        p = -m sum_{k=1}^{n-1} (4 R^2 sin^2(pi k/n) + eps2)^(-1/2) - m/sqrt(eps2).
    """
    for n, R, e2, m, t0 in [(3, 1.0, 1e-3, 1.0, 0.1), (4, 2.5, 0.3, 0.5, 0.0),
                            (7, 1.3, 1e-6, 2.0, 1.0), (12, 0.8, 1e-2, 1 / 12, 0.37)]:
        t = t0 + 2 * np.pi * np.arange(n) / n
        xyz = np.stack([R * np.cos(t), R * np.sin(t), np.zeros(n)], axis=1)
        r = orc.accel_exact(_bodies(xyz, m), e2)
        s2 = np.sin(np.pi * np.arange(1, n) / n) ** 2
        A = m * np.sum(2 * R * s2 / (4 * R * R * s2 + e2) ** 1.5)
        p = -m * np.sum(1 / np.sqrt(4 * R * R * s2 + e2)) - m / math.sqrt(e2)
        want = -A * xyz / R
        B = r["bound_a"]
        err = np.linalg.norm(r["acc"] - want, axis=1)
        if np.any(err > 1e-13 * B):
            raise AssertionError(f"ring n={n}: accel err/B {err / B}")
        _close(r["pot"], np.full(n, p), 1e-13 * abs(p), f"ring n={n} potential")
        if np.any(r["acc"][:, 2] != 0.0):
            raise AssertionError("ring: out-of-plane acceleration")


def pin_third_law(orc):
    """Newton's third law: pair forces cancel, so sum_i m_i a_i = 0 up to rounding."""
    rng = np.random.Generator(np.random.PCG64(4))
    for n, e2 in [(50, 1e-4), (200, 1e-2), (97, 1e-6)]:
        x = rng.uniform(-1, 1, size=(n, 3))
        m = rng.uniform(0.1, 2.0, size=n)
        r = orc.accel_exact(_bodies(x, m), e2)
        tot = np.linalg.norm((m[:, None] * r["acc"]).sum(axis=0))
        scale = float((m * r["bound_a"]).sum())
        if tot > 1e-12 * scale:
            raise AssertionError(f"third law: |sum m a| = {tot:.3e} vs scale {scale:.3e}")


# ---------------------------------------------------------------- exact scaling

def pin_mass_scaling(orc):
    """Doubling every mass doubles a, p, B and P exactly (power-of-two scaling)."""
    rng = np.random.Generator(np.random.PCG64(5))
    x = rng.uniform(-1, 1, size=(40, 3))
    m = rng.uniform(0.5, 1.5, size=40)
    r1 = orc.accel_exact(_bodies(x, m), 1e-3)
    r2 = orc.accel_exact(_bodies(x, 2 * m), 1e-3)
    for k in ("acc", "pot", "bound_a", "bound_p"):
        if not np.array_equal(r2[k], 2 * r1[k]):
            raise AssertionError(f"mass scaling not exact for {k}")


def pin_length_scaling(orc):
    """Positions x 2^k and eps2 x 4^k give a x 2^-2k and p x 2^-k exactly."""
    rng = np.random.Generator(np.random.PCG64(6))
    x = rng.uniform(-1, 1, size=(40, 3))
    m = rng.uniform(0.5, 1.5, size=40)
    r1 = orc.accel_exact(_bodies(x, m), 1e-3)
    for k in (-3, 2, 5):
        s = 2.0 ** k
        r2 = orc.accel_exact(_bodies(s * x, m), 1e-3 * s * s)
        if not np.array_equal(r2["acc"], r1["acc"] / (s * s)):
            raise AssertionError(f"length scaling 2^{k}: acceleration")
        if not np.array_equal(r2["pot"], r1["pot"] / s):
            raise AssertionError(f"length scaling 2^{k}: potential")


def pin_translation(orc):
    """On a dyadic grid differences are exact, so a shift changes nothing, bit for bit."""
    rng = np.random.Generator(np.random.PCG64(7))
    k = rng.integers(-512, 512, size=(60, 3))
    x = k * 2.0 ** -10
    m = rng.integers(2048, 6144, size=60) * 2.0 ** -12
    r1 = orc.accel_exact(_bodies(x, m), 2.0 ** -10)
    r2 = orc.accel_exact(_bodies(x + np.array([0.5, -0.25, 0.125]), m), 2.0 ** -10)
    for key in ("acc", "pot", "bound_a", "bound_p"):
        if not np.array_equal(r1[key], r2[key]):
            raise AssertionError(f"translation changed {key}")


# ---------------------------------------------------------------- Euler

def pin_euler_free_particle(orc):
    """A lone body feels no force: x advances by dt v per step, v stays put."""
    pos = np.array([[0.25, -1.5, 3.0, 2.0]])
    vel = np.array([[1.0, 0.5, -2.0, 0.0]])
    dt = 0.125
    p, v = orc.euler_exact(pos, vel, dt, 1e-4, 3)
    want = pos[0, :3].copy()
    for _ in range(3):
        want = want + dt * vel[0, :3]
    _close(p[0, :3], want, 0.0, "free particle position")
    _close(v[0], vel[0], 0.0, "free particle velocity")
    if p[0, 3] != 2.0:
        raise AssertionError("mass changed by the step")


def pin_euler_two_body(orc):
    """One step of the 3-4-5 system: x' = x + dt v (old v), v' = v + dt a(x) (old x)."""
    pos = _bodies([[0, 0, 0], [3, 4, 0]], [1.0, 2.0])
    vel = np.array([[0.5, 0.0, 0.25, 0.0], [0.0, -1.0, 0.0, 0.0]])
    dt = 0.0625
    p, v = orc.euler_exact(pos, vel, dt, 11.0, 1)
    a = np.array([[1 / 36, 1 / 27, 0], [-1 / 72, -1 / 54, 0]])
    _close(p[:, :3], pos[:, :3] + dt * vel[:, :3], 0.0, "Euler position uses the old velocity")
    _close(v[:, :3], vel[:, :3] + dt * a, 1e-17, "Euler velocity uses a(x^n)")
    _close(p[:, 3], pos[:, 3], 0.0, "mass preserved")


def pin_energy_two_body(orc):
    """E = sum m v^2/2 - m0 m1/sqrt(r^2+eps2) for the 3-4-5 system (pair counted once)."""
    pos = _bodies([[0, 0, 0], [3, 4, 0]], [1.0, 2.0])
    vel = np.array([[0.5, 0.0, 0.25, 0.0], [0.0, -1.0, 0.0, 0.0]])
    E, K, W = orc.energy_exact(pos, vel, 11.0)
    k_want = 0.5 * 1.0 * (0.25 + 0.0625) + 0.5 * 2.0 * 1.0
    _close([K, W, E], [k_want, -2.0 / 6.0, k_want - 2.0 / 6.0], 1e-16, "two-body energy")


# ---------------------------------------------------------------- diagnostics
# Not on the pages: kinetic energy, the pair energy built from the pages' potential
# (Nakasato No.4), momentum and angular momentum are the textbook definitions.

def pin_diagnostics_two_body(orc):
    """The 3-4-5 system: every diagnostic by hand. K = 1/2 (0.3125) + 1/2 2 (1) = 1.15625;
    W = -m0 m1/6 = -1/3 (pair once); P = (0.5, -2, 0.25); L = m1 (3, 4, 0) x (0, -1, 0) =
    2 (0, 0, -3) = (0, 0, -6) plus m0 0 x v0 = 0; M = 3; centre of mass (2, 8/3, 0)."""
    pos = _bodies([[0, 0, 0], [3, 4, 0]], [1.0, 2.0])
    vel = np.array([[0.5, 0.0, 0.25, 0.0], [0.0, -1.0, 0.0, 0.0]])
    for pot in (None, [-2.0 / 6.0 - 1.0 / math.sqrt(11.0), -1.0 / 6.0 - 2.0 / math.sqrt(11.0)]):
        d = orc.diagnostics_exact(pos, vel, 11.0, pot=pot)
        _close([d["kinetic"], d["potential"], d["total"]], [1.15625, -1 / 3, 1.15625 - 1 / 3],
               1e-15, f"two-body energies (pot given: {pot is not None})")
        _close(d["momentum"], [0.5, -2.0, 0.25], 0.0, "two-body momentum")
        _close(d["angular_momentum"], [0.0, 0.0, -6.0], 0.0, "two-body angular momentum")
        _close([d["mass"]], [3.0], 0.0, "two-body mass")
        _close(d["centre_of_mass"], [2.0, 8.0 / 3.0, 0.0], 1e-15, "two-body centre of mass")


def pin_diagnostics_rotating_ring(orc):
    """A regular n-gon of masses m at radius R, each moving tangentially at speed u:
    K = n m u^2/2, W = -(n m^2/2) sum_k (4 R^2 sin^2(pi k/n) + eps2)^(-1/2), P = 0,
    L = (0, 0, n m R u), centre of mass at the origin."""
    for n, R, e2, m, u, t0 in [(5, 1.5, 1e-3, 0.2, 0.7, 0.3), (8, 0.5, 0.04, 1.0, -1.25, 0.0)]:
        t = t0 + 2 * np.pi * np.arange(n) / n
        xyz = np.stack([R * np.cos(t), R * np.sin(t), np.zeros(n)], axis=1)
        vel = np.zeros((n, 4))
        vel[:, 0] = -u * np.sin(t)
        vel[:, 1] = u * np.cos(t)
        d = orc.diagnostics_exact(_bodies(xyz, m), vel, e2)
        s2 = np.sin(np.pi * np.arange(1, n) / n) ** 2
        w = -(n * m * m / 2) * np.sum(1 / np.sqrt(4 * R * R * s2 + e2))
        _close([d["kinetic"], d["potential"]], [n * m * u * u / 2, w], 1e-13 * abs(w),
               f"ring n={n} energies")
        _close(d["momentum"], [0, 0, 0], 1e-14, f"ring n={n} momentum")
        _close(d["angular_momentum"], [0, 0, n * m * R * u], 1e-14, f"ring n={n} L")
        _close(d["centre_of_mass"], [0, 0, 0], 1e-15, f"ring n={n} centre of mass")


def pin_diagnostics_pair_sum(orc):
    """W from the per-body potentials (self term removed analytically) equals the sum over
    distinct pairs (j != i skipped) of the energy routine, for random bodies."""
    rng = np.random.Generator(np.random.PCG64(8))
    x = rng.uniform(-1, 1, size=(60, 3))
    m = rng.uniform(0.1, 2.0, size=60)
    v = np.zeros((60, 4))
    v[:, :3] = rng.uniform(-1, 1, size=(60, 3))
    d = orc.diagnostics_exact(_bodies(x, m), v, 1e-3)
    E, K, W = orc.energy_exact(_bodies(x, m), v, 1e-3)
    _close([d["kinetic"], d["potential"]], [K, W], 1e-12 * abs(W), "pair-sum energy")


def pin_diagnostics_euler_momentum(orc):
    """One Euler step changes momentum by dt sum m a = 0 (third law): conserved to rounding;
    centre of mass moves by dt P / M exactly in exact arithmetic."""
    rng = np.random.Generator(np.random.PCG64(9))
    x = rng.uniform(-1, 1, size=(40, 3))
    m = rng.uniform(0.5, 1.5, size=40)
    v = np.zeros((40, 4))
    v[:, :3] = rng.uniform(-1, 1, size=(40, 3))
    pos = _bodies(x, m)
    dt = 1e-2
    d0 = orc.diagnostics_exact(pos, v, 1e-3)
    p1, v1 = orc.euler_exact(pos, v, dt, 1e-3, 1)
    d1 = orc.diagnostics_exact(p1, v1, 1e-3)
    scale = float(np.sum(m * np.linalg.norm(v[:, :3], axis=1))) + 1.0
    _close(d1["momentum"], d0["momentum"], 1e-13 * scale, "Euler step momentum")
    want = np.array(d0["centre_of_mass"]) + dt * np.array(d0["momentum"]) / d0["mass"]
    _close(d1["centre_of_mass"], want, 1e-14, "Euler step centre of mass")


# ---------------------------------------------------------------- near field
# The all-pairs sum restricted to listed cells (GPU Gems 3 ch. 31 study page, section 6:
# near-field leaf cells use all-pairs; Nakasato No.34: neighbour-particle algorithms).

def _csr(lists):
    off = np.zeros(len(lists) + 1, np.int32)
    off[1:] = np.cumsum([len(x) for x in lists])
    flat = np.array([c for x in lists for c in x], np.int32)
    return off, flat


def _random_cells(seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    sizes = [7, 0, 12, 1, 20, 9]  # an empty cell included
    n = sum(sizes)
    x = rng.uniform(-1, 1, size=(n, 3))
    m = rng.uniform(0.1, 2.0, size=n)
    start = np.zeros(len(sizes) + 1, np.int32)
    start[1:] = np.cumsum(sizes)
    return _bodies(x, m), start


def pin_p2p_full_lists_equal_direct_sum(orc):
    """Every cell listing every cell in ascending order sums every j in ascending order: the
    result equals the direct sum bit for bit."""
    pos, start = _random_cells(10)
    nc = len(start) - 1
    off, flat = _csr([list(range(nc))] * nc)
    r = orc.p2p_exact(pos, 1e-3, start, off, flat)
    d = orc.accel_exact(pos, 1e-3)
    for k in ("acc", "pot", "bound_a", "bound_p"):
        if not np.array_equal(r[k], d[k]):
            raise AssertionError(f"p2p with full lists differs from the direct sum in {k}")


def pin_p2p_self_lists_equal_subsystems(orc):
    """Each cell listing only itself gives the direct sum of that cell's bodies alone."""
    pos, start = _random_cells(11)
    nc = len(start) - 1
    off, flat = _csr([[c] for c in range(nc)])
    r = orc.p2p_exact(pos, 1e-3, start, off, flat)
    for c in range(nc):
        a, b = start[c], start[c + 1]
        if a == b:
            continue
        d = orc.accel_exact(pos[a:b], 1e-3)
        if not (np.array_equal(r["acc"][a:b], d["acc"]) and np.array_equal(r["pot"][a:b], d["pot"])):
            raise AssertionError(f"cell {c}: self list differs from its subsystem")


def pin_p2p_skips_bad_entries_and_empty_lists(orc):
    """Entries outside [0, ncell) add nothing; an empty list gives exact zeros."""
    pos, start = _random_cells(12)
    nc = len(start) - 1
    good = [[0, 2], [], [5, 4], [1], [3, 3], [2]]
    bad = [[-1, 0, 2, nc], [nc + 7], [5, -3, 4], [1, 99], [3, 3, -1], [2]]
    r1 = orc.p2p_exact(pos, 1e-3, start, *_csr(good))
    r2 = orc.p2p_exact(pos, 1e-3, start, *_csr(bad))
    for k in ("acc", "pot"):
        if not np.array_equal(r1[k], r2[k]):
            raise AssertionError(f"invalid list entries changed {k}")
    a, b = start[1], start[2]
    if a != b or not np.all(r1["acc"][start[1]:start[2]] == 0):
        raise AssertionError("empty cell / empty list not zero")
    # cell 1 is empty; cell 3 (one body) lists cell 1 only in a variant: exact zeros
    r3 = orc.p2p_exact(pos, 1e-3, start, *_csr([[0], [], [2], [1], [4], [5]]))
    i = start[3]
    if not (np.all(r3["acc"][i] == 0) and r3["pot"][i] == 0):
        raise AssertionError("a list of only an empty cell must give zeros")


def _grid_cells_f32(pos, lo, h, dims):
    """Cell coordinates decided in float32 as the GPU decides them: floor((x - lo) * (1/h))."""
    x = pos[:, :3].astype(np.float32)
    inv = np.float32(1.0) / np.float32(h)
    f = np.floor((x - np.asarray(lo, np.float32)) * inv)
    f = np.nan_to_num(f, nan=0.0)
    return np.clip(f, 0, np.asarray(dims) - 1).astype(np.int64)


def pin_near_grid_small_grids_equal_direct_sum(orc):
    """With at most 2 cells per axis every cell neighbours every other: the near field is the
    direct sum, bit for bit (both sum every j in ascending order)."""
    rng = np.random.Generator(np.random.PCG64(13))
    x = rng.uniform(-1, 1, size=(50, 3)).astype(np.float32).astype(np.float64)
    m = rng.uniform(0.1, 2.0, size=50)
    pos = _bodies(x, m)
    d = orc.accel_exact(pos, 1e-3)
    for dims, h in (((1, 1, 1), 4.0), ((2, 2, 1), 1.0), ((2, 2, 2), 1.25)):
        r = orc.near_grid_exact(pos, 1e-3, (-1.0, -1.0, -1.0), h, dims)
        for k in ("acc", "pot", "bound_a", "bound_p"):
            if not np.array_equal(r[k], d[k]):
                raise AssertionError(f"near grid {dims}: differs from the direct sum in {k}")


def pin_near_grid_separated_clusters(orc):
    """Two clusters three cells apart do not see each other: each gets its own direct sum."""
    rng = np.random.Generator(np.random.PCG64(14))
    a = rng.uniform(0.0, 1.0, size=(20, 3))
    b = rng.uniform(0.0, 1.0, size=(15, 3)) + np.array([10.0, 0.0, 0.0])
    m = rng.uniform(0.5, 1.5, size=35)
    pos = _bodies(np.concatenate([a, b]), m)
    r = orc.near_grid_exact(pos, 1e-3, (0.0, 0.0, 0.0), 2.5, (5, 1, 1))
    da = orc.accel_exact(pos[:20], 1e-3)
    db = orc.accel_exact(pos[20:], 1e-3)
    if not (np.array_equal(r["acc"][:20], da["acc"]) and np.array_equal(r["acc"][20:], db["acc"])):
        raise AssertionError("separated clusters interact in the near field")
    if not (np.array_equal(r["pot"][:20], da["pot"]) and np.array_equal(r["pot"][20:], db["pot"])):
        raise AssertionError("separated clusters: potentials")


def pin_near_grid_equals_lists(orc):
    """The grid near field equals the list form built independently here (bodies sorted by
    cell, 27-neighbour lists): same terms, other order, so to 1e-13 of B and P."""
    rng = np.random.Generator(np.random.PCG64(15))
    n = 300
    x = rng.uniform(-1, 1, size=(n, 3)).astype(np.float32).astype(np.float64)
    m = rng.uniform(0.1, 2.0, size=n)
    pos = _bodies(x, m)
    lo, h, dims = (-1.0, -1.0, -1.0), 0.4, (5, 5, 5)
    k = _grid_cells_f32(pos, lo, h, dims)
    cid = (k[:, 2] * dims[1] + k[:, 1]) * dims[0] + k[:, 0]
    order = np.argsort(cid, kind="stable")
    nc = dims[0] * dims[1] * dims[2]
    start = np.searchsorted(cid[order], np.arange(nc + 1)).astype(np.int32)
    lists = []
    for c in range(nc):
        cx, cy, cz = c % dims[0], (c // dims[0]) % dims[1], c // (dims[0] * dims[1])
        nb = []
        for dz in (-1, 0, 1):
            for dy in (-1, 0, 1):
                for dx in (-1, 0, 1):
                    X, Y, Z = cx + dx, cy + dy, cz + dz
                    if 0 <= X < dims[0] and 0 <= Y < dims[1] and 0 <= Z < dims[2]:
                        nb.append((Z * dims[1] + Y) * dims[0] + X)
        lists.append(nb)
    r_list = orc.p2p_exact(pos[order], 1e-3, start, *_csr(lists))
    r_grid = orc.near_grid_exact(pos, 1e-3, lo, h, dims)
    back = np.empty(n, np.int64)
    back[order] = np.arange(n)
    err = np.linalg.norm(r_list["acc"][back] - r_grid["acc"], axis=1)
    if np.any(err > 1e-13 * r_grid["bound_a"] + 1e-300):
        raise AssertionError(f"grid vs lists: max err {np.max(err):.3e}")
    _close(r_list["pot"][back], r_grid["pot"], 1e-13 * np.max(r_grid["bound_p"]), "grid vs lists p")


# ------------------------------------------------------------------ shards of a split evaluation

def _band_items(nb):
    """The band-pair work items of a split evaluation, enumerated as the library describes
    them: for every band A the diagonal (A, A) and the pairs (A, (A + d) mod nb) for
    d = 1 .. nb // 2, where for even nb the opposite pair d = nb / 2 is taken only from the
    lower band. Yields (owner band, frozenset of the two bands)."""
    for a in range(nb):
        yield a, frozenset((a,))
        for d in range(1, nb // 2 + 1):
            if 2 * d == nb and a >= nb // 2:
                continue
            yield a, frozenset((a, (a + d) % nb))


def pin_shard_items_cover_each_pair_once(orc):
    """One body per band, masses 2^-j, all at the origin, eps2 = 1: a shard's potential at
    body i is minus the sum of 2^-j over the j it pairs i with, so its bits name the set
    exactly. With one shard per band that set must be the partners of i in the items the
    band owns, by an enumeration written independently of the oracle; and the items must
    cover every unordered pair once (odd and even band counts)."""
    for n in (11, 12):
        items = list(_band_items(n))
        pairs = [p for _, p in items]
        want = {frozenset((i, j)) for i in range(n) for j in range(n)}
        if len(pairs) != len(set(pairs)) or set(pairs) != want:
            raise AssertionError(f"n={n}: items do not cover each unordered band pair once")
        pos = np.zeros((n, 4))
        pos[:, 3] = [2.0 ** -j for j in range(n)]
        for s in range(n):
            r = orc.shard_exact(pos, 1.0, 1, s, n)
            if np.any(r["acc"] != 0.0):
                raise AssertionError("coincident bodies must give zero acceleration")
            for i in range(n):
                # partner of i in each item of band s that holds i (itself for the diagonal)
                expect = sorted(i if len(p) == 1 else min(p - {i})
                                for a, p in items if a == s and i in p)
                bits = int(round(-r["pot"][i] * 2.0 ** n))  # sum of 2^(n - j) over the j
                got = [j for j in range(n) if bits >> (n - j) & 1]
                if got != expect:
                    raise AssertionError(f"n={n} shard {s} body {i}: pairs {got} != {expect}")


def pin_shard_single_equals_direct_sum(orc):
    """A single shard owns every band: the result is the direct sum bit for bit."""
    pos, _ = _random_cells(13)
    for band in (1, 5, 64):
        r = orc.shard_exact(pos, 1e-3, band, 0, 1)
        d = orc.accel_exact(pos, 1e-3)
        for k in ("acc", "pot", "bound_a", "bound_p"):
            if not np.array_equal(r[k], d[k]):
                raise AssertionError(f"band {band}: one shard differs from the direct sum in {k}")


def pin_shards_add_up_to_direct_sum(orc):
    """Over all shards the parts add up to the direct sum (fp64 rounding only), for even and
    odd band counts and shard counts that do and do not divide them; the error scales add up
    the same way."""
    rng = np.random.default_rng(77)
    for n, band, shards in ((700, 64, (2, 3, 11)), (512, 64, (2, 3, 8)), (97, 8, (5, 13))):
        pos = _bodies(rng.uniform(-1, 1, (n, 3)), rng.uniform(0.5, 1.5, n) / n)
        d = orc.accel_exact(pos, 1e-3)
        for S in shards:
            parts = [orc.shard_exact(pos, 1e-3, band, s, S) for s in range(S)]
            for k in ("acc", "pot", "bound_a", "bound_p"):
                tot = sum(p[k] for p in parts)
                scale = d["bound_a"] if k == "acc" else d["bound_p"]
                if k == "acc":
                    err = np.linalg.norm(tot - d[k], axis=1)
                else:
                    err = np.abs(tot - d[k])
                if np.any(err > 1e-13 * scale):
                    raise AssertionError(f"n={n} S={S}: shards do not add up in {k}")


# ------------------------------------------------------------------ near field on octree leaves

def pin_near_tree_one_leaf_equals_direct_sum(orc):
    """With leaf_size >= N the root is the only leaf: the tree near field is the whole direct
    sum, bit for bit (same terms, same order)."""
    rng = np.random.Generator(np.random.PCG64(21))
    for n in (1, 2, 37, 400):
        x = rng.uniform(-1, 1, size=(n, 3)).astype(np.float32).astype(np.float64)
        pos = _bodies(x, rng.uniform(0.1, 2.0, size=n))
        full = orc.accel_exact(pos, 1e-3)
        for leaf in (n, n + 5):
            r = orc.near_tree_exact(pos, 1e-3, leaf)
            for k in ("acc", "pot", "bound_a", "bound_p"):
                if not np.array_equal(r[k], full[k]):
                    raise AssertionError(f"one leaf (N={n}, leaf_size={leaf}): {k} differs")


def _lattice(cells, k, seed, zcells=None):
    """k bodies per cell of a lattice of `cells` cubic cells per axis on [0, 1]^3 (zcells along
    z: a box of height zcells / cells), placed inside their cells away from the faces, plus a
    body at (0, 0, 0) and one at x = y = 1 inside the top layer of cells, so the tree's root
    cube is [0, 1]^3 and both corner bodies fall in lattice cells."""
    rng = np.random.Generator(np.random.PCG64(seed))
    zc = cells if zcells is None else zcells
    pts = []
    for c in range(cells):
        for b in range(cells):
            for a in range(zc):
                for _ in range(k):
                    u = rng.uniform(0.15, 0.85, size=3)
                    pts.append(((c + u[0]) / cells, (b + u[1]) / cells, (a + u[2]) / cells))
    pts += [(0.0, 0.0, 0.0), (1.0, 1.0, 1.0 if zc == cells else (zc - 0.5) / cells)]
    x = np.asarray(pts, dtype=np.float32).astype(np.float64)
    return _bodies(x, rng.uniform(0.5, 1.5, size=x.shape[0]))


def pin_near_tree_full_octree_equals_grid(orc):
    """k = 2 bodies in every cell of an 8^3 lattice (the two corner cells hold 3): every cell
    holds at most leaf_size = 3 bodies and every cell of the 4^3 lattice above it 16 or more,
    so the leaves are exactly the 8^3 cells and the tree near field is the 27-cell grid near
    field of that lattice (independent definition), bit for bit; with leaf_size = 17 the
    leaves are the 4^3 cells. On a box half as high (8 x 8 x 4 cells) the cells stay cubic:
    the root cube's side is the largest extent."""
    for cells, zc, leaf, dims in ((8, 8, 3, (8, 8, 8)), (8, 8, 17, (4, 4, 4)),
                                  (8, 4, 3, (8, 8, 4))):
        pos = _lattice(cells, 2, 30 + leaf + zc, zcells=zc)
        r = orc.near_tree_exact(pos, 1e-3, leaf)
        g = orc.near_grid_exact(pos, 1e-3, (0.0, 0.0, 0.0), 1.0 / dims[0], dims)
        for k in ("acc", "pot", "bound_a", "bound_p"):
            if not np.array_equal(r[k], g[k]):
                raise AssertionError(f"full octree (leaf_size={leaf}, {dims}): {k} differs "
                                     "from the grid")


def pin_near_tree_deep_lattice(orc):
    """Leaves deep in the tree: two bodies in each cell of a 4^3 lattice of side 2^-13 at the
    origin (which fills the level-11 cell there), one more at (0, 0, 0) and one at (1, 1, 1),
    so the root cube is [0, 1]^3. With leaf_size = 3 the lattice cells are the leaves (level
    13; every coarser node around them holds 16 or more), so a lattice body's near field is
    the grid near field of the lattice; the body at (1, 1, 1) is alone in its octant and
    touches no other leaf, leaving only its self term."""
    rng = np.random.Generator(np.random.PCG64(45))
    h = 2.0 ** -13
    c = np.stack(np.meshgrid(*[np.arange(4)] * 3, indexing="ij"), -1).reshape(-1, 3)
    c = np.repeat(c, 2, axis=0)
    x = (c + rng.uniform(0.15, 0.85, size=c.shape)) * h
    x = np.concatenate([x, [[0.0, 0.0, 0.0], [1.0, 1.0, 1.0]]]).astype(np.float32)
    pos = _bodies(x.astype(np.float64), rng.uniform(0.5, 1.5, size=x.shape[0]))
    e2 = 1e-9
    r = orc.near_tree_exact(pos, e2, 3)
    lat = pos[:-1]
    g = orc.near_grid_exact(lat, e2, (0.0, 0.0, 0.0), h, (4, 4, 4))
    for k in ("acc", "pot", "bound_a", "bound_p"):
        want = g[k]
        got = r[k][:-1]
        if not np.array_equal(got, want):
            raise AssertionError(f"deep lattice: {k} differs from the grid near field")
    m = pos[-1, 3]
    if not (np.all(r["acc"][-1] == 0.0) and r["pot"][-1] == -m / math.sqrt(e2)):
        raise AssertionError("deep lattice: the lone body's near field is not its self term")


def pin_near_tree_mixed_levels(orc):
    """Leaves at two levels, neighbour sets derived by hand. The octant [0, 1/2]^3 holds two
    bodies in each of its eight level-2 cells (16 > leaf_size = 2: it splits; its cells are
    leaves); each of the other seven octants holds one body (a level-1 leaf). All eight
    octants meet at the centre, so every octant touches every other; a level-2 cell
    (a, b, c), a, b, c in {0, 1}, touches the octant (o_x, o_y, o_z) iff a = 1 wherever
    o_x = 1, and likewise for b and c; the eight level-2 cells all meet at (1/4, 1/4, 1/4).
    The expected sums come from explicit lists (another summation order: to 1e-13)."""
    rng = np.random.Generator(np.random.PCG64(41))
    pts, cell_of = [], []
    for a in (0, 1):
        for b in (0, 1):
            for c in (0, 1):
                for t in range(2):
                    if (a, b, c, t) == (0, 0, 0, 0):
                        pts.append((0.0, 0.0, 0.0))  # the root's lower corner
                    else:
                        u = rng.uniform(0.15, 0.85, size=3)
                        pts.append(((a + u[0]) / 4, (b + u[1]) / 4, (c + u[2]) / 4))
                    cell_of.append(("d", a, b, c))
    octants = [(ox, oy, oz) for ox in (0, 1) for oy in (0, 1) for oz in (0, 1)
               if (ox, oy, oz) != (0, 0, 0)]
    for o in octants:
        if o == (1, 1, 1):
            pts.append((1.0, 1.0, 1.0))  # the root's upper corner
        else:
            u = rng.uniform(0.1, 0.9, size=3)
            pts.append(tuple((o[d] + u[d]) / 2 for d in range(3)))
        cell_of.append(("s",) + o)
    x = np.asarray(pts, dtype=np.float32).astype(np.float64)
    pos = _bodies(x, rng.uniform(0.5, 1.5, size=x.shape[0]))
    groups = sorted(set(cell_of))
    members = {g: [i for i, c in enumerate(cell_of) if c == g] for g in groups}

    def touches(g, h):
        if g[0] == h[0]:
            return True  # dense cells meet at (1/4, 1/4, 1/4); octants at the centre
        dense, sparse = (g, h) if g[0] == "d" else (h, g)
        return all(dense[1 + d] == 1 for d in range(3) if sparse[1 + d] == 1)

    order = [i for g in groups for i in members[g]]
    start = np.cumsum([0] + [len(members[g]) for g in groups]).astype(np.int32)
    lists = [[gi2 for gi2, h in enumerate(groups) if touches(g, h)] for g in groups]
    r_list = orc.p2p_exact(pos[order], 1e-3, start, *_csr(lists))
    r_tree = orc.near_tree_exact(pos, 1e-3, 2)
    back = np.empty(len(order), np.int64)
    back[order] = np.arange(len(order))
    err = np.linalg.norm(r_list["acc"][back] - r_tree["acc"], axis=1)
    if np.any(err > 1e-13 * r_tree["bound_a"] + 1e-300):
        raise AssertionError(f"mixed-level tree vs hand lists: max err {np.max(err):.3e}")
    _close(r_list["pot"][back], r_tree["pot"], 1e-13 * np.max(r_tree["bound_p"]),
           "mixed-level tree vs hand lists p")


def pin_near_tree_third_law(orc):
    """Leaf neighbourhood is symmetric (two leaves are near or not, whichever is the
    target), so the near-field forces cancel in pairs: sum_i m_i a_i = 0 to 1e-12 of
    sum_i m_i B_i, on clustered bodies whose leaves sit at many levels."""
    rng = np.random.Generator(np.random.PCG64(51))
    core = rng.normal(0.0, 0.05, size=(300, 3))
    halo = rng.uniform(-1.0, 1.0, size=(200, 3))
    x = np.concatenate([core, halo]).astype(np.float32).astype(np.float64)
    m = rng.uniform(0.5, 1.5, size=x.shape[0])
    pos = _bodies(x, m)
    for leaf in (1, 4, 16):
        r = orc.near_tree_exact(pos, 1e-4, leaf)
        tot = np.sum(m[:, None] * r["acc"], axis=0)
        scale = np.sum(m * r["bound_a"])
        if np.linalg.norm(tot) > 1e-12 * scale:
            raise AssertionError(f"tree third law (leaf_size={leaf}): |sum m a| = "
                                 f"{np.linalg.norm(tot):.3e} against {scale:.3e}")
        # a finer tree keeps fewer neighbours: the sum of the P scales cannot grow
        if leaf > 1:
            r1 = orc.near_tree_exact(pos, 1e-4, 1)
            if np.sum(r1["bound_p"]) > np.sum(r["bound_p"]) * (1 + 1e-12):
                raise AssertionError("tree: leaf_size 1 keeps more neighbours than "
                                     f"leaf_size {leaf}")


ALL_PINS = [
    pin_single_body,
    pin_two_body_345,
    pin_two_body_random,
    pin_decimal_bruteforce,
    pin_symmetric_centre,
    pin_ring,
    pin_third_law,
    pin_mass_scaling,
    pin_length_scaling,
    pin_translation,
    pin_euler_free_particle,
    pin_euler_two_body,
    pin_energy_two_body,
    pin_diagnostics_two_body,
    pin_diagnostics_rotating_ring,
    pin_diagnostics_pair_sum,
    pin_diagnostics_euler_momentum,
    pin_p2p_full_lists_equal_direct_sum,
    pin_p2p_self_lists_equal_subsystems,
    pin_p2p_skips_bad_entries_and_empty_lists,
    pin_near_grid_small_grids_equal_direct_sum,
    pin_near_grid_separated_clusters,
    pin_near_grid_equals_lists,
    pin_shard_items_cover_each_pair_once,
    pin_shard_single_equals_direct_sum,
    pin_shards_add_up_to_direct_sum,
    pin_near_tree_one_leaf_equals_direct_sum,
    pin_near_tree_full_octree_equals_grid,
    pin_near_tree_deep_lattice,
    pin_near_tree_mixed_levels,
    pin_near_tree_third_law,
]
