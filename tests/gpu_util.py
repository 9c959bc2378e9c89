"""Helpers for the GPU parity tests: run the HIP path through the C ABI and
compare with the fp64 oracle under the per-body bounds.

Bounds (per body i; B_i and P_i are the oracle's error scales):
  acceleration: ||a_gpu - a_ref||_2 <= 1e-5 * B_i,  B_i = sum_j m_j |r_ij| / (r_ij^2 + eps2)^(3/2)
  potential:    |p_gpu - p_ref|     <= 1e-5 * P_i,  P_i = sum_j m_j / (r_ij^2 + eps2)^(1/2)
  one Euler step, per component (u = 2^-23):
    |x_gpu - x_ref| <= u (|x| + |dt v|)
    |v_gpu - v_ref| <= |dt| 1e-5 B_i + u (|v| + |dt a_ref|)
"""

from __future__ import annotations

import numpy as np

TOL = 1e-5
U23 = 2.0 ** -23


def dev():
    import torch

    return torch.device("cuda:0")


def to_dev(a: np.ndarray):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def gpu_accel(pos_h: np.ndarray, eps2, pot=True, plan=None):
    """(acc float32 (N,4), pot float32 (N,) or None) from the HIP path."""
    import torch

    import direct_all_pairs_amd as nb

    pos = to_dev(pos_h)
    acc, p = nb.accel(pos, float(eps2), pot=pot, plan=plan)
    torch.cuda.synchronize()
    return acc.cpu().numpy(), (p.cpu().numpy() if p is not None else None)


def gpu_step(pos_h, vel_h, dt, eps2, nsteps, plan=None):
    import torch

    import direct_all_pairs_amd as nb

    pos = to_dev(pos_h)
    vel = to_dev(vel_h)
    nb.step(pos, vel, float(dt), float(eps2), nsteps, plan=plan)
    torch.cuda.synchronize()
    return pos.cpu().numpy(), vel.cpu().numpy()


def _ratio(err, scale):
    """err / scale, where a zero scale allows only an exact zero error."""
    out = np.where(err == 0, 0.0, np.inf)
    np.divide(err, scale, out=out, where=scale > 0)
    return out


def accel_errors(acc, pot, ref, idx=None):
    """Per-body normalised errors (err_a / B, err_p / P) for rows idx of the GPU output."""
    a = acc if idx is None else acc[idx]
    e_a = _ratio(np.linalg.norm(a[:, :3].astype(np.float64) - ref["acc"], axis=1), ref["bound_a"])
    e_p = None
    if pot is not None:
        p = pot if idx is None else pot[idx]
        e_p = _ratio(np.abs(p.astype(np.float64) - ref["pot"]), ref["bound_p"])
    return e_a, e_p


def assert_accel_parity(acc, pot, ref, idx=None, what=""):
    e_a, e_p = accel_errors(acc, pot, ref, idx)
    assert np.all(np.isfinite(e_a)), f"{what}: non-finite acceleration"
    worst = int(np.argmax(e_a))
    assert e_a.max() <= TOL, f"{what}: accel err/B = {e_a.max():.3e} at row {worst}"
    a = acc if idx is None else acc[idx]
    assert np.all(a[:, 3] == 0.0), f"{what}: acc.w not zero"
    if e_p is not None:
        assert e_p.max() <= TOL, f"{what}: pot err/P = {e_p.max():.3e}"
    return float(e_a.max()), (float(e_p.max()) if e_p is not None else None)


def assert_step_parity(pos0, vel0, pos1, vel1, dt, ref, idx=None, what=""):
    """One Euler step from (pos0, vel0) (float32, the GPU's pre-step state) to (pos1, vel1).

    ref is the oracle's accel at x^n for rows idx (all rows if None).
    """
    sl = slice(None) if idx is None else idx
    x0 = pos0[sl, :3].astype(np.float64)
    v0 = vel0[sl, :3].astype(np.float64)
    x1 = pos1[sl, :3].astype(np.float64)
    v1 = vel1[sl, :3].astype(np.float64)
    dt = float(np.float32(dt))
    x_ref = x0 + dt * v0
    v_ref = v0 + dt * ref["acc"]
    bx = U23 * (np.abs(x0) + np.abs(dt * v0))
    bv = abs(dt) * TOL * ref["bound_a"][:, None] + U23 * (np.abs(v0) + np.abs(dt * ref["acc"]))
    ex = np.abs(x1 - x_ref)
    ev = np.abs(v1 - v_ref)
    assert np.all(ex <= bx), f"{what}: position step error {np.max(ex - bx):.3e} over bound"
    assert np.all(ev <= bv), f"{what}: velocity step error {np.max(ev - bv):.3e} over bound"
    assert np.array_equal(pos1[sl, 3], pos0[sl, 3]), f"{what}: mass changed"
    assert np.array_equal(vel1[sl, 3], vel0[sl, 3]), f"{what}: vel.w changed"
