"""fp64 CPU oracle for direct all-pairs softened gravity (ctypes wrapper of oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests/, by ``__graft_entry__.smoke()``
and by the cpu_baseline leg of ``bench.py``. The product library never imports
or links it, and it shares no code with the HIP path.

Inputs are the float32 body records the GPU receives, widened exactly to
float64; eps2 and dt are taken as their float32 values, widened, unless the
``*_exact`` entry points are used. See oracle.c for the formulas, their
sources on the pages and the readings taken.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
SRC = _HERE / "oracle.c"
LIB = _HERE / "liboracle.so"

_c_double_p = ctypes.POINTER(ctypes.c_double)
_c_int64_p = ctypes.POINTER(ctypes.c_int64)

GCC_FLAGS = ["-O2", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off"]


def compile_oracle(src: Path, out: Path) -> Path:
    """gcc -O2 -fopenmp, no fast-math, no FMA contraction."""
    tmp = out.with_suffix(".so.tmp")
    subprocess.run(["gcc", *GCC_FLAGS, "-o", str(tmp), str(src), "-lm"], check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> Path:
    if force or not LIB.exists():
        compile_oracle(SRC, LIB)
    return LIB


def _ptr(a, ctype=_c_double_p):
    if a is None:
        return ctypes.cast(None, ctype)
    return a.ctypes.data_as(ctype)


def _bodies64(arr) -> np.ndarray:
    a = np.asarray(arr)
    if a.ndim != 2 or a.shape[1] != 4:
        raise ValueError("bodies must have shape (N, 4)")
    return np.ascontiguousarray(a, dtype=np.float64)


def as_f32(x) -> float:
    """A scalar parameter as the float32 value the GPU path receives, widened."""
    return float(np.float32(x))


class Oracle:
    """One loaded build of oracle.c (the tests also load deliberately broken copies)."""

    def __init__(self, libpath: Path | str):
        lib = ctypes.CDLL(str(libpath))
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_accel.argtypes = [_c_double_p, ctypes.c_int64, ctypes.c_double, _c_int64_p,
                                     ctypes.c_int64, _c_double_p, _c_double_p, _c_double_p,
                                     _c_double_p]
        lib.oracle_accel.restype = ctypes.c_int
        lib.oracle_euler.argtypes = [_c_double_p, _c_double_p, ctypes.c_int64, ctypes.c_double,
                                     ctypes.c_double, ctypes.c_int64]
        lib.oracle_euler.restype = ctypes.c_int
        lib.oracle_energy.argtypes = [_c_double_p, _c_double_p, ctypes.c_int64, ctypes.c_double,
                                      _c_double_p, _c_double_p]
        lib.oracle_energy.restype = ctypes.c_double
        lib.oracle_diagnostics.argtypes = [_c_double_p, _c_double_p, _c_double_p, ctypes.c_int64,
                                           ctypes.c_double, _c_double_p]
        lib.oracle_diagnostics.restype = ctypes.c_int
        _i32p = ctypes.POINTER(ctypes.c_int32)
        lib.oracle_p2p.argtypes = [_c_double_p, ctypes.c_int64, ctypes.c_double, _i32p,
                                   ctypes.c_int32, _i32p, _i32p, _c_double_p, _c_double_p,
                                   _c_double_p, _c_double_p]
        lib.oracle_p2p.restype = ctypes.c_int
        lib.oracle_near_grid.argtypes = [_c_double_p, ctypes.c_int64, ctypes.c_double,
                                         _c_double_p, ctypes.c_double, _i32p, _c_int64_p,
                                         ctypes.c_int64, _c_double_p, _c_double_p, _c_double_p,
                                         _c_double_p]
        lib.oracle_near_grid.restype = ctypes.c_int
        lib.oracle_shard.argtypes = [_c_double_p, ctypes.c_int64, ctypes.c_double, ctypes.c_int64,
                                     ctypes.c_int64, ctypes.c_int64, _c_int64_p, ctypes.c_int64,
                                     _c_double_p, _c_double_p, _c_double_p, _c_double_p]
        lib.oracle_shard.restype = ctypes.c_int
        lib.oracle_near_tree.argtypes = [_c_double_p, ctypes.c_int64, ctypes.c_double,
                                         ctypes.c_int64, _c_int64_p, ctypes.c_int64, _c_double_p,
                                         _c_double_p, _c_double_p, _c_double_p]
        lib.oracle_near_tree.restype = ctypes.c_int
        self._lib = lib

    def num_threads(self) -> int:
        return int(self._lib.oracle_num_threads())

    def accel_exact(self, pos, eps2: float, targets=None) -> dict:
        """Accelerations, potentials and error scales; float64 bodies and eps2 used as given.

        Returns float64 arrays acc (nt, 3), pot (nt,), bound_a (nt,), bound_p (nt,)
        for the listed target indices (default: every body, in order).
        """
        p = _bodies64(pos)
        n = p.shape[0]
        if targets is None:
            t, nt = None, n
        else:
            t = np.ascontiguousarray(targets, dtype=np.int64)
            nt = t.shape[0]
        acc = np.zeros((nt, 3))
        pot = np.zeros(nt)
        ba = np.zeros(nt)
        bp = np.zeros(nt)
        rc = self._lib.oracle_accel(_ptr(p), n, float(eps2), _ptr(t, _c_int64_p), nt, _ptr(acc),
                                    _ptr(pot), _ptr(ba), _ptr(bp))
        if rc != 0:
            raise ValueError("oracle_accel rejected its arguments")
        return {"acc": acc, "pot": pot, "bound_a": ba, "bound_p": bp}

    def accel(self, pos, eps2, targets=None) -> dict:
        """As accel_exact, with eps2 rounded to float32 first (the GPU path's value)."""
        return self.accel_exact(pos, as_f32(eps2), targets)

    def euler_exact(self, pos, vel, dt: float, eps2: float, nsteps: int = 1):
        """nsteps explicit Euler steps in float64; returns new (pos64, vel64) arrays."""
        p = _bodies64(pos).copy()
        v = _bodies64(vel).copy()
        if p.shape != v.shape:
            raise ValueError("pos and vel shapes differ")
        rc = self._lib.oracle_euler(_ptr(p), _ptr(v), p.shape[0], float(dt), float(eps2),
                                    int(nsteps))
        if rc != 0:
            raise ValueError("oracle_euler rejected its arguments")
        return p, v

    def euler(self, pos, vel, dt, eps2, nsteps: int = 1):
        """As euler_exact, with dt and eps2 rounded to float32 first."""
        return self.euler_exact(pos, vel, as_f32(dt), as_f32(eps2), nsteps)

    def energy_exact(self, pos, vel, eps2: float):
        """(E, K, W): total, kinetic and softened pair potential energy (pairs counted once)."""
        p = _bodies64(pos)
        v = _bodies64(vel)
        k = ctypes.c_double()
        w = ctypes.c_double()
        e = self._lib.oracle_energy(_ptr(p), _ptr(v), p.shape[0], float(eps2), ctypes.byref(k),
                                    ctypes.byref(w))
        return float(e), float(k.value), float(w.value)

    def energy(self, pos, vel, eps2):
        return self.energy_exact(pos, vel, as_f32(eps2))

    def diagnostics_exact(self, pos, vel, eps2: float, pot=None) -> dict:
        """K, W, E, momentum, angular momentum, mass and centre of mass of a state; W from the
        given potentials p_i (self term included, as the method returns them) or, if pot is
        None, from the oracle's own potential sum."""
        p = _bodies64(pos)
        v = _bodies64(vel)
        if p.shape != v.shape:
            raise ValueError("pos and vel shapes differ")
        pp = None if pot is None else np.ascontiguousarray(pot, dtype=np.float64)
        if pp is not None and pp.shape != (p.shape[0],):
            raise ValueError("pot must hold one value per body")
        out = np.zeros(13)
        rc = self._lib.oracle_diagnostics(_ptr(p), _ptr(v), _ptr(pp), p.shape[0], float(eps2),
                                          _ptr(out))
        if rc != 0:
            raise ValueError("oracle_diagnostics rejected its arguments")
        return unpack_diagnostics(out)

    def diagnostics(self, pos, vel, eps2, pot=None) -> dict:
        return self.diagnostics_exact(pos, vel, as_f32(eps2), pot)


    def p2p_exact(self, pos, eps2: float, cell_start, list_off, cells) -> dict:
        """Near field over cell interaction lists (CSR: cell_start[ncell+1], list_off[ncell+1],
        cells[list_off[-1]]); float64 bodies and eps2 as given. Arrays as in accel_exact."""
        p = _bodies64(pos)
        n = p.shape[0]
        cs = np.ascontiguousarray(cell_start, dtype=np.int32)
        lo = np.ascontiguousarray(list_off, dtype=np.int32)
        li = np.ascontiguousarray(cells, dtype=np.int32)
        if li.size == 0:
            li = np.zeros(1, np.int32)
        ncell = cs.shape[0] - 1
        if lo.shape[0] != ncell + 1:
            raise ValueError("list_off must have ncell + 1 entries")
        acc = np.zeros((n, 3))
        pot = np.zeros(n)
        ba = np.zeros(n)
        bp = np.zeros(n)
        i32 = ctypes.POINTER(ctypes.c_int32)
        rc = self._lib.oracle_p2p(_ptr(p), n, float(eps2), _ptr(cs, i32), ncell, _ptr(lo, i32),
                                  _ptr(li, i32), _ptr(acc), _ptr(pot), _ptr(ba), _ptr(bp))
        if rc != 0:
            raise ValueError("oracle_p2p rejected its arguments")
        return {"acc": acc, "pot": pot, "bound_a": ba, "bound_p": bp}

    def p2p(self, pos, eps2, cell_start, list_off, cells) -> dict:
        return self.p2p_exact(pos, as_f32(eps2), cell_start, list_off, cells)

    def near_grid_exact(self, pos, eps2: float, lo, h: float, dims, targets=None) -> dict:
        """Near field on a uniform grid by definition (neighbouring cells by coordinates)."""
        p = _bodies64(pos)
        n = p.shape[0]
        lo64 = np.ascontiguousarray(lo, dtype=np.float64)
        d32 = np.ascontiguousarray(dims, dtype=np.int32)
        if targets is None:
            t, nt = None, n
        else:
            t = np.ascontiguousarray(targets, dtype=np.int64)
            nt = t.shape[0]
        acc = np.zeros((nt, 3))
        pot = np.zeros(nt)
        ba = np.zeros(nt)
        bp = np.zeros(nt)
        rc = self._lib.oracle_near_grid(_ptr(p), n, float(eps2), _ptr(lo64), float(h),
                                        _ptr(d32, ctypes.POINTER(ctypes.c_int32)),
                                        _ptr(t, _c_int64_p), nt, _ptr(acc), _ptr(pot), _ptr(ba),
                                        _ptr(bp))
        if rc != 0:
            raise ValueError("oracle_near_grid rejected its arguments")
        return {"acc": acc, "pot": pot, "bound_a": ba, "bound_p": bp}

    def near_grid(self, pos, eps2, lo, h, dims, targets=None) -> dict:
        """As near_grid_exact with eps2, lo and h rounded to float32 first (the GPU's values)."""
        lo32 = [as_f32(v) for v in lo]
        return self.near_grid_exact(pos, as_f32(eps2), lo32, as_f32(h), dims, targets)

    def near_tree_exact(self, pos, eps2: float, leaf_size: int, targets=None) -> dict:
        """Near field over the leaves of the Morton-order octree (leaves of at most leaf_size
        bodies; leaves near when their closed cubes meet), by definition."""
        p = _bodies64(pos)
        n = p.shape[0]
        if targets is None:
            t, nt = None, n
        else:
            t = np.ascontiguousarray(targets, dtype=np.int64)
            nt = t.shape[0]
        acc = np.zeros((nt, 3))
        pot = np.zeros(nt)
        ba = np.zeros(nt)
        bp = np.zeros(nt)
        rc = self._lib.oracle_near_tree(_ptr(p), n, float(eps2), int(leaf_size),
                                        _ptr(t, _c_int64_p), nt, _ptr(acc), _ptr(pot), _ptr(ba),
                                        _ptr(bp))
        if rc != 0:
            raise ValueError("oracle_near_tree rejected its arguments")
        return {"acc": acc, "pot": pot, "bound_a": ba, "bound_p": bp}

    def near_tree(self, pos, eps2, leaf_size, targets=None) -> dict:
        """As near_tree_exact with eps2 rounded to float32 first (the GPU's value)."""
        return self.near_tree_exact(pos, as_f32(eps2), leaf_size, targets)

    def shard_exact(self, pos, eps2: float, band: int, shard: int, nshards: int,
                    targets=None) -> dict:
        """One shard's part of the direct sum (the pairs of the bands it owns, see
        oracle_shard); float64 bodies and eps2 as given. Arrays as in accel_exact; pot is
        minus the shard's sum of m_j / r."""
        p = _bodies64(pos)
        n = p.shape[0]
        if targets is None:
            t, nt = None, n
        else:
            t = np.ascontiguousarray(targets, dtype=np.int64)
            nt = t.shape[0]
        acc = np.zeros((nt, 3))
        pot = np.zeros(nt)
        ba = np.zeros(nt)
        bp = np.zeros(nt)
        rc = self._lib.oracle_shard(_ptr(p), n, float(eps2), int(band), int(shard), int(nshards),
                                    _ptr(t, _c_int64_p), nt, _ptr(acc), _ptr(pot), _ptr(ba),
                                    _ptr(bp))
        if rc != 0:
            raise ValueError("oracle_shard rejected its arguments")
        return {"acc": acc, "pot": pot, "bound_a": ba, "bound_p": bp}

    def shard(self, pos, eps2, band, shard, nshards, targets=None) -> dict:
        return self.shard_exact(pos, as_f32(eps2), band, shard, nshards, targets)


def unpack_diagnostics(out) -> dict:
    """The 13-value diagnostics record as a dict (same order as oracle_diagnostics)."""
    out = [float(x) for x in out]
    return {"kinetic": out[0], "potential": out[1], "total": out[2], "momentum": out[3:6],
            "angular_momentum": out[6:9], "mass": out[9], "centre_of_mass": out[10:13]}


_default: Oracle | None = None


def get() -> Oracle:
    """The oracle built from oracle.c (compiled on first use if nothing is built, or if the
    source is newer than the library)."""
    global _default
    if _default is None:
        if not LIB.exists() or LIB.stat().st_mtime < SRC.stat().st_mtime:
            build()
        _default = Oracle(LIB)
    return _default


def num_threads() -> int:
    return get().num_threads()


def accel(pos, eps2, targets=None) -> dict:
    return get().accel(pos, eps2, targets)


def accel_exact(pos, eps2, targets=None) -> dict:
    return get().accel_exact(pos, eps2, targets)


def euler(pos, vel, dt, eps2, nsteps: int = 1):
    return get().euler(pos, vel, dt, eps2, nsteps)


def euler_exact(pos, vel, dt, eps2, nsteps: int = 1):
    return get().euler_exact(pos, vel, dt, eps2, nsteps)


def energy(pos, vel, eps2):
    return get().energy(pos, vel, eps2)


def energy_exact(pos, vel, eps2):
    return get().energy_exact(pos, vel, eps2)


def diagnostics(pos, vel, eps2, pot=None) -> dict:
    return get().diagnostics(pos, vel, eps2, pot)


def diagnostics_exact(pos, vel, eps2, pot=None) -> dict:
    return get().diagnostics_exact(pos, vel, eps2, pot)


def p2p(pos, eps2, cell_start, list_off, cells) -> dict:
    return get().p2p(pos, eps2, cell_start, list_off, cells)


def near_grid(pos, eps2, lo, h, dims, targets=None) -> dict:
    return get().near_grid(pos, eps2, lo, h, dims, targets)


def shard(pos, eps2, band, shard_index, nshards, targets=None) -> dict:
    return get().shard(pos, eps2, band, shard_index, nshards, targets)


def near_tree(pos, eps2, leaf_size, targets=None) -> dict:
    return get().near_tree(pos, eps2, leaf_size, targets)
