"""Python binding of the gfx950 direct all-pairs softened-gravity library.

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libnbody_amd.so`` (C ABI in include/nbody.h). The functions with
the C names take raw device pointers or torch tensors (their ``data_ptr()`` is
passed); ``accel`` and ``step`` are small conveniences on torch tensors that
allocate outputs with torch and call the same entry points on the current
torch stream.

Importing this module loads the library and fails loudly if it has not been
built (``python direct_all_pairs_amd/build.py`` or ``__graft_entry__.build()``).
There is no CPU fallback.
"""

from __future__ import annotations

import ctypes
from pathlib import Path

_PKG = Path(__file__).resolve().parent
LIB_PATH = _PKG / "libnbody_amd.so"

NBODY_OK, NBODY_EINVAL, NBODY_EALIGN, NBODY_EHIP, NBODY_ENOMEM = 0, 1, 2, 3, 4
BCAST_AUTO, BCAST_LDS, BCAST_SCALAR, BCAST_READLANE = 0, 1, 2, 3
BCAST_NAMES = {BCAST_LDS: "lds", BCAST_SCALAR: "scalar", BCAST_READLANE: "readlane"}
MODE_AUTO, MODE_TILES, MODE_PAIRS, MODE_SMALL = 0, 1, 2, 3
MODE_NAMES = {MODE_TILES: "tiles", MODE_PAIRS: "pairs", MODE_SMALL: "small"}
NEAR_AUTO, NEAR_ONE_SIDED, NEAR_PAIRS = 0, 1, 2


class NbodyError(RuntimeError):
    def __init__(self, code: int, func: str, msg: str):
        super().__init__(f"{func} returned {code}: {msg}")
        self.code = code


class nbody_plan(ctypes.Structure):
    _fields_ = [("bcast", ctypes.c_int32), ("tpl", ctypes.c_int32),
                ("splits", ctypes.c_int32), ("chunk", ctypes.c_int32), ("wg", ctypes.c_int32),
                ("mode", ctypes.c_int32), ("band", ctypes.c_int32), ("passes", ctypes.c_int32),
                ("run", ctypes.c_int32)]

    def as_dict(self) -> dict:
        return {"mode": MODE_NAMES.get(self.mode, self.mode),
                "bcast": BCAST_NAMES.get(self.bcast, self.bcast), "tpl": self.tpl,
                "splits": self.splits, "chunk": self.chunk, "wg": self.wg, "band": self.band,
                "passes": self.passes, "run": self.run}


class nbody_tree_stats(ctypes.Structure):
    _fields_ = [("leaves", ctypes.c_int64), ("list_entries", ctypes.c_int64),
                ("pair_terms", ctypes.c_int64)]

    def as_dict(self) -> dict:
        return {"leaves": self.leaves, "list_entries": self.list_entries,
                "pair_terms": self.pair_terms}


# torch (device memory and streams) is imported first: its bundled HIP runtime
# carries the same soname (libamdhip64.so.7) the library links against, so the
# loader binds the library to the runtime already in the process instead of
# starting a second one that would not see the device.
import torch  # noqa: E402,F401

if not LIB_PATH.exists():
    raise ImportError(f"{LIB_PATH} is not built; run `python direct_all_pairs_amd/build.py` "
                      "(hipcc, gfx950) first. There is no CPU fallback.")

_lib = ctypes.CDLL(str(LIB_PATH))
_vp, _i64, _f32, _int = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int
_lib.nbody_accel.argtypes = [_vp, _i64, _f32, _vp, _vp, _vp]
_lib.nbody_accel_plan.argtypes = [_vp, _i64, _f32, _vp, _vp, ctypes.POINTER(nbody_plan), _vp]
_lib.nbody_step.argtypes = [_vp, _vp, _i64, _f32, _f32, _i64, _vp]
_lib.nbody_step_plan.argtypes = [_vp, _vp, _i64, _f32, _f32, _i64, ctypes.POINTER(nbody_plan),
                                 _vp]
_lib.nbody_step_noalloc.argtypes = [_vp, _vp, _i64, _f32, _f32, _i64, _vp]
_lib.nbody_time_kernel.argtypes = [_vp, _vp]
_lib.nbody_plan_for.argtypes = [_i64, _int, ctypes.POINTER(nbody_plan)]
_lib.nbody_diagnostics.argtypes = [_vp, _vp, _vp, _i64, _f32, _vp, _vp]
_lib.nbody_p2p.argtypes = [_vp, _i64, _f32, _vp, ctypes.c_int32, _vp, _vp, _i64, _vp, _vp, _vp]
_lib.nbody_near_grid.argtypes = [_vp, _i64, _f32, ctypes.POINTER(ctypes.c_float), _f32,
                                 ctypes.POINTER(ctypes.c_int32), _vp, _vp, _vp]
_lib.nbody_near_grid_kernel.argtypes = [_vp, _i64, _f32, ctypes.POINTER(ctypes.c_float), _f32,
                                        ctypes.POINTER(ctypes.c_int32), ctypes.c_int32, _vp, _vp,
                                        _vp]
_lib.nbody_near_tree.argtypes = [_vp, _i64, _f32, _i64, _vp, _vp, ctypes.POINTER(nbody_tree_stats),
                                 _vp]
_lib.nbody_accel_soa.argtypes = [_vp, _vp, _vp, _vp, _i64, _f32, _vp, _vp, _vp, _vp, _vp]
_lib.nbody_step_soa.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _f32, _f32, _i64, _vp]
_lib.nbody_accel_shard.argtypes = [_vp, _i64, _f32, ctypes.c_int32, ctypes.c_int32, _int,
                                   ctypes.POINTER(nbody_plan), _vp, _vp]
_lib.nbody_shard_finish.argtypes = [_vp, _i64, ctypes.c_int32, _i64, _i64, _vp, _vp, _vp]
_lib.nbody_last_error.restype = ctypes.c_char_p
_lib.nbody_release_workspace.argtypes = []
_lib.nbody_version.restype = ctypes.c_char_p
for _f in ("nbody_accel", "nbody_accel_plan", "nbody_step", "nbody_step_plan",
           "nbody_step_noalloc", "nbody_time_kernel", "nbody_accel_soa", "nbody_step_soa", "nbody_accel_shard", "nbody_shard_finish",
           "nbody_p2p", "nbody_near_grid", "nbody_near_grid_kernel", "nbody_near_tree",
           "nbody_diagnostics", "nbody_plan_for", "nbody_release_workspace"):
    getattr(_lib, _f).restype = _int

EXPORTS = ("nbody_accel", "nbody_accel_plan", "nbody_step", "nbody_step_plan",
           "nbody_step_noalloc", "nbody_time_kernel", "nbody_accel_soa", "nbody_step_soa",
           "nbody_accel_shard", "nbody_shard_finish", "nbody_p2p", "nbody_near_grid",
           "nbody_near_grid_kernel", "nbody_near_tree", "nbody_diagnostics", "nbody_plan_for", "nbody_last_error", "nbody_release_workspace",
           "nbody_version")
DIAG_FIELDS = ("kinetic", "potential", "total", "momentum", "angular_momentum", "mass",
               "centre_of_mass")


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()  # torch tensor


def _stream(stream):
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream  # torch.cuda.Stream


def _check(rc: int, func: str) -> int:
    if rc != NBODY_OK:
        raise NbodyError(rc, func, nbody_last_error())
    return rc


def nbody_last_error() -> str:
    return _lib.nbody_last_error().decode()


def nbody_version() -> str:
    return _lib.nbody_version().decode()


def nbody_release_workspace() -> int:
    return _check(_lib.nbody_release_workspace(), "nbody_release_workspace")


def nbody_accel(pos_xyzm, N: int, eps2: float, acc_out, pot_out=None, stream=None,
                check: bool = True) -> int:
    rc = _lib.nbody_accel(_ptr(pos_xyzm), int(N), float(eps2), _ptr(acc_out), _ptr(pot_out),
                          _stream(stream))
    return _check(rc, "nbody_accel") if check else rc


def nbody_accel_plan(pos_xyzm, N: int, eps2: float, acc_out, pot_out=None, plan=None,
                     stream=None, check: bool = True) -> int:
    p = None
    if plan is not None:
        p = plan if isinstance(plan, nbody_plan) else make_plan(**plan)
    rc = _lib.nbody_accel_plan(_ptr(pos_xyzm), int(N), float(eps2), _ptr(acc_out),
                               _ptr(pot_out), ctypes.byref(p) if p is not None else None,
                               _stream(stream))
    return _check(rc, "nbody_accel_plan") if check else rc


def nbody_step(pos, vel, N: int, dt: float, eps2: float, nsteps: int, stream=None,
               check: bool = True) -> int:
    rc = _lib.nbody_step(_ptr(pos), _ptr(vel), int(N), float(dt), float(eps2), int(nsteps),
                         _stream(stream))
    return _check(rc, "nbody_step") if check else rc


def nbody_step_plan(pos, vel, N: int, dt: float, eps2: float, nsteps: int, plan=None,
                    stream=None, check: bool = True) -> int:
    p = None
    if plan is not None:
        p = plan if isinstance(plan, nbody_plan) else make_plan(**plan)
    rc = _lib.nbody_step_plan(_ptr(pos), _ptr(vel), int(N), float(dt), float(eps2), int(nsteps),
                              ctypes.byref(p) if p is not None else None, _stream(stream))
    return _check(rc, "nbody_step_plan") if check else rc


def nbody_step_noalloc(pos, vel, N: int, dt: float, eps2: float, nsteps: int, stream=None,
                       check: bool = True) -> int:
    rc = _lib.nbody_step_noalloc(_ptr(pos), _ptr(vel), int(N), float(dt), float(eps2),
                                 int(nsteps), _stream(stream))
    return _check(rc, "nbody_step_noalloc") if check else rc


def _event(ev):
    """A raw hipEvent_t: None, an int, or a torch.cuda.Event that has been recorded once
    (torch creates the underlying event at its first record)."""
    if ev is None or isinstance(ev, int):
        return ev
    h = ev.cuda_event
    if not h:
        raise ValueError("record the torch.cuda.Event once before passing it (it is created "
                         "lazily)")
    return h


def nbody_time_kernel(start, stop, check: bool = True) -> int:
    rc = _lib.nbody_time_kernel(_event(start), _event(stop))
    return _check(rc, "nbody_time_kernel") if check else rc


def nbody_accel_soa(x, y, z, m, N: int, eps2: float, ax, ay, az, pot_out=None, stream=None,
                    check: bool = True) -> int:
    rc = _lib.nbody_accel_soa(_ptr(x), _ptr(y), _ptr(z), _ptr(m), int(N), float(eps2), _ptr(ax),
                              _ptr(ay), _ptr(az), _ptr(pot_out), _stream(stream))
    return _check(rc, "nbody_accel_soa") if check else rc


def nbody_step_soa(x, y, z, m, vx, vy, vz, N: int, dt: float, eps2: float, nsteps: int,
                   stream=None, check: bool = True) -> int:
    rc = _lib.nbody_step_soa(_ptr(x), _ptr(y), _ptr(z), _ptr(m), _ptr(vx), _ptr(vy), _ptr(vz),
                             int(N), float(dt), float(eps2), int(nsteps), _stream(stream))
    return _check(rc, "nbody_step_soa") if check else rc


def nbody_accel_shard(pos_xyzm, N: int, eps2: float, shard: int, nshards: int, partial_out,
                      want_pot: bool = True, plan=None, stream=None, check: bool = True) -> int:
    p = None
    if plan is not None:
        p = plan if isinstance(plan, nbody_plan) else make_plan(**plan)
    rc = _lib.nbody_accel_shard(_ptr(pos_xyzm), int(N), float(eps2), int(shard), int(nshards),
                                int(bool(want_pot)), ctypes.byref(p) if p is not None else None,
                                _ptr(partial_out), _stream(stream))
    return _check(rc, "nbody_accel_shard") if check else rc


def nbody_shard_finish(partials, N: int, nshards: int, t0: int, t1: int, acc_out, pot_out=None,
                       stream=None, check: bool = True) -> int:
    rc = _lib.nbody_shard_finish(_ptr(partials), int(N), int(nshards), int(t0), int(t1),
                                 _ptr(acc_out), _ptr(pot_out), _stream(stream))
    return _check(rc, "nbody_shard_finish") if check else rc


def nbody_p2p(pos, N: int, eps2: float, cell_start, ncell: int, list_off, cells, nlist: int,
              acc_out, pot_out=None, stream=None, check: bool = True) -> int:
    rc = _lib.nbody_p2p(_ptr(pos), int(N), float(eps2), _ptr(cell_start), int(ncell),
                        _ptr(list_off), _ptr(cells), int(nlist), _ptr(acc_out), _ptr(pot_out),
                        _stream(stream))
    return _check(rc, "nbody_p2p") if check else rc


def nbody_near_grid(pos, N: int, eps2: float, lo, h: float, dims, acc_out, pot_out=None,
                    stream=None, check: bool = True) -> int:
    """lo (3 floats) and dims (3 ints) are host values."""
    lo_c = (ctypes.c_float * 3)(*[float(v) for v in lo]) if lo is not None else None
    dims_c = (ctypes.c_int32 * 3)(*[int(v) for v in dims]) if dims is not None else None
    rc = _lib.nbody_near_grid(_ptr(pos), int(N), float(eps2), lo_c, float(h), dims_c,
                              _ptr(acc_out), _ptr(pot_out), _stream(stream))
    return _check(rc, "nbody_near_grid") if check else rc


def nbody_near_grid_kernel(pos, N: int, eps2: float, lo, h: float, dims, kernel: int, acc_out,
                           pot_out=None, stream=None, check: bool = True) -> int:
    """nbody_near_grid with the near-field kernel chosen (NEAR_AUTO, NEAR_ONE_SIDED,
    NEAR_PAIRS)."""
    lo_c = (ctypes.c_float * 3)(*[float(v) for v in lo]) if lo is not None else None
    dims_c = (ctypes.c_int32 * 3)(*[int(v) for v in dims]) if dims is not None else None
    rc = _lib.nbody_near_grid_kernel(_ptr(pos), int(N), float(eps2), lo_c, float(h), dims_c,
                                     int(kernel), _ptr(acc_out), _ptr(pot_out), _stream(stream))
    return _check(rc, "nbody_near_grid_kernel") if check else rc


def nbody_near_tree(pos, N: int, eps2: float, leaf_size: int, acc_out, pot_out=None,
                    stats: nbody_tree_stats | None = None, stream=None, check: bool = True) -> int:
    """stats: an nbody_tree_stats to fill (host), or None."""
    rc = _lib.nbody_near_tree(_ptr(pos), int(N), float(eps2), int(leaf_size), _ptr(acc_out),
                              _ptr(pot_out), ctypes.byref(stats) if stats is not None else None,
                              _stream(stream))
    return _check(rc, "nbody_near_tree") if check else rc


def nbody_diagnostics(pos, vel, N: int, eps2: float, out, pot=None, stream=None,
                      check: bool = True) -> int:
    """out: device buffer of 13 float64 (one nbody_diag); pot: device potentials or None."""
    rc = _lib.nbody_diagnostics(_ptr(pos), _ptr(vel), _ptr(pot), int(N), float(eps2), _ptr(out),
                                _stream(stream))
    return _check(rc, "nbody_diagnostics") if check else rc


def nbody_plan_for(N: int, want_pot: bool = False) -> nbody_plan:
    p = nbody_plan()
    _check(_lib.nbody_plan_for(int(N), int(bool(want_pot)), ctypes.byref(p)), "nbody_plan_for")
    return p


def make_plan(bcast=0, tpl=0, splits=0, chunk=0, wg=0, mode=0, band=0, passes=0,
              run=0) -> nbody_plan:
    if isinstance(bcast, str):
        bcast = {v: k for k, v in BCAST_NAMES.items()}[bcast]
    if isinstance(mode, str):
        mode = {v: k for k, v in MODE_NAMES.items()}[mode]
    return nbody_plan(int(bcast), int(tpl), int(splits), int(chunk), int(wg), int(mode), int(band),
                      int(passes), int(run))


# ------------------------------------------------------------ torch conveniences

def _bodies(t, name):
    import torch

    if not (isinstance(t, torch.Tensor) and t.is_cuda and t.dtype == torch.float32
            and t.dim() == 2 and t.shape[1] == 4 and t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous float32 CUDA tensor of shape (N, 4)")
    return t


def accel(pos, eps2: float, pot: bool = True, plan=None):
    """Accelerations (N, 4) with w = 0 and, if pot, potentials (N,), on the current stream."""
    import torch

    _bodies(pos, "pos")
    n = pos.shape[0]
    acc = torch.empty_like(pos)
    p = torch.empty(n, dtype=torch.float32, device=pos.device) if pot else None
    with torch.cuda.device(pos.device):  # the library works on the current device and stream
        if plan is None:
            nbody_accel(pos, n, eps2, acc, p)
        else:
            nbody_accel_plan(pos, n, eps2, acc, p, plan)
    return acc, p


def step(pos, vel, dt: float, eps2: float, nsteps: int = 1, plan=None):
    """nsteps Euler steps in place on pos and vel (N, 4) tensors, on the current stream."""
    import torch

    _bodies(pos, "pos")
    _bodies(vel, "vel")
    if vel.shape != pos.shape or vel.device != pos.device:
        raise ValueError("pos and vel differ in shape or device")
    with torch.cuda.device(pos.device):
        if plan is None:
            nbody_step(pos, vel, pos.shape[0], dt, eps2, nsteps)
        else:
            nbody_step_plan(pos, vel, pos.shape[0], dt, eps2, nsteps, plan)
    return pos, vel


def near_tree(pos, eps2: float, leaf_size: int, pot: bool = True):
    """Near field over octree leaves of at most leaf_size bodies, on the current stream:
    (acc (N, 4), pot (N,) or None, stats dict). Waits once on the stream for the build."""
    import torch

    _bodies(pos, "pos")
    n = pos.shape[0]
    acc = torch.empty_like(pos)
    p = torch.empty(n, dtype=torch.float32, device=pos.device) if pot else None
    st = nbody_tree_stats()
    with torch.cuda.device(pos.device):
        nbody_near_tree(pos, n, eps2, leaf_size, acc, p, st)
    return acc, p, st.as_dict()


def unpack_diag(vals) -> dict:
    """The 13 float64 of an nbody_diag as a dict."""
    v = [float(x) for x in vals]
    return {"kinetic": v[0], "potential": v[1], "total": v[2], "momentum": v[3:6],
            "angular_momentum": v[6:9], "mass": v[9], "centre_of_mass": v[10:13]}


def diagnostics(pos, vel, eps2: float, pot=None) -> dict:
    """nbody_diagnostics on (N, 4) tensors (pot: (N,) tensor or None), on the current stream;
    synchronises the stream and returns the values as a dict."""
    import torch

    _bodies(pos, "pos")
    _bodies(vel, "vel")
    if vel.shape != pos.shape or vel.device != pos.device:
        raise ValueError("pos and vel differ in shape or device")
    if pot is not None and not (isinstance(pot, torch.Tensor) and pot.is_cuda
                                and pot.dtype == torch.float32 and pot.shape == (pos.shape[0],)
                                and pot.is_contiguous() and pot.device == pos.device):
        raise ValueError("pot must be a contiguous float32 tensor of shape (N,) on pos's device")
    with torch.cuda.device(pos.device):
        out = torch.zeros(13, dtype=torch.float64, device=pos.device)
        nbody_diagnostics(pos, vel, pos.shape[0], eps2, out, pot)
        torch.cuda.current_stream().synchronize()
        return unpack_diag(out.cpu().tolist())
