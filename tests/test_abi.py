"""C-ABI library: loads, exports every declared symbol, rejects bad arguments
before any HIP call. CPU only (no compute call is made)."""

import ctypes
import math
import re
import subprocess
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
HEADER = ROOT / "include" / "nbody.h"


@pytest.fixture(scope="module")
def nb():
    lib = ROOT / "direct_all_pairs_amd" / "libnbody_amd.so"
    if not lib.exists():
        import __graft_entry__

        __graft_entry__._hip_build_module().build()
    import direct_all_pairs_amd

    return direct_all_pairs_amd


def declared_functions():
    text = re.sub(r"/\*.*?\*/", "", HEADER.read_text(), flags=re.S)
    return sorted(set(re.findall(r"\b(nbody_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for f in ("nbody_accel", "nbody_step", "nbody_last_error", "nbody_release_workspace"):
        assert f in names


def test_exports_every_declared_symbol(nb):
    lib = ctypes.CDLL(str(nb.LIB_PATH))
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", str(nb.LIB_PATH)], capture_output=True,
                         text=True).stdout
    exported = set(re.findall(r" T (nbody_\w+)", out))
    assert set(declared_functions()) <= exported
    assert set(nb.EXPORTS) == set(declared_functions())
    # nothing else: the kernels and launchers stay internal (hidden visibility)
    assert set(re.findall(r" T (\S+)", out)) == set(declared_functions())


def test_library_links_no_oracle_and_no_torch(nb):
    out = subprocess.run(["ldd", str(nb.LIB_PATH)], capture_output=True, text=True).stdout
    assert "oracle" not in out and "torch" not in out and "amdhip64" in out


def test_product_sources_never_touch_the_oracle():
    pkg = ROOT / "direct_all_pairs_amd"
    for f in list(pkg.rglob("*.py")) + list(pkg.rglob("*.hip")) + list(pkg.rglob("*.h")):
        text = f.read_text()
        assert "oracle" not in text.lower(), f"{f} mentions the oracle"


A = 1 << 20  # a fake, 16-byte aligned address: never dereferenced (checks fail first)
B = 1 << 28


def call_accel(nb, pos=A, n=16, eps2=1e-4, acc=B, pot=None):
    return nb.nbody_accel(pos, n, eps2, acc, pot, stream=0, check=False)


def test_n_zero_is_a_no_op(nb):
    assert call_accel(nb, pos=None, n=0, acc=None) == nb.NBODY_OK
    assert nb.nbody_step(None, None, 0, 1e-3, 1e-4, 5, stream=0, check=False) == nb.NBODY_OK
    assert nb.nbody_step(A, B, 10, 1e-3, 1e-4, 0, stream=0, check=False) == nb.NBODY_OK


@pytest.mark.parametrize("kw,code", [
    (dict(n=-1), 1), (dict(n=2**31), 1), (dict(n=2**30 + 1), 1), (dict(pos=None), 1),
    (dict(acc=None), 1),
    (dict(eps2=0.0), 1), (dict(eps2=-1e-4), 1), (dict(eps2=math.nan), 1),
    (dict(eps2=math.inf), 1), (dict(eps2=1e-40), 1), (dict(eps2=1e-30), 1),
    # the lower bound 2^-84: the float just below it is rejected; 2^-84 itself passes the
    # eps2 check and the call fails at the next one (a misaligned pointer), before any HIP call
    (dict(eps2=2.0 ** -84 * (1 - 2.0 ** -24)), 1), (dict(eps2=2.0 ** -84, pos=A + 4), 2),
    (dict(pos=A + 4), 2), (dict(acc=B + 8), 2), (dict(pot=B + 2), 2),
    (dict(acc=A + 16), 1), (dict(pot=A + 64), 1), (dict(pot=B + 16), 1),
])
def test_accel_rejects(nb, kw, code):
    assert call_accel(nb, **kw) == code
    assert nb.nbody_last_error() != ""


@pytest.mark.parametrize("args,code", [
    ((A, B, -1, 1e-3, 1e-4, 1), 1), ((A, B, 16, 1e-3, 1e-4, -1), 1),
    ((None, B, 16, 1e-3, 1e-4, 1), 1), ((A, None, 16, 1e-3, 1e-4, 1), 1),
    ((A, B, 16, math.nan, 1e-4, 1), 1), ((A, B, 16, math.inf, 1e-4, 1), 1),
    ((A, B, 16, 1e-3, 0.0, 1), 1), ((A + 4, B, 16, 1e-3, 1e-4, 1), 2),
    ((A, B + 4, 16, 1e-3, 1e-4, 1), 2), ((A, A + 128, 16, 1e-3, 1e-4, 1), 1),
])
def test_step_rejects(nb, args, code):
    assert nb.nbody_step(*args, stream=0, check=False) == code
    # the static-scratch variant runs the same checks first
    assert nb.nbody_step_noalloc(*args, stream=0, check=False) == code


def test_noalloc_trivial_calls_are_no_ops(nb):
    assert nb.nbody_step_noalloc(None, None, 0, 1e-3, 1e-4, 5, stream=0, check=False) == 0
    assert nb.nbody_step_noalloc(A, B, 10, 1e-3, 1e-4, 0, stream=0, check=False) == 0


def test_time_kernel_takes_both_events_or_none(nb):
    assert nb.nbody_time_kernel(A, None, check=False) == nb.NBODY_EINVAL
    assert nb.nbody_time_kernel(None, B, check=False) == nb.NBODY_EINVAL
    assert "both" in nb.nbody_last_error()
    assert nb.nbody_time_kernel(None, None, check=False) == nb.NBODY_OK


C = 1 << 29


@pytest.mark.parametrize("kw,code", [
    (dict(n=-1), 1), (dict(out=None), 1), (dict(pos=None), 1), (dict(vel=None), 1),
    (dict(eps2=0.0), 1), (dict(eps2=math.nan), 1), (dict(out=C + 4), 2), (dict(pos=A + 8), 2),
    (dict(vel=B + 4), 2), (dict(pot=C + 4096 + 2), 2), (dict(out=A + 32), 1),
    (dict(out=B + 16), 1), (dict(pot=C + 4096, out=C + 4096 + 8), 1),
])
def test_diagnostics_rejects(nb, kw, code):
    args = dict(pos=A, vel=B, n=16, eps2=1e-4, out=C, pot=None)
    args.update(kw)
    rc = nb.nbody_diagnostics(args["pos"], args["vel"], args["n"], args["eps2"], args["out"],
                              pot=args["pot"], stream=0, check=False)
    assert rc == code, kw
    assert nb.nbody_last_error() != ""


@pytest.mark.parametrize("bad,code", [
    (dict(n=-1), 1), (dict(x=None), 1), (dict(m=None), 1), (dict(az=None), 1),
    (dict(eps2=0.0), 1), (dict(y=A + 4096 + 2), 2), (dict(ay=C + 8192 + 1), 2),
    (dict(pot=C + 3), 2), (dict(ax=A), 1), (dict(ay=C), 1), (dict(pot=C + 8192 + 32), 1),
])
def test_accel_soa_rejects(nb, bad, code):
    a = dict(x=A, y=A + 4096, z=A + 8192, m=A + 12288, n=16, eps2=1e-4, ax=C, ay=C + 8192,
             az=C + 16384, pot=None)
    a.update(bad)
    rc = nb.nbody_accel_soa(a["x"], a["y"], a["z"], a["m"], a["n"], a["eps2"], a["ax"], a["ay"],
                            a["az"], a["pot"], stream=0, check=False)
    assert rc == code, bad
    assert nb.nbody_last_error() != ""


@pytest.mark.parametrize("bad,code", [
    (dict(n=-1), 1), (dict(nsteps=-1), 1), (dict(vz=None), 1), (dict(m=None), 1),
    (dict(dt=math.inf), 1), (dict(x=A + 1), 2), (dict(vy=B + 4096 + 2), 2),
    (dict(vx=A), 1), (dict(m=A + 4096 + 32), 1),
])
def test_step_soa_rejects(nb, bad, code):
    a = dict(x=A, y=A + 4096, z=A + 8192, m=A + 12288, vx=B, vy=B + 4096, vz=B + 8192, n=16,
             dt=1e-3, eps2=1e-4, nsteps=1)
    a.update(bad)
    rc = nb.nbody_step_soa(a["x"], a["y"], a["z"], a["m"], a["vx"], a["vy"], a["vz"], a["n"],
                           a["dt"], a["eps2"], a["nsteps"], stream=0, check=False)
    assert rc == code, bad
    assert nb.nbody_last_error() != ""


def test_soa_zero_work_is_a_no_op(nb):
    assert nb.nbody_accel_soa(None, None, None, None, 0, 1e-4, None, None, None, None,
                              stream=0, check=False) == nb.NBODY_OK
    assert nb.nbody_step_soa(A, A + 4096, A + 8192, A + 12288, B, B + 4096, B + 8192, 16, 1e-3,
                             1e-4, 0, stream=0, check=False) == nb.NBODY_OK


@pytest.mark.parametrize("bad,code", [
    (dict(n=-1), 1), (dict(ncell=-1), 1), (dict(nlist=-1), 1), (dict(nlist=2**31), 1),
    (dict(pos=None), 1), (dict(acc=None), 1), (dict(cs=None), 1), (dict(lo=None), 1),
    (dict(cells=None), 1), (dict(eps2=0.0), 1), (dict(pos=A + 8), 2), (dict(cs=C + 2), 2),
    (dict(pot=B + 4096 + 1), 2), (dict(acc=A + 16), 1), (dict(acc=C), 1),
    (dict(pot=B + 64), 1),
])
def test_p2p_rejects(nb, bad, code):
    a = dict(pos=A, n=16, eps2=1e-4, cs=C, ncell=4, lo=C + 4096, cells=C + 8192, nlist=10, acc=B,
             pot=None)
    a.update(bad)
    rc = nb.nbody_p2p(a["pos"], a["n"], a["eps2"], a["cs"], a["ncell"], a["lo"], a["cells"],
                      a["nlist"], a["acc"], a["pot"], stream=0, check=False)
    assert rc == code, bad
    assert nb.nbody_last_error() != ""


def test_p2p_nothing_to_do(nb):
    assert nb.nbody_p2p(None, 0, 1e-4, None, 0, None, None, 0, None, stream=0,
                        check=False) == nb.NBODY_OK
    assert nb.nbody_p2p(A, 16, 1e-4, None, 0, None, None, 0, B, stream=0,
                        check=False) == nb.NBODY_OK


@pytest.mark.parametrize("bad,code", [
    (dict(n=-1), 1), (dict(dims=(0, 4, 4)), 1), (dict(dims=(4, -1, 4)), 1),
    (dict(dims=(1 << 10, 1 << 10, 1 << 9)), 1), (dict(lo=(0.0, math.nan, 0.0)), 1),
    (dict(lo=(math.inf, 0.0, 0.0)), 1), (dict(h=0.0), 1), (dict(h=-1.0), 1),
    (dict(h=math.inf), 1), (dict(h=1e-39), 1), (dict(pos=None), 1), (dict(acc=None), 1),
    (dict(eps2=-1.0), 1), (dict(pos=A + 4), 2), (dict(acc=B + 4), 2), (dict(pot=C + 2), 2),
    (dict(acc=A + 64), 1), (dict(pot=A), 1), (dict(lo=None), 1), (dict(dims=None), 1),
])
def test_near_grid_rejects(nb, bad, code):
    a = dict(pos=A, n=16, eps2=1e-4, lo=(-1.0, -1.0, -1.0), h=0.5, dims=(4, 4, 4), acc=B,
             pot=None)
    a.update(bad)
    rc = nb.nbody_near_grid(a["pos"], a["n"], a["eps2"], a["lo"], a["h"], a["dims"], a["acc"],
                            a["pot"], stream=0, check=False)
    assert rc == code, bad
    assert nb.nbody_last_error() != ""


@pytest.mark.parametrize("bad,code", [
    (dict(n=-1), 1), (dict(n=(1 << 30) + 1), 1), (dict(leaf=0), 1), (dict(leaf=-5), 1),
    (dict(pos=None), 1), (dict(acc=None), 1), (dict(eps2=0.0), 1), (dict(eps2=math.inf), 1),
    (dict(eps2=2.0 ** -86), 1), (dict(pos=A + 4), 2), (dict(acc=B + 4), 2),
    (dict(pot=C + 2), 2), (dict(acc=A + 64), 1), (dict(pot=A), 1), (dict(pot=B + 16), 1),
])
def test_near_tree_rejects(nb, bad, code):
    a = dict(pos=A, n=16, eps2=1e-4, leaf=4, acc=B, pot=None)
    a.update(bad)
    st = nb.nbody_tree_stats(7, 7, 7)
    rc = nb.nbody_near_tree(a["pos"], a["n"], a["eps2"], a["leaf"], a["acc"], a["pot"], st,
                            stream=0, check=False)
    assert rc == code, bad
    assert nb.nbody_last_error() != ""


def test_near_tree_nothing_to_do(nb):
    st = nb.nbody_tree_stats(7, 7, 7)
    assert nb.nbody_near_tree(None, 0, 1e-4, 1, None, None, st, stream=0,
                              check=False) == nb.NBODY_OK
    assert (st.leaves, st.list_entries, st.pair_terms) == (0, 0, 0)
    assert nb.nbody_near_tree(None, 0, 1e-4, 1, None, None, None, stream=0,
                              check=False) == nb.NBODY_OK


PAIRS512 = dict(mode=2, band=512)


@pytest.mark.parametrize("bad,code", [
    (dict(n=-1), 1), (dict(nshards=0), 1), (dict(shard=-1), 1), (dict(shard=4), 1),
    (dict(plan=dict(mode=1)), 1), (dict(plan=dict(mode=0)), 1), (dict(nshards=33, shard=0), 1),
    (dict(pos=None), 1), (dict(out=None), 1), (dict(eps2=0.0), 1), (dict(eps2=math.nan), 1),
    (dict(pos=A + 4), 2), (dict(out=B + 8), 2), (dict(out=A + 64), 1),
    (dict(plan=dict(mode=2, band=300)), 1), (dict(plan=dict(mode=2, tpl=2)), 1),
])
def test_accel_shard_rejects(nb, bad, code):
    a = dict(pos=A, n=16384, eps2=1e-4, shard=1, nshards=4, plan=PAIRS512, out=B)
    a.update(bad)
    rc = nb.nbody_accel_shard(a["pos"], a["n"], a["eps2"], a["shard"], a["nshards"], a["out"],
                              plan=a["plan"], stream=0, check=False)
    assert rc == code, bad
    assert nb.nbody_last_error() != ""


@pytest.mark.parametrize("bad,code", [
    (dict(n=-1), 1), (dict(nshards=0), 1), (dict(t0=-1), 1), (dict(t0=9, t1=8), 1),
    (dict(t1=17), 1), (dict(parts=None), 1), (dict(acc=None), 1), (dict(parts=A + 4), 2),
    (dict(acc=B + 4), 2), (dict(pot=C + 2), 2), (dict(acc=A + 256), 1), (dict(pot=A), 1),
    (dict(pot=B), 1),
])
def test_shard_finish_rejects(nb, bad, code):
    a = dict(parts=A, n=16, nshards=3, t0=2, t1=10, acc=B, pot=C)
    a.update(bad)
    rc = nb.nbody_shard_finish(a["parts"], a["n"], a["nshards"], a["t0"], a["t1"], a["acc"],
                               a["pot"], stream=0, check=False)
    assert rc == code, bad
    assert nb.nbody_last_error() != ""


def test_shard_nothing_to_do(nb):
    assert nb.nbody_accel_shard(None, 0, 1e-4, 0, 1, None, stream=0, check=False) == nb.NBODY_OK
    assert nb.nbody_shard_finish(None, 16, 2, 5, 5, None, None, stream=0,
                                 check=False) == nb.NBODY_OK


def test_plan_rejects_bad_fields(nb):
    for plan in (dict(bcast=7), dict(tpl=3), dict(splits=-1), dict(splits=5000), dict(mode=4),
                 dict(mode=3, tpl=2), dict(mode=3, tpl=64), dict(mode=3, splits=2),
                 dict(mode=3, wg=64), dict(mode=3, band=512), dict(mode=3, bcast="scalar"),
                 dict(band=300), dict(mode=2, splits=4), dict(mode=2, tpl=2), dict(mode=2, tpl=1),
                 dict(mode=2, band=256, tpl=8), dict(mode=2, band=128), dict(mode=2, passes=-1),
                 dict(mode=2, band=4096, tpl=4), dict(mode=2, band=8192),
                 dict(mode=1, passes=2), dict(mode=3, passes=2),
                 dict(mode=2, run=-1), dict(mode=2, run=(1 << 16) + 1), dict(mode=1, run=2),
                 dict(mode=3, run=2), dict(run=-3),
                 dict(mode=2, bcast="scalar"), dict(wg=512, bcast="scalar"), dict(wg=96),
                 dict(wg=64, bcast="readlane")):
        rc = nb.nbody_accel_plan(A, 16, 1e-4, B, None, plan=plan, stream=0, check=False)
        assert rc == nb.NBODY_EINVAL, plan


def test_error_raises_in_checked_mode(nb):
    with pytest.raises(nb.NbodyError) as ei:
        nb.nbody_accel(A, -5, 1e-4, B, None, stream=0)
    assert ei.value.code == nb.NBODY_EINVAL and "N=-5" in str(ei.value)


def test_version(nb):
    assert "gfx950" in nb.nbody_version()


def test_torch_conveniences_reject_bad_tensors(nb):
    """accel / step / diagnostics check their tensors before any library call: CPU tensors,
    wrong dtype or shape, non-contiguous views (no GPU needed)."""
    import torch

    good_shape = torch.zeros(8, 4)
    for bad in (good_shape, torch.zeros(8, 4, dtype=torch.float64), torch.zeros(8, 3),
                torch.zeros(4, 8).t()):
        with pytest.raises(ValueError):
            nb.accel(bad, 1e-4)
        with pytest.raises(ValueError):
            nb.step(bad, bad, 1e-3, 1e-4)
        with pytest.raises(ValueError):
            nb.diagnostics(bad, bad, 1e-4)


@pytest.mark.parametrize("kernel", [-1, 3, 100])
def test_near_grid_kernel_rejects_unknown_kernel(nb, kernel):
    rc = nb.nbody_near_grid_kernel(A, 16, 1e-4, (0.0, 0.0, 0.0), 1.0, (1, 1, 1), kernel, B, None,
                                   stream=0, check=False)
    assert rc == nb.NBODY_EINVAL and "kernel" in nb.nbody_last_error()
