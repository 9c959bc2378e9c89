"""Compile the gfx950 HIP library (C ABI of include/nbody.h) in-tree with hipcc."""

from __future__ import annotations

import os
import shutil
import subprocess
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
LIB = PKG / "libnbody_amd.so"
# Test build with the LDS race probe compiled in (loaded only by the race-probe tests).
PROBE_LIB = PKG / "libnbody_amd_probe.so"
SOURCES = [CSRC / "api.hip", CSRC / "kernels.hip"]

# -packed-fp32-ops is switched off on purpose: no v_pk_*_f32 is generated.
HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-ffp-contract=fast",
    "-fvisibility=hidden",
    "-mcode-object-version=5",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and Path(c).exists():
            return c
    raise RuntimeError("hipcc not found")


def _command(extra_flags, tmp: Path) -> list[str]:
    return [hipcc(), *HIPCC_FLAGS, *(extra_flags or []), f"-I{ROOT / 'include'}",
            "-o", str(tmp), *map(str, SOURCES)]


def build(extra_flags: list[str] | None = None, out: Path = LIB, verbose: bool = False) -> Path:
    tmp = out.with_name(out.name + ".tmp")
    cmd = _command(extra_flags, tmp)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{' '.join(cmd)}\n{r.stderr}")
    if verbose and r.stderr:
        print(r.stderr)
    os.replace(tmp, out)
    return out


def build_all(verbose: bool = False) -> list[Path]:
    """The library and its race-probe test build, compiled side by side."""
    jobs = [(LIB, []), (PROBE_LIB, ["-DNBK_RACE_PROBE"])]
    procs = []
    for out, flags in jobs:
        tmp = out.with_name(out.name + ".tmp")
        cmd = _command(flags, tmp)
        procs.append((out, tmp, cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                                      stderr=subprocess.PIPE, text=True)))
    errors = []
    for out, tmp, cmd, pr in procs:
        _, err = pr.communicate()
        if pr.returncode != 0:
            errors.append(f"hipcc failed ({pr.returncode}):\n{' '.join(cmd)}\n{err}")
        else:
            if verbose and err:
                print(err)
            os.replace(tmp, out)
    if errors:
        raise RuntimeError("\n".join(errors))
    return [out for out, _ in jobs]


if __name__ == "__main__":
    print(build_all(verbose=True))
