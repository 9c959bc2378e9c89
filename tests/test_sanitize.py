"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

- The C ABI: the library's sources and a driver (`sanitize/abi_driver.cpp`) that calls every
  entry point with arguments its checks reject before any HIP call; host code sanitized, GPU
  code built as usual (each -fsanitize flag applies to the host pass only).
- The oracle: oracle.c and a driver (`sanitize/oracle_driver.c`) that runs every function on
  small inputs, ragged sizes, bad lists, clamped grid cells, shard edges and bad arguments.
Any sanitizer finding aborts the driver and fails the test.
"""

from __future__ import annotations

import os
import shutil
import subprocess
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
HERE = Path(__file__).resolve().parent / "sanitize"
HIPCC = "/opt/rocm/bin/hipcc"


def _run(exe: Path, env_extra: dict) -> subprocess.CompletedProcess:
    env = dict(os.environ, **env_extra)
    return subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)


@pytest.mark.skipif(not Path(HIPCC).exists(), reason="hipcc not available")
def test_abi_checks_under_sanitizers(tmp_path):
    csrc = ROOT / "direct_all_pairs_amd" / "csrc"
    exe = tmp_path / "abi_san"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all",
           f"-I{ROOT / 'include'}", "-o", str(exe), str(HERE / "abi_driver.cpp"),
           "-x", "hip", str(csrc / "api.hip"), str(csrc / "kernels.hip")]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-3000:]
    # the HIP runtime's own allocations at load time are not ours to report
    r = _run(exe, {"ASAN_OPTIONS": "detect_leaks=0", "UBSAN_OPTIONS": "print_stacktrace=1"})
    assert r.returncode == 0 and "ok: 0 failures" in r.stdout, r.stdout + r.stderr[-3000:]


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_sanitizers(tmp_path):
    exe = tmp_path / "oracle_san"
    cmd = ["gcc", "-O1", "-g", "-fopenmp", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-ffp-contract=off", "-o", str(exe),
           str(HERE / "oracle_driver.c"), str(ROOT / "oracle" / "oracle.c"), "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    r = _run(exe, {"OMP_NUM_THREADS": "2", "ASAN_OPTIONS": "detect_leaks=1"})
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout + r.stderr[-3000:]
