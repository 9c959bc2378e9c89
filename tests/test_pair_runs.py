"""The run schedule of the pair-symmetric evaluation, checked on the CPU.

An owner band's band pairs d = 1 .. floor(nb/2) are split into runs of consecutive d, one
workgroup each, whose sums share one slot; the slot count and the launch grid follow from the
run count. This test takes the schedule's functions out of the kernel header, compiles them
for the host with g++ and checks for every band count up to 600 and run lengths 1 to 70, 128
and 1000: the runs are non-empty, consecutive and cover 1 .. floor(nb/2) exactly; their number
is pair_runs; runs of K (K >= 16) end in four shorter runs covering the last K values.
"""

from __future__ import annotations

import shutil
import subprocess
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
HEADER = ROOT / "direct_all_pairs_amd" / "csrc" / "kernels.h"

DRIVER = r"""
#include <cstdio>
#define __host__
#define __device__
%s
static int check(int nb, int K)
{
    const int D = nb / 2, R = pair_runs(nb, K);
    if (run_start(0, nb, K) != 0 || run_start(R, nb, K) != D) return 1;
    for (int r = 0; r < R; ++r) {
        const int a = run_start(r, nb, K), b = run_start(r + 1, nb, K);
        if (b <= a) return 2;          // empty run
        if (b - a > K) return 3;       // longer than K
    }
    if (K >= 16 && D > K) {
        if (R < 4 || run_start(R - 4, nb, K) != D - K) return 4;
        for (int r = R - 4; r < R - 1; ++r)
            if (run_start(r + 1, nb, K) - run_start(r, nb, K) != K / 4) return 5;
    }
    if (pair_slots(nb, K) != 1 + R + D) return 6;
    return 0;
}
int main()
{
    int ks[74];
    int nk = 0;
    for (int k = 1; k <= 70; ++k) ks[nk++] = k;
    ks[nk++] = 128;
    ks[nk++] = 1000;
    for (int nb = 1; nb <= 600; ++nb)
        for (int i = 0; i < nk; ++i)
            if (int r = check(nb, ks[i])) {
                std::printf("fail %%d at nb %%d K %%d\n", r, nb, ks[i]);
                return 1;
            }
    std::printf("ok\n");
    return 0;
}
"""


def _schedule_source() -> str:
    text = HEADER.read_text()
    start = text.index("constexpr int kRunSplitMin")
    end = text.index("// Pair-symmetric evaluation over bands of `band` bodies", start)
    return text[start:end]


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_pair_run_schedule(tmp_path):
    src = tmp_path / "runs.cpp"
    src.write_text(DRIVER % _schedule_source())
    exe = tmp_path / "runs"
    build = subprocess.run(["g++", "-std=c++17", "-O2", "-o", str(exe), str(src)],
                           capture_output=True, text=True, timeout=120)
    assert build.returncode == 0, build.stderr[-3000:]
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0 and run.stdout.strip() == "ok", run.stdout + run.stderr
