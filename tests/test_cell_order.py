"""The launch order of grid cells in the near-field kernel, checked on the CPU.

The kernel maps each workgroup's launch index to a cell (`GridLists::cell`): with heavy cells
first, the interior cells, then faces, edges and corners. Every cell must be evaluated exactly
once, whatever the grid, so the mapping must be a bijection of [0, dx*dy*dz). This test takes
the mapping's source text out of the kernel file, compiles it for the host with g++ and checks,
for every grid up to 12 cells a side and a few large ones: a bijection; with heavy_first the
neighbourhood sizes never grow along the launch order; without it, the identity.
"""

from __future__ import annotations

import shutil
import subprocess
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
KERNELS = ROOT / "direct_all_pairs_amd" / "csrc" / "kernels.hip"

DRIVER = r"""
#include <cstdio>
#include <vector>
struct G {
    int dx, dy, dz;
    int *nbr;
    int heavy_first;
%s
};
static int hood(int c, int dx, int dy, int dz)
{
    const int v[3] = {c %% dx, (c / dx) %% dy, c / (dx * dy)}, d[3] = {dx, dy, dz};
    int k = 1;
    for (int i = 0; i < 3; ++i) k *= (v[i] > 0) + 1 + (v[i] < d[i] - 1);
    return k;
}
static int check(int dx, int dy, int dz, int heavy)
{
    G g{dx, dy, dz, nullptr, heavy};
    const int n = dx * dy * dz;
    std::vector<char> seen(n, 0);
    int prev = 28;
    for (int b = 0; b < n; ++b) {
        const int c = g.cell(b);
        if (c < 0 || c >= n || seen[c]) return 1;
        seen[c] = 1;
        if (!heavy && c != b) return 2;
        const int k = hood(c, dx, dy, dz);
        if (heavy && dx >= 3 && dy >= 3 && dz >= 3 && k > prev) return 3;
        prev = k;
    }
    return 0;
}
int main()
{
    for (int heavy = 0; heavy < 2; ++heavy) {
        for (int dx = 1; dx <= 12; ++dx)
            for (int dy = 1; dy <= 12; ++dy)
                for (int dz = 1; dz <= 12; ++dz)
                    if (int r = check(dx, dy, dz, heavy)) {
                        std::printf("fail %%d at %%d %%d %%d heavy %%d\n", r, dx, dy, dz, heavy);
                        return 1;
                    }
        const int big[4][3] = {{16, 16, 16}, {64, 64, 64}, {3, 100, 7}, {128, 5, 40}};
        for (const auto &d : big)
            if (int r = check(d[0], d[1], d[2], heavy)) {
                std::printf("fail %%d at %%d %%d %%d heavy %%d\n", r, d[0], d[1], d[2], heavy);
                return 1;
            }
    }
    std::printf("ok\n");
    return 0;
}
"""


def _mapping_source() -> str:
    text = KERNELS.read_text()
    start = text.index("    __device__ int at(int x, int y, int z) const")
    end = text.index("    __device__ const int *pre() const", start)
    return text[start:end].replace("__device__ ", "")


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_grid_cell_launch_order_is_a_bijection(tmp_path):
    src = tmp_path / "cell_order.cpp"
    src.write_text(DRIVER % _mapping_source())
    exe = tmp_path / "cell_order"
    build = subprocess.run(["g++", "-std=c++17", "-O1", "-o", str(exe), str(src)],
                           capture_output=True, text=True, timeout=120)
    assert build.returncode == 0, build.stderr[-3000:]
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0 and run.stdout.strip() == "ok", run.stdout + run.stderr
