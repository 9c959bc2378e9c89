"""The pair-symmetric near-grid kernel's cell bookkeeping, checked on the CPU.

Each unordered pair of neighbouring cells must be evaluated by exactly one of its two cells
(the owner, the one with the lower linear index), over the owner's five runs of consecutive
cells, and every body must find the slots of the pairs it belongs to. This test takes the
bookkeeping functions (the direction table, the launch mapping and the runs) out of the kernel
file, compiles them for the host with g++ and checks, for every grid up to 9 cells a side and
a few large ones:
- the launch mapping is a bijection of the cells (with and without heavy cells first), and
  with heavy cells first exactly the cells with all 13 forward neighbours come first;
- the cells an owner's runs cover are exactly its neighbours with a higher linear index, each
  once, inside the grid, with the direction number of its offset;
- every unordered neighbour pair is covered by exactly one owner;
- the finish's test for slot 1 + k of a cell (the cell minus direction k lies in the grid) holds
  exactly when that cell is the owner's neighbour in direction k.
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
#define __host__
#define __device__
%s
static int nfwd(int c, int dx, int dy, int dz)
{
    const int x = c %% dx, y = (c / dx) %% dy, z = c / (dx * dy);
    int k = 0;
    for (int q = 0; q < kSymDirs; ++q) {
        const int X = x + sym_dir_dx(q), Y = y + sym_dir_dy(q), Z = z + sym_dir_dz(q);
        k += X >= 0 && X < dx && Y >= 0 && Y < dy && Z < dz;
    }
    return k;
}
static int check(int dx, int dy, int dz)
{
    const int n = dx * dy * dz;
    for (int heavy = 0; heavy < 2; ++heavy) {
        std::vector<char> seen(n, 0);
        const bool active = heavy && dx >= 3 && dy >= 3 && dz >= 2;
        const int ni = active ? (dx - 2) * (dy - 2) * (dz - 1) : 0;
        for (int b = 0; b < n; ++b) {
            const int c = sym_cell(b, dx, dy, dz, heavy != 0);
            if (c < 0 || c >= n || seen[c]) return 1;
            seen[c] = 1;
            if (!active && c != b) return 2;
            const int k = nfwd(c, dx, dy, dz);
            if (active && (b < ni) != (k == kSymDirs)) return 3;
        }
    }
    std::vector<int> pairs((size_t)n * 27, 0);  // times the pair (c, neighbour offset) is covered
    for (int c = 0; c < n; ++c) {
        const int cx = c %% dx, cy = (c / dx) %% dy, cz = c / (dx * dy);
        std::vector<char> got(kSymDirs, 0);
        for (int t = 0; t < kSymRuns; ++t) {
            int y, z, xf, xl, k0;
            if (!sym_run(t, cx, cy, cz, dx, dy, dz, y, z, xf, xl, k0)) continue;
            if (y < 0 || y >= dy || z < 0 || z >= dz || xf < 0 || xl >= dx || xf > xl) return 4;
            for (int x = xf; x <= xl; ++x) {
                const int k = k0 + (x - xf);
                if (k < 0 || k >= kSymDirs) return 5;
                if (x - cx != sym_dir_dx(k) || y - cy != sym_dir_dy(k) || z - cz != sym_dir_dz(k))
                    return 6;
                const int o = (z * dy + y) * dx + x;
                if (o <= c) return 7;  // owners take the neighbours above them
                if (got[k]++) return 8;
                const int lo = c, off = (sym_dir_dx(k) + 1) + 3 * (sym_dir_dy(k) + 1) + 9 * (sym_dir_dz(k) + 1);
                pairs[(size_t)lo * 27 + off]++;
            }
        }
        for (int k = 0; k < kSymDirs; ++k) {
            const int X = cx + sym_dir_dx(k), Y = cy + sym_dir_dy(k), Z = cz + sym_dir_dz(k);
            const bool in = X >= 0 && X < dx && Y >= 0 && Y < dy && Z < dz;
            if (in != (got[k] != 0)) return 9;
            // the finish, from the neighbour's side: its cell minus dir k is c
            if (in) {
                const int ox = X - sym_dir_dx(k), oy = Y - sym_dir_dy(k), oz = Z - sym_dir_dz(k);
                if (!(ox >= 0 && ox < dx && oy >= 0 && oy < dy && oz >= 0)) return 10;
                if ((oz * dy + oy) * dx + ox != c) return 11;
            }
        }
    }
    // every unordered neighbour pair exactly once
    for (int c = 0; c < n; ++c) {
        const int cx = c %% dx, cy = (c / dx) %% dy, cz = c / (dx * dy);
        for (int ddz = -1; ddz <= 1; ++ddz)
            for (int ddy = -1; ddy <= 1; ++ddy)
                for (int ddx = -1; ddx <= 1; ++ddx) {
                    const int X = cx + ddx, Y = cy + ddy, Z = cz + ddz;
                    if (X < 0 || X >= dx || Y < 0 || Y >= dy || Z < 0 || Z >= dz) continue;
                    const int o = (Z * dy + Y) * dx + X;
                    if (o <= c) continue;
                    if (pairs[(size_t)c * 27 + (ddx + 1) + 3 * (ddy + 1) + 9 * (ddz + 1)] != 1) return 12;
                }
    }
    // the finish's test: slot 1 + k of a body in cell b exists iff b - dir_k is in the grid
    for (int b = 0; b < n; ++b) {
        const int bx = b %% dx, by = (b / dx) %% dy, bz = b / (dx * dy);
        for (int k = 0; k < kSymDirs; ++k) {
            const int ox = bx - sym_dir_dx(k), oy = by - sym_dir_dy(k), oz = bz - sym_dir_dz(k);
            const bool owner_in = ox >= 0 && ox < dx && oy >= 0 && oy < dy && oz >= 0;
            bool covered = false;
            if (owner_in) {
                int y, z, xf, xl, k0;
                const int t = k == 0 ? 0 : (k < 4 ? 1 : 2 + (k - 4) / 3);
                if (sym_run(t, ox, oy, oz, dx, dy, dz, y, z, xf, xl, k0))
                    covered = y == by && z == bz && bx >= xf && bx <= xl && k0 + (bx - xf) == k;
            }
            if (owner_in != covered) return 13;
        }
    }
    return 0;
}
int main()
{
    for (int dx = 1; dx <= 9; ++dx)
        for (int dy = 1; dy <= 9; ++dy)
            for (int dz = 1; dz <= 9; ++dz)
                if (int r = check(dx, dy, dz)) {
                    std::printf("fail %%d at %%d %%d %%d\n", r, dx, dy, dz);
                    return 1;
                }
    const int big[5][3] = {{16, 16, 16}, {40, 40, 40}, {3, 100, 7}, {128, 5, 20}, {1, 1, 300}};
    for (const auto &d : big)
        if (int r = check(d[0], d[1], d[2])) {
            std::printf("fail %%d at %%d %%d %%d\n", r, d[0], d[1], d[2]);
            return 1;
        }
    std::printf("ok\n");
    return 0;
}
"""


def _bookkeeping_source() -> str:
    text = KERNELS.read_text()
    start = text.index("constexpr int kSymRuns")
    end = text.index("struct SymShared {", start)
    return text[start:end]


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_sym_grid_bookkeeping(tmp_path):
    src = tmp_path / "sym_order.cpp"
    src.write_text(DRIVER % _bookkeeping_source())
    exe = tmp_path / "sym_order"
    build = subprocess.run(["g++", "-std=c++17", "-O2", "-o", str(exe), str(src)],
                           capture_output=True, text=True, timeout=120)
    assert build.returncode == 0, build.stderr[-3000:]
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert run.returncode == 0 and run.stdout.strip() == "ok", run.stdout + run.stderr
