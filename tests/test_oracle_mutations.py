"""Each plausible mistake planted in a copy of oracle.c must trip at least one pin.

The copies are built in a temporary directory on the CPU; the real oracle is
never modified. This shows the pins are tight enough to catch a dropped term,
a wrong sign or index, a transposed operand or a wrong update order.
"""

import shutil

import pytest

import oracle
import pins

# (name, text in oracle.c, replacement)
MUTATIONS = [
    ("r_ij sign flipped in x", "pos[4 * j + 0] - xi", "xi - pos[4 * j + 0]"),
    ("eps instead of eps^2", "const double q = r2 + eps2;", "const double q = r2 + eps2 * eps2;"),
    ("self term skipped", "for (int64_t j = 0; j < n; ++j) add_pair(pos, i, j, eps2, &s);",
     "for (int64_t j = 0; j < n; ++j) if (j != i) add_pair(pos, i, j, eps2, &s);"),
    ("exponent 1 instead of 3/2", "const double q32 = q * sqrt(q);", "const double q32 = q;"),
    ("target mass instead of source mass", "const double mj = pos[4 * j + 3];",
     "const double mj = pos[4 * i + 3];"),
    ("potential sign", "s->pp -= mj / sqrt(q);", "s->pp += mj / sqrt(q);"),
    ("y component uses dx", "s->ay += mj * dy / q32;", "s->ay += mj * dx / q32;"),
    ("last source dropped", "for (int64_t j = 0; j < n; ++j) add_pair(pos, i, j, eps2, &s);",
     "for (int64_t j = 0; j < n - 1; ++j) add_pair(pos, i, j, eps2, &s);"),
    ("B scale without |r|", "s->sa += mj * sqrt(r2) / q32;", "s->sa += mj / q32;"),
    ("Euler: velocity first",
     "for (int c = 0; c < 3; ++c) pos[4 * i + c] += dt * vel[4 * i + c];  /* old v */\n"
     "            for (int c = 0; c < 3; ++c) vel[4 * i + c] += dt * acc[3 * i + c];",
     "for (int c = 0; c < 3; ++c) vel[4 * i + c] += dt * acc[3 * i + c];\n"
     "            for (int c = 0; c < 3; ++c) pos[4 * i + c] += dt * vel[4 * i + c];"),
    ("energy pairs counted twice", "wi[i] = 0.5 * pos[4 * i + 3] * s;", "wi[i] = pos[4 * i + 3] * s;"),
    ("z acceleration dropped", "s->az += mj * dz / q32;", "s->az += 0.0;"),
    ("kinetic energy without 1/2", "k += 0.5 * m * (vx * vx + vy * vy + vz * vz);",
     "k += m * (vx * vx + vy * vy + vz * vz);"),
    ("self term added instead of removed", "w += 0.5 * m * (pot[i] + m * inv_eps);",
     "w += 0.5 * m * (pot[i] - m * inv_eps);"),
    ("angular momentum cross product reversed", "ang[2] += m * (x * vy - y * vx);",
     "ang[2] += m * (y * vx - x * vy);"),
    ("momentum uses position", "mom[1] += m * vy;", "mom[1] += m * y;"),
    ("centre of mass unweighted", "mx[0] += m * x;", "mx[0] += x;"),
    ("near grid: one-sided neighbourhood", "if (dd < -1 || dd > 1) near = 0;",
     "if (dd < -1 || dd > 0) near = 0;"),
    ("near grid: cell by rounding", "float f = floorf(d * inv_h);", "float f = roundf(d * inv_h);"),
    ("p2p: last body of each source cell dropped",
     "for (int64_t j = cell_start[s]; j < cell_start[s + 1]; ++j)\n",
     "for (int64_t j = cell_start[s]; j < cell_start[s + 1] - 1; ++j)\n"),
    ("p2p: negative list entry read as cell 0",
     "const int32_t s = list[e];\n                if (s < 0 || s >= ncell) continue;",
     "const int32_t s = list[e] < 0 ? 0 : list[e];\n                if (s >= ncell) continue;"),
    ("shard: opposite bands go to the upper band", "return bi < bj ? bi : bj;",
     "return bi > bj ? bi : bj;"),
    ("shard: opposite bands counted from both sides", "if (2 * up < nb) return bi;",
     "if (2 * up <= nb) return bi;"),
    ("shard: band ranges overlap", "b1 = (shard + 1) * nb / nshards;",
     "b1 = (shard + 1) * nb / nshards + 1;"),
    ("near tree: open cubes (face neighbours dropped)",
     "if (bj[d] > bi[d] + bi[3] || bi[d] > bj[d] + bj[3]) near = 0;",
     "if (bj[d] >= bi[d] + bi[3] || bi[d] >= bj[d] + bj[3]) near = 0;"),
    ("near tree: leaf holds fewer than leaf_size",
     "if (keys_in(sorted, n, p << s, (p + 1) << s) <= leaf_size) {",
     "if (keys_in(sorted, n, p << s, (p + 1) << s) < leaf_size) {"),
    ("near tree: deepest level instead of the first",
     "                level = L;\n                break;", "                level = L;"),
    ("near tree: root side is the smallest extent", "if (ext > side) side = ext;",
     "if (side == 0.0f || ext < side) side = ext;"),
    ("near tree: top face not clamped into the last cell",
     "if (f > cells - 1.0f) f = cells - 1.0f;", "if (f > cells) f = cells;"),
    ("near tree: leaf corner one level off", "box[4 * j + d] = o << (D - level);",
     "box[4 * j + d] = o << (D - 1 - level);"),
    ("near tree: ten levels instead of 21", "#define TREE_LEVELS 21", "#define TREE_LEVELS 10"),
]


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_mutation(tmp_path, name, old, new):
    src = oracle.SRC.read_text()
    assert src.count(old) == 1, f"mutation anchor not found exactly once: {name}"
    mutated = tmp_path / "oracle_mut.c"
    mutated.write_text(src.replace(old, new))
    lib = oracle.compile_oracle(mutated, tmp_path / "liboracle_mut.so")
    orc = oracle.Oracle(lib)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(orc)
        except AssertionError:
            caught.append(pin.__name__)
        except (ValueError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"no pin caught the planted mistake: {name}"
