"""Measurement bookkeeping against the counts the pages print. CPU only."""

import json
from pathlib import Path

import pytest

import bench

GOLDEN = Path(__file__).resolve().parent / "golden"


def test_lab_counts():
    g = json.loads((GOLDEN / "lab_counts.json").read_text())
    assert bench.interactions(g["N"]) == g["pair_interactions"]
    assert bench.tile_global_loads(g["N"], g["p"]) == g["normalized_global_loads"]


def test_twenty_flops_per_pair():
    g = json.loads((GOLDEN / "flops_per_pair.json").read_text())
    parts = g["r_ij"] + g["dist_sqr"] + g["inv_dist_cube"] + g["s"] + g["accumulate"]
    assert parts == g["total"] == bench.FLOPS_PER_INTERACTION


def test_peak_from_unit_counts():
    # 256 CUs x 4 SIMDs x 16 lanes x 2 (FMA) x 2 (packed) x 2.4 GHz
    assert abs(256 * 4 * 16 * 2 * 2 * 2.4e9 / 1e12 - bench.FP32_VECTOR_PEAK_TFLOPS) < 0.1


def test_multi_gpu_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


@pytest.mark.parametrize("n,band,nshards", [(1, 512, 1), (1 << 20, 2048, 8), (3000, 512, 3),
                                            (20011, 512, 40), (5000, 1024, 5), (4096, 512, 8)])
def test_shard_interactions_add_up_to_n_squared(n, band, nshards):
    parts = [bench.shard_interactions(n, band, s, nshards) for s in range(nshards)]
    assert sum(parts) == n * n
    assert min(parts) > 0


@pytest.mark.parametrize("n,band,passes", [(1, 512, 1), (1 << 20, 2048, 1), (1 << 20, 2048, 3),
                                           (3000, 512, 1), (20011, 256, 1), (5000, 1024, 2)])
def test_pair_item_terms_cover_every_ordered_pair_once(n, band, passes):
    """Summed over the band ranges of all passes, the pair kernel's items hold every unordered
    pair of distinct-band bodies once and every same-band ordered pair once: one-sided terms
    plus twice the pairs is N^2, and the one-sided terms are the squared band sizes."""
    nb = (n + band - 1) // band
    edges = [q * nb // passes for q in range(passes + 1)]
    parts = [bench.pair_item_terms(n, band, a, b) for a, b in zip(edges, edges[1:])]
    diag = sum(p[0] for p in parts)
    off = sum(p[1] for p in parts)
    assert diag + 2 * off == n * n
    sizes = [min(band, n - b * band) for b in range(nb)]
    assert diag == sum(s * s for s in sizes)
    # the same split by shards (nbody_accel_shard's band ranges) counts the same
    assert sum(bench.shard_interactions(n, band, q, passes) for q in range(passes)) == n * n


def test_first_launch_flops_match_the_formulation():
    """The pair kernel's FP32 flops per launch: 30 per unordered pair and 21 per one-sided
    term with the potential (26 and 19 without); one-sided kernels 21 (19) per term."""

    class Plan:
        mode, band, passes, tpl, bcast = 2, 2048, 1, 8, 1

    n = 1 << 20
    w = bench.first_launch_work(n, Plan, True)
    assert w["interactions"] == n * n
    assert w["units"] == {"one_sided_terms": n * 2048, "pairs": (n * n - n * 2048) // 2}
    assert w["flops"] == 21 * n * 2048 + 30 * (n * n - n * 2048) // 2
    assert bench.first_launch_work(n, Plan, False)["flops"] == (19 * n * 2048
                                                                + 26 * (n * n - n * 2048) // 2)
    Plan.mode = 3
    assert bench.first_launch_work(4096, Plan, True)["flops"] == 21 * 4096 * 4096


def test_cpu_sample_is_the_protocol_set():
    idx, _ = bench.cpu_sample_targets(1 << 20)
    n = 1 << 20
    assert len(idx) == 65536 + 2048 and len(set(idx.tolist())) == len(idx)
    assert list(idx[:1024]) == list(range(1024)) and list(idx[-1024:]) == list(range(n - 1024, n))
    idx2, _ = bench.cpu_sample_targets(65536)
    assert list(idx2) == list(range(65536))


def test_near_roofline_counts_issued_flops():
    """The near-field line's roofline: 21 issued FP32 flops per one-sided term with the
    potential (19 without) over the event-timed kernel."""
    r = bench.near_roofline(10 ** 9, 10.0, True, "p2p")
    assert r["flops_per_launch"] == 21 * 10 ** 9
    assert abs(r["achieved"] - 2.1) < 1e-9 and r["unit"] == "TFLOP/s"
    assert abs(r["frac"] - round(2.1 / bench.FP32_VECTOR_PEAK_TFLOPS, 4)) < 1e-12
    assert bench.near_roofline(10 ** 9, 10.0, False, "p2p")["flops_per_launch"] == 19 * 10 ** 9


@pytest.mark.parametrize("dims,n,seed", [((3, 4, 5), 700, 1), ((1, 1, 1), 50, 2), ((6, 2, 1), 300, 3)])
def test_near_grid_pair_units_count_each_neighbour_pair_once(dims, n, seed):
    """The pair-symmetric near grid's units against brute force over the bodies: unordered
    pairs {i, j}, i != j, in neighbouring cells (cells differing by at most one per axis, same
    cell excluded), and one-sided self terms (ordered pairs in one cell, i = j included); twice
    the first plus the second is the one-sided near field's term count."""
    import numpy as np

    rng = np.random.default_rng(seed)
    lo, h = (-1.0, -1.0, -1.0), 0.4
    pos = np.zeros((n, 4), np.float32)
    pos[:, :3] = rng.uniform(-1.2, -1.0 + h * max(dims) + 0.2, size=(n, 3))
    pos[:, 3] = 1.0
    x = pos[:, :3].astype(np.float32)
    k = np.floor((x - np.asarray(lo, np.float32)) * (np.float32(1.0) / np.float32(h)))
    k = np.clip(k, 0, np.asarray(dims) - 1).astype(np.int64)
    cell = (k[:, 2] * dims[1] + k[:, 1]) * dims[0] + k[:, 0]
    pairs = self_terms = 0
    for i in range(n):
        for j in range(n):
            if cell[i] == cell[j]:
                self_terms += 1
            elif i < j and np.all(np.abs(k[i] - k[j]) <= 1):
                pairs += 1
    got = bench.near_grid_pair_units(pos, lo, h, dims)
    assert got == (pairs, self_terms)
    assert bench.near_grid_terms(pos, lo, h, dims) == 2 * pairs + self_terms


def test_near_roofline_pair_units():
    """The pair kernel's near-field roofline: 30 flops per unordered pair and 21 per self
    term with the potential (26 and 19 without)."""
    r = bench.near_roofline(0, 10.0, True, "p2p_sym", (10 ** 9, 10 ** 8))
    assert r["flops_per_launch"] == 30 * 10 ** 9 + 21 * 10 ** 8
    assert r["units_per_launch"] == {"pairs": 10 ** 9, "one_sided_terms": 10 ** 8}
    r0 = bench.near_roofline(0, 10.0, False, "p2p_sym", (10 ** 9, 10 ** 8))
    assert r0["flops_per_launch"] == 26 * 10 ** 9 + 19 * 10 ** 8
