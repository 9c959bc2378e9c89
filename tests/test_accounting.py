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
