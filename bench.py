"""Throughput benchmark of the direct all-pairs softened-gravity path on one MI355X.

Default workload: N = 1,048,576 bodies, uniform cube [-1,1]^3, masses uniform in
[0.5, 1.5]/N, eps2 = 1e-4, one acceleration + potential evaluation per step
(nbody_accel through the C ABI), inputs resident in HBM.

Prints one JSON line:
  value    = whole-job body-body interactions per second, in G/s (N^2 per step)
  gflops_at_20, pct_fp32_peak_at_20 = the metric's convention: 20 flop per
             interaction (the pair-routine count on the CSDN "Cuda Nbody笔记"
             page / GPU Gems 3 ch. 31) over the whole call
  roofline = the pair-term kernel alone (HIP events the library records around
             its launch, nbody_time_kernel) against the FP32 vector peak, with
             the FP32 flops its own formulation issues per launch (a symmetric
             pair 30, a one-sided term 21 with the potential; 26 and 19 without)
  cpu_baseline = the fp64 oracle on the host cores: every target for N <= 67584,
             else 65,536 random targets plus the first and last 1024 bodies
             against all N sources, with the full-N time extrapolated
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
if str(ROOT) not in sys.path:
    sys.path.insert(0, str(ROOT))

FLOPS_PER_INTERACTION = 20  # 3 (r_ij) + 6 (|r|^2 + eps^2) + 4 (inv^3) + 1 (m inv^3) + 6 (a +=)
FP32_VECTOR_PEAK_TFLOPS = 157.3  # MI355X: 256 CU x 2.4 GHz x 256 FP32 flop/clk/CU (packed FMA)
# FP32 flops (FMA = 2, v_rsq_f32 = 1) of one pair term as the kernels write it:
#  one-sided term (tiles and small-N kernels, the diagonal items of the pair kernel):
#    3 sub (d), 3 FMA (|d|^2 + eps2), rsq, 3 mul (m / r^3), 3 FMA (a) [+ 1 FMA (p)]
#  unordered pair of the pair kernel (applied to both bodies):
#    3 sub, 3 FMA, rsq, 2 mul (inv^3), 2 mul (m_i / r^3, m_j / r^3), 6 FMA (a_i, a_j)
#    [+ 2 FMA (p_i, p_j)]
FLOPS_ONE_SIDED = {True: 21, False: 19}   # keyed by "with the potential"
FLOPS_PAIR = {True: 30, False: 26}
PROFILE_TRAFFIC = ROOT / "profiles" / "accel_cube1m_traffic.json"
KERNEL_SOURCES = [ROOT / "direct_all_pairs_amd" / "csrc" / "kernels.hip",
                  ROOT / "direct_all_pairs_amd" / "csrc" / "kernels.h"]


def interactions(n: int) -> int:
    """Pair interactions per evaluation: every target against every source, self pairs
    included (N^2), as the GPU Gems 3 ch. 31 study page's lab counts them."""
    return n * n


def pair_item_terms(n: int, band: int, a0: int, a1: int) -> tuple[int, int]:
    """(one-sided terms, unordered pairs) of the pair kernel's items (A, d) for bands A in
    [a0, a1): the diagonal item (A, 0) takes |A|^2 one-sided terms (self pairs included), item
    (A, d), d = 1 .. nb/2, the |A| |B| pairs with B = (A + d) mod nb, where for even nb the
    item d = nb/2 exists only for A < nb/2."""
    import numpy as np

    nb = (n + band - 1) // band
    size = np.minimum(band, n - band * np.arange(nb, dtype=np.int64))
    a = np.arange(a0, a1, dtype=np.int64)
    diag = int(np.sum(size[a] ** 2))
    off = 0
    for d in range(1, nb // 2 + 1):
        own = a if not (2 * d == nb) else a[a < nb // 2]
        off += int(np.sum(size[own] * size[(own + d) % nb]))
    return diag, off


def first_launch_work(n: int, plan, pot: bool) -> dict:
    """The pair terms and FP32 flops of the first pair-term kernel launch of one evaluation
    (the launch nbody_time_kernel brackets): the whole evaluation, or pass 0 of a
    multi-pass pair plan."""
    mode = {1: "tiles", 2: "pairs", 3: "small"}[plan.mode]
    if mode == "pairs":
        nb = (n + plan.band - 1) // plan.band
        a1 = nb // max(1, plan.passes)  # pass 0: bands [0, floor(nb / passes))
        diag, off = pair_item_terms(n, plan.band, 0, a1)
        flops = FLOPS_ONE_SIDED[pot] * diag + FLOPS_PAIR[pot] * off
        name = f"accel_pairs<{plan.tpl}, {plan.band}, {str(pot).lower()}>"
        return {"kernel": name, "interactions": diag + 2 * off, "flops": flops,
                "units": {"one_sided_terms": diag, "pairs": off},
                "flops_per_unit": {"one_sided_term": FLOPS_ONE_SIDED[pot],
                                   "pair": FLOPS_PAIR[pot]}}
    if mode == "small":
        name = f"accel_small<{plan.tpl}, ...>"
    else:
        bcast = {1: "lds", 2: "scalar", 3: "readlane"}[plan.bcast]
        name = f"accel_{bcast}<{plan.tpl}, ...>"
    return {"kernel": name, "interactions": n * n, "flops": FLOPS_ONE_SIDED[pot] * n * n,
            "units": {"one_sided_terms": n * n},
            "flops_per_unit": {"one_sided_term": FLOPS_ONE_SIDED[pot]}}


def tile_global_loads(n: int, p: int) -> int:
    """Global body loads per evaluation with p-body shared tiles: N^2 / p."""
    return n * n // p


def code_tokens(text: str) -> str:
    """C++ source without comments and whitespace runs: what the compiler sees, so that a
    comment-only edit does not count as a kernel change (string literals hold no comment
    markers in these files)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(code_tokens(f.read_text()).encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel_hash: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken
    on the current kernel source; else None."""
    try:
        d = json.loads(PROFILE_TRAFFIC.read_text())
    except (OSError, ValueError):
        return None
    if d.get("kernel_source_hash") != kernel_hash:
        return None
    return d.get("hbm_bytes_per_launch")


def cpu_sample_targets(n: int) -> tuple[object, str]:
    """The oracle's targets for the CPU baseline: every body for N <= 67,584; above, 65,536
    distinct random bodies (seed 12345) from [1024, N - 1024) plus [0, 1024) and
    [N - 1024, N), against all N sources."""
    import numpy as np

    if n <= 65536 + 2048:
        return np.arange(n), f"all {n} targets"
    rng = np.random.default_rng(12345)
    mid = 1024 + rng.choice(n - 2048, 65536, replace=False)
    idx = np.concatenate([np.arange(1024), np.sort(mid), np.arange(n - 1024, n)])
    return idx, "65,536 random targets plus [0, 1024) and [N - 1024, N)"


def cpu_baseline(pos_h, eps2, gpu_acc=None, gpu_pot=None):
    """Time the fp64 oracle (as it stands) on the sample of cpu_sample_targets against all N
    sources; report its rate, the full-N time extrapolated from it, and, with the GPU's
    accelerations (and potentials) of the same workload, their largest error on the sample in
    units of the per-body bounds B_i (and P_i)."""
    import numpy as np

    import oracle

    n = pos_h.shape[0]
    threads = oracle.num_threads()
    idx, what = cpu_sample_targets(n)
    oracle.accel(pos_h, eps2, targets=np.arange(min(n, threads)))  # start the thread pool
    t0 = time.perf_counter()
    ref = oracle.accel(pos_h, eps2, targets=idx)
    t = time.perf_counter() - t0
    rate = len(idx) * n / t
    out = {
        "value": rate / 1e9,
        "unit": "G interactions/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{what} ({len(idx)} targets) x all {n} sources, fp64 acceleration + "
                  f"potential + bounds: {t:.1f} s measured",
        "full_n_seconds": n * t / len(idx),
        "full_n_seconds_is": "measured" if len(idx) == n else
                             "extrapolated from the sample's rate (N / sample targets x its time)",
    }
    if gpu_acc is not None:
        a = np.asarray(gpu_acc)[idx, :3].astype(np.float64)
        err = np.linalg.norm(a - ref["acc"], axis=1)
        out["gpu_max_err_over_B"] = float(np.max(err / ref["bound_a"]))
        if gpu_pot is not None:
            e_p = np.abs(np.asarray(gpu_pot)[idx].astype(np.float64) - ref["pot"])
            out["gpu_max_pot_err_over_P"] = float(np.max(e_p / ref["bound_p"]))
    return out


class ClockSampler:
    """Samples the GPU's shader clocks with `amd-smi metric -c --json` (a child process, one
    call after another) while the benchmark runs; each sample is the mean of the per-XCD gfx
    clocks in MHz. Nothing is sampled where amd-smi is missing or prints no clocks."""

    def __init__(self):
        import threading

        self.samples: list[float] = []
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    def _one(self):
        import subprocess

        r = subprocess.run(["amd-smi", "metric", "-c", "--json"], capture_output=True, text=True,
                           timeout=20)
        txt = r.stdout[r.stdout.find("{") if r.stdout.lstrip()[:1] != "[" else 0:]
        d = json.loads(txt)
        g = d[0] if isinstance(d, list) else d.get("gpu_data", [d])[0]
        clk = [v["clk"]["value"] for k, v in g["clock"].items()
               if k.startswith("gfx") and isinstance(v.get("clk"), dict)
               and isinstance(v["clk"].get("value"), (int, float))]
        return sum(clk) / len(clk) if clk else None

    def _run(self):
        while not self._stop.is_set():
            try:
                v = self._one()
            except Exception:
                return
            if v is not None and not self._stop.is_set():
                self.samples.append(float(v))
            self._stop.wait(0.2)

    @property
    def started(self) -> bool:
        return self._thread.ident is not None

    def __enter__(self):
        self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        self._thread.join(timeout=30)

    def summary(self, frac_at_nominal: float):
        if not self.samples:
            return None
        v = sorted(self.samples)
        med = v[len(v) // 2]
        return {"median_mhz": round(med), "samples": len(v),
                "source": "amd-smi metric -c, mean of the XCD gfx clocks, sampled from the end of "
                "the second warm-up call to the end of the timed steps",
                "roofline_frac_at_measured_sclk": round(frac_at_nominal * 2400.0 / med, 4)}


def copy_calibration(nbytes: int) -> int:
    """A plain copy of known size: reads and writes nbytes once per launch."""
    import torch

    n = nbytes // 16
    src = torch.ones((n, 4), dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n * 16, "launches": 2}), flush=True)
    return 0


def sweep(nb, w, pos, vel, acc, pot, args) -> int:
    """Every layout of the workload's call (nbody_accel_plan, or nbody_step_plan for the
    stepping workloads), HIP-event timed; fastest layout last. Sequentially (args.steps calls
    per layout after args.warmup), or with args.rounds > 0 round-robin: every layout is timed
    over args.steps calls once per round, so that clock drift falls on all layouts alike, and
    the median of the rounds is reported."""
    import torch

    n = w.n
    stepping = w.nsteps > 0 and args.workload != "disk4096"
    stream = torch.cuda.current_stream()
    split_opts = [0, 1, 2, 4, 8, 16, 32, 64, 128]
    layouts = [("lds", t, wg) for t in (1, 2, 4) for wg in (64, 128, 256, 512)]
    layouts += [(b, t, 256) for b in ("scalar", "readlane") for t in (1, 2, 4, 8)]
    layouts += [("pairs", 4, 256)]
    layouts += [("pairs", t, band) for t in (4, 8) for band in (512, 1024, 2048)]
    layouts += [("pairs", 8, 4096)]
    if n <= 65536:
        layouts += [("small", tw, 256) for tw in (4, 8, 16, 32)]
    if args.sweep_only != "all":
        keep = set()
        for m in args.sweep_only.split(","):
            keep |= set({"tiles": ("lds", "scalar", "readlane")}.get(m, (m,)))
        layouts = [lay for lay in layouts if lay[0] in keep]
    cases = []
    for bcast, tpl, wg in layouts:
        for splits in (split_opts if bcast == "lds" else [0]):
            if splits and (splits - 1) * wg >= n:  # some chunk would be empty
                continue
            if bcast == "pairs":
                plan = nb.make_plan(mode="pairs", band=wg, tpl=tpl)
            elif bcast == "small":
                plan = nb.make_plan(mode="small", tpl=tpl)
            else:
                plan = nb.make_plan(mode="tiles", bcast=bcast, tpl=tpl, splits=splits, wg=wg)
            cases.append((bcast, tpl, wg, splits, plan))

    def call(plan):
        if stepping:
            nb.nbody_step_plan(pos, vel, n, float(w.dt), float(w.eps2), w.nsteps, plan, stream)
        else:
            nb.nbody_accel_plan(pos, n, float(w.eps2), acc, pot, plan, stream)

    def timed(plan):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            call(plan)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    times = [[] for _ in cases]
    if args.rounds > 0:
        for c in cases:
            for _ in range(max(1, args.warmup)):
                call(c[4])
        torch.cuda.synchronize()
        for _ in range(args.rounds):
            for k, c in enumerate(cases):
                times[k].append(timed(c[4]))
    else:
        for k, c in enumerate(cases):
            for _ in range(max(1, args.warmup)):
                call(c[4])
            times[k].append(timed(c[4]))
    results = []
    evals = w.nsteps if stepping else 1
    for (bcast, tpl, wg, splits, plan), t in zip(cases, times):
        ms = sorted(t)[len(t) // 2]
        r = {"workload": args.workload, "N": n, "potential": pot is not None,
             "call": "nbody_step_plan" if stepping else "nbody_accel_plan",
             "bcast": bcast, "tpl": tpl, "wg": wg, "splits": splits or "auto",
             "ms": round(ms, 4), "us_per_eval": round(ms * 1e3 / evals, 3),
             "G_int_per_s": round(interactions(n) * evals / ms / 1e6, 2),
             "timing": f"median of {args.rounds} round-robin rounds" if args.rounds > 0
             else "sequential"}
        results.append(r)
        print(json.dumps(r), flush=True)
    best = max(results, key=lambda r: r["G_int_per_s"])
    print(json.dumps({"best": best, "auto_plan": nb.nbody_plan_for(n, pot is not None).as_dict()}),
          flush=True)
    return 0


def near_grid_counts(pos_h, lo, h, dims):
    """Bodies per cell, as an array indexed (z, y, x) (cells decided in float32, as the library
    decides them)."""
    import numpy as np

    x = pos_h[:, :3].astype(np.float32)
    inv = np.float32(1.0) / np.float32(h)
    k = np.floor((x - np.asarray(lo, np.float32)) * inv)
    k = np.clip(np.nan_to_num(k, nan=0.0), 0, np.asarray(dims) - 1).astype(np.int64)
    cnt = np.zeros(dims[::-1], np.int64)
    np.add.at(cnt, (k[:, 2], k[:, 1], k[:, 0]), 1)
    return cnt


def near_grid_terms(pos_h, lo, h, dims) -> int:
    """Pair terms of the grid near field: sum over cells of n_c times the bodies in its 27-cell
    neighbourhood."""
    import numpy as np

    cnt = near_grid_counts(pos_h, lo, h, dims)
    pad = np.pad(cnt, 1)
    nbr = sum(pad[1 + dz:1 + dz + dims[2], 1 + dy:1 + dy + dims[1], 1 + dx:1 + dx + dims[0]]
              for dz in (-1, 0, 1) for dy in (-1, 0, 1) for dx in (-1, 0, 1))
    return int(np.sum(cnt * nbr))


def near_grid_pair_units(pos_h, lo, h, dims) -> tuple[int, int]:
    """The pair-symmetric near-grid kernel's units: (unordered pairs of bodies in neighbouring
    cells, each evaluated once; one-sided terms of the cells with themselves, sum of n_c^2).
    Twice the pairs plus the self terms are the near field's pair terms."""
    import numpy as np

    cnt = near_grid_counts(pos_h, lo, h, dims)
    self_terms = int(np.sum(cnt * cnt))
    return (near_grid_terms(pos_h, lo, h, dims) - self_terms) // 2, self_terms


def near_roofline(terms: int, kernel_ms: float, pot: bool, kernel: str,
                  pairs: tuple[int, int] | None = None) -> dict:
    """The near-field kernel against the FP32 vector peak: its own flops per launch over the
    event-timed launch. One-sided: 21 per term with the potential, 19 without, as in the tile
    kernel. Pair-symmetric (pairs = (unordered pairs, self terms)): 30 (26) per pair and 21
    (19) per self term, as in the all-pairs pair kernel; padding lanes are not counted."""
    if pairs is not None:
        npair, nself = pairs
        flops = FLOPS_PAIR[pot] * npair + FLOPS_ONE_SIDED[pot] * nself
        achieved = flops / (kernel_ms * 1e-3) / 1e12
        return {"bound": "alu", "kernel": kernel, "achieved": round(achieved, 2),
                "peak": FP32_VECTOR_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / FP32_VECTOR_PEAK_TFLOPS, 4), "traffic": None,
                "flops_per_launch": flops,
                "units_per_launch": {"pairs": npair, "one_sided_terms": nself},
                "flops_per_unit": {"pair": FLOPS_PAIR[pot], "one_sided_term": FLOPS_ONE_SIDED[pot]},
                "launch_ms_mean": round(kernel_ms, 4)}
    flops = FLOPS_ONE_SIDED[pot] * terms
    achieved = flops / (kernel_ms * 1e-3) / 1e12
    return {"bound": "alu", "kernel": kernel, "achieved": round(achieved, 2),
            "peak": FP32_VECTOR_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(achieved / FP32_VECTOR_PEAK_TFLOPS, 4), "traffic": None,
            "flops_per_launch": flops, "units_per_launch": {"one_sided_terms": terms},
            "flops_per_unit": {"one_sided_term": FLOPS_ONE_SIDED[pot]},
            "launch_ms_mean": round(kernel_ms, 4)}


def near_cpu_baseline(ref_fn, n: int, acc, pot) -> dict:
    """Time the oracle's near field (ref_fn(targets) -> dict) on a fixed sample: 4096 random
    targets (seed 0) plus the first and last 256 bodies; report targets per second, the
    full-N time extrapolated from it, and the GPU's largest error on the sample in units of
    the per-body bounds."""
    import numpy as np

    import oracle

    rng = np.random.default_rng(0)
    idx = np.unique(np.concatenate([rng.integers(0, n, 4096), np.arange(min(256, n)),
                                    np.arange(max(0, n - 256), n)]))
    t0 = time.perf_counter()
    ref = ref_fn(idx)
    t = time.perf_counter() - t0
    a = np.asarray(acc)[idx, :3].astype(np.float64)
    out = {"value": round(len(idx) / t, 1), "unit": "targets/s", "cores": oracle.num_threads(),
           "kind": "oracle",
           "sample": f"4096 random targets (seed 0) + the first and last 256 ({len(idx)} "
                     f"targets), fp64 near field + bounds: {t:.2f} s measured",
           "full_n_seconds": n * t / len(idx),
           "full_n_seconds_is": "extrapolated from the sample's rate",
           "gpu_max_err_over_B": float(np.max(np.linalg.norm(a - ref["acc"], axis=1)
                                              / ref["bound_a"]))}
    if pot is not None:
        e_p = np.abs(np.asarray(pot)[idx].astype(np.float64) - ref["pot"])
        out["gpu_max_pot_err_over_P"] = float(np.max(e_p / ref["bound_p"]))
    return out


def near_grid_bench(nb, w, pos, args) -> int:
    """Time nbody_near_grid (binning, sort, near-field kernel, scatter) on a cubic grid of
    args.near_grid cells per axis over [-1, 1]^3; one JSON line (not the contract line)."""
    import torch

    d = args.near_grid
    lo, h, dims = (-1.0, -1.0, -1.0), 2.0 / d, (d, d, d)
    n = w.n
    kernel = {"auto": nb.NEAR_AUTO, "one-sided": nb.NEAR_ONE_SIDED,
              "pairs": nb.NEAR_PAIRS}[args.near_kernel]
    if kernel == nb.NEAR_AUTO:
        # the library's rule: pairs from 96 to 2048 bodies per cell, at least two cells per
        # compute unit, and its 14 slots of N records within 1/16 of device memory
        props = torch.cuda.get_device_properties(pos.device)
        kernel = (nb.NEAR_PAIRS if 96 * d ** 3 <= n <= 2048 * d ** 3
                  and d ** 3 >= 2 * props.multi_processor_count
                  and 14 * 16 * n <= props.total_memory // 16 else nb.NEAR_ONE_SIDED)
    acc = torch.empty_like(pos)
    pot = torch.empty(n, dtype=torch.float32, device=pos.device)
    stream = torch.cuda.current_stream()
    for _ in range(max(1, args.warmup)):
        nb.nbody_near_grid_kernel(pos, n, float(w.eps2), lo, h, dims, kernel, acc, pot, stream)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    ks = [torch.cuda.Event(enable_timing=True) for _ in range(2 * args.steps)]
    for e in ks:
        e.record(stream)
    e0.record(stream)
    for k in range(args.steps):
        nb.nbody_time_kernel(ks[2 * k], ks[2 * k + 1])
        nb.nbody_near_grid_kernel(pos, n, float(w.eps2), lo, h, dims, kernel, acc, pot, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    nb.nbody_time_kernel(None, None)
    ms = e0.elapsed_time(e1) / args.steps
    kms = sum(ks[2 * k].elapsed_time(ks[2 * k + 1]) for k in range(args.steps)) / args.steps
    terms = near_grid_terms(w.pos, lo, h, dims)
    line = {"workload": args.workload, "N": n, "dims": dims, "h": h,
            "bodies_per_cell": n / (d ** 3), "pair_terms": terms, "ms": round(ms, 4),
            "G_terms_per_s": round(terms / ms / 1e6, 2), "kernel_ms": round(kms, 4),
            "kernel_G_terms_per_s": round(terms / kms / 1e6, 2),
            "kernel": "pairs" if kernel == nb.NEAR_PAIRS else "one-sided",
            "roofline": (near_roofline(terms, kms, True, "p2p_sym_kernel (forward neighbour cells)",
                                       near_grid_pair_units(w.pos, lo, h, dims))
                         if kernel == nb.NEAR_PAIRS else
                         near_roofline(terms, kms, True, "p2p_kernel (grid neighbourhoods)"))}
    if args.cpu_budget > 0:
        import oracle

        line["cpu_baseline"] = near_cpu_baseline(
            lambda t: oracle.near_grid(w.pos, w.eps2, lo, h, dims, targets=t), n,
            acc.cpu().numpy(), pot.cpu().numpy())
    print(json.dumps({"near_grid": line}), flush=True)
    return 0


def near_tree_bench(nb, w, pos, args) -> int:
    """Time nbody_near_tree (bounds, keys, sort, leaves, lists, near-field kernel) with leaves
    of at most args.near_tree bodies; one JSON line (not the contract line). Each call waits
    once on the stream for the leaf count, so a call's time includes that round trip; the
    stats come from one extra call before the timed ones."""
    import torch

    leaf = args.near_tree
    n = w.n
    acc = torch.empty_like(pos)
    pot = torch.empty(n, dtype=torch.float32, device=pos.device)
    stream = torch.cuda.current_stream()
    st = nb.nbody_tree_stats()
    nb.nbody_near_tree(pos, n, float(w.eps2), leaf, acc, pot, st, stream)  # stats: one call
    for _ in range(max(1, args.warmup)):
        nb.nbody_near_tree(pos, n, float(w.eps2), leaf, acc, pot, None, stream)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    ks = [torch.cuda.Event(enable_timing=True) for _ in range(2 * args.steps)]
    for e in ks:
        e.record(stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for k in range(args.steps):
        nb.nbody_time_kernel(ks[2 * k], ks[2 * k + 1])
        nb.nbody_near_tree(pos, n, float(w.eps2), leaf, acc, pot, None, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / args.steps
    nb.nbody_time_kernel(None, None)
    ms = e0.elapsed_time(e1) / args.steps
    kms = sum(ks[2 * k].elapsed_time(ks[2 * k + 1]) for k in range(args.steps)) / args.steps
    terms = st.pair_terms
    line = {"workload": args.workload, "N": n, "leaf_size": leaf, **st.as_dict(),
            "bodies_per_leaf": round(n / st.leaves, 2), "ms": round(ms, 4),
            "wall_ms": round(wall, 4), "G_terms_per_s": round(terms / ms / 1e6, 2),
            "kernel_ms": round(kms, 4), "kernel_G_terms_per_s": round(terms / kms / 1e6, 2),
            "build_ms": round(ms - kms, 4),
            "roofline": near_roofline(terms, kms, True, "p2p_kernel (octree leaf lists)")}
    if args.cpu_budget > 0:
        import oracle

        line["cpu_baseline"] = near_cpu_baseline(
            lambda t: oracle.near_tree(w.pos, w.eps2, leaf, targets=t), n,
            acc.cpu().numpy(), pot.cpu().numpy())
    print(json.dumps({"near_tree": line}), flush=True)
    return 0


def shard_interactions(n: int, band: int, shard: int, nshards: int) -> int:
    """Interactions (ordered pairs, N^2 in all) that shard `shard` of `nshards` evaluates:
    its bands' diagonal items one-sided (self pairs included), the other items for both
    bodies of each pair."""
    nb = (n + band - 1) // band
    size = [min(band, n - b * band) for b in range(nb)]
    total = 0
    for a in range(shard * nb // nshards, (shard + 1) * nb // nshards):
        total += size[a] * size[a]
        for d in range(1, nb // 2 + 1):
            if 2 * d == nb and a >= nb // 2:
                continue
            total += 2 * size[a] * size[(a + d) % nb]
    return total


def shard_bench(nb, w, pos, args) -> int:
    """Time nbody_accel_shard for every shard of an evaluation split args.shard ways (one
    GPU's share of a multi-GPU evaluation, at its real shape) and nbody_shard_finish of one
    GPU's targets; one JSON line per shard and a summary line (not the contract line)."""
    import torch

    n, S = w.n, args.shard
    stream = torch.cuda.current_stream()
    band = nb.nbody_plan_for(n).band or 512
    plan = nb.make_plan(mode="pairs", band=band)
    out = torch.empty((S, n, 4), device=pos.device)
    acc = torch.empty((n // S + 1, 4), device=pos.device)
    pot = torch.empty((n // S + 1,), device=pos.device)
    per = []
    for s in range(S):
        def call():
            nb.nbody_accel_shard(pos, n, float(w.eps2), s, S, out[s], True, plan, stream)
        for _ in range(max(1, args.warmup)):
            call()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            call()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        it = shard_interactions(n, band, s, S)
        nbands = (n + band - 1) // band
        diag, off = pair_item_terms(n, band, s * nbands // S, (s + 1) * nbands // S)
        flops = FLOPS_ONE_SIDED[True] * diag + FLOPS_PAIR[True] * off
        r = {"workload": args.workload, "N": n, "band": band, "shard": s, "nshards": S,
             "ms": round(ms, 4), "interactions": it, "G_int_per_s": round(it / ms / 1e6, 1),
             "frac_fp32_peak": round(flops / ms / 1e9 / FP32_VECTOR_PEAK_TFLOPS, 4),
             "pct_fp32_peak_at_20": round(100 * FLOPS_PER_INTERACTION * it / ms / 1e9
                                          / FP32_VECTOR_PEAK_TFLOPS, 2)}
        per.append(r)
        print(json.dumps(r), flush=True)
    t0, t1 = 0, n // S
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    nb.nbody_shard_finish(out, n, S, t0, t1, acc, pot, stream)
    e0.record(stream)
    for _ in range(args.steps):
        nb.nbody_shard_finish(out, n, S, t0, t1, acc, pot, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    fin = e0.elapsed_time(e1) / args.steps
    worst = max(r["ms"] for r in per)
    print(json.dumps({"shard_summary": {
        "nshards": S, "max_shard_ms": worst, "min_shard_ms": min(r["ms"] for r in per),
        "finish_ms_per_gpu": round(fin, 4),
        "evaluation_G_int_per_s_if_shards_ran_in_parallel": round(
            interactions(n) / (worst + fin) / 1e6, 1),
        "note": "compute only: the exchange of the N-record parts between GPUs is not timed"}}),
        flush=True)
    return 0


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: 10; 200 for plummer65536, 2000 for disk4096, "
                         "100 for --near-grid and --near-tree, whose calls take milliseconds)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed warm-up steps (default: 2; 50 for plummer65536 and 200 for "
                         "disk4096, so that the shader clock has ramped up)")
    ap.add_argument("--workload", default="cube1m", choices=sorted(
        ["cube1m", "plummer65536", "disk4096", "cube2048_steps", "two_plummer300007"]),
        help="which of the five workloads to time (default: the N=1,048,576 cube)")
    ap.add_argument("--n", type=int, default=None, help="override N of the workload")
    ap.add_argument("--bcast", default=None, help="lds | scalar | readlane (default: auto plan)")
    ap.add_argument("--tpl", type=int, default=0)
    ap.add_argument("--splits", type=int, default=0)
    ap.add_argument("--no-pot", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=1.0,
                    help="0 skips cpu_baseline; any other value runs it (its sample is fixed: "
                         "every target up to N = 67584, else 65,536 random targets plus the "
                         "first and last 1024)")
    ap.add_argument("--sweep", action="store_true",
                    help="time every (broadcast, targets-per-lane, tile, splits) layout of the "
                         "workload's call and print one JSON line per layout (no contract line)")
    ap.add_argument("--sweep-only", default="all",
                    help="restrict --sweep to modes: all, or a comma list of tiles, pairs, small")
    ap.add_argument("--rounds", type=int, default=0,
                    help="--sweep: time the layouts round-robin over this many rounds (median "
                         "reported) instead of one after another")
    ap.add_argument("--near-grid", type=int, default=0, metavar="D",
                    help="only time nbody_near_grid on a D^3 grid over [-1, 1]^3 (near field; "
                         "prints its own JSON line, no contract line)")
    ap.add_argument("--near-kernel", default="auto", choices=["auto", "one-sided", "pairs"],
                    help="--near-grid: the near-field kernel (default: the library's choice)")
    ap.add_argument("--near-tree", type=int, default=0, metavar="LEAF",
                    help="only time nbody_near_tree with leaves of at most LEAF bodies (near "
                         "field over octree leaves; prints its own JSON line, no contract line)")
    ap.add_argument("--shard", type=int, default=0, metavar="S",
                    help="only time nbody_accel_shard for each of S shards of the workload's "
                         "evaluation (one GPU's share of an S-GPU split) and the merge of one "
                         "GPU's targets; prints its own JSON lines, no contract line")
    ap.add_argument("--no-clock", action="store_true",
                    help="do not sample the shader clock with amd-smi during the timed steps "
                         "(sampled only when a step takes 20 ms or more and --warmup >= 2)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES (twice) and exit; "
                         "used to scale the HBM byte counters of rocprofv3")
    args = ap.parse_args(argv)
    short = {"plummer65536": (200, 50), "disk4096": (2000, 200)}
    steps0, warm0 = short.get(args.workload, (10, 2)) if args.n is None else (10, 2)
    if args.near_grid or args.near_tree:
        steps0, warm0 = 100, 20  # a call takes milliseconds: warm the clock up first
    if args.steps is None:
        args.steps = steps0
    if args.warmup is None:
        args.warmup = warm0

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    if args.copy_calibration:
        return copy_calibration(args.copy_calibration)

    import direct_all_pairs_amd as nb
    import workloads

    dev = torch.device("cuda:0")
    w = workloads.make(args.workload, n=args.n)
    n = w.n
    stepping = w.nsteps > 0 and args.workload != "disk4096"
    want_pot = (not args.no_pot) and not stepping
    pos = torch.from_numpy(w.pos).to(dev)
    vel = torch.from_numpy(w.vel).to(dev)
    acc = torch.empty_like(pos)
    pot = torch.empty(n, dtype=torch.float32, device=dev) if want_pot else None
    plan = None
    if args.bcast or args.tpl or args.splits:
        plan = nb.make_plan(bcast=args.bcast or 0, tpl=args.tpl, splits=args.splits)
    eff = nb.nbody_plan_for(n, want_pot)
    if plan is not None:
        eff = nb.make_plan(bcast=plan.bcast or eff.bcast, tpl=plan.tpl or eff.tpl,
                           splits=plan.splits or eff.splits, mode=nb.MODE_TILES)
    stream = torch.cuda.current_stream()
    evals_per_step = w.nsteps if stepping else 1

    def one_step():
        if stepping:
            nb.nbody_step(pos, vel, n, float(w.dt), float(w.eps2), w.nsteps, stream)
        elif plan is None:
            nb.nbody_accel(pos, n, float(w.eps2), acc, pot, stream)
        else:
            nb.nbody_accel_plan(pos, n, float(w.eps2), acc, pot, plan, stream)

    if args.sweep:
        return sweep(nb, w, pos, vel, acc, pot, args)
    if args.near_grid:
        return near_grid_bench(nb, w, pos, args)
    if args.near_tree:
        return near_tree_bench(nb, w, pos, args)
    if args.shard:
        return shard_bench(nb, w, pos, args)

    diag0 = nb.diagnostics(pos, vel, float(w.eps2)) if stepping else None
    # The clock is sampled only when a step is long (>= 20 ms): for microsecond steps the
    # timed loop is bound by host enqueue, which a child process could disturb.
    clock = ClockSampler()
    for k in range(args.warmup):
        t_call = time.perf_counter()
        one_step()
        if k == 0:
            torch.cuda.synchronize()  # first call: scratch allocation, code loading
        elif k == 1:
            torch.cuda.synchronize()
            if not args.no_clock and time.perf_counter() - t_call >= 0.02:
                clock.__enter__()
    torch.cuda.synchronize()

    def events(k):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(k)]
        for e in ev:
            e.record(stream)  # torch creates the HIP event at its first record
        return ev

    # per step: the whole call (torch events around it) and its first pair-term kernel
    # launch alone (events the library records around that launch on the same stream)
    starts, ends = events(args.steps), events(args.steps)
    kstarts, kends = events(args.steps), events(args.steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        nb.nbody_time_kernel(kstarts[k], kends[k])
        starts[k].record(stream)
        one_step()
        ends[k].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    nb.nbody_time_kernel(None, None)
    if not args.no_clock and clock.started:
        clock.__exit__()
    ev_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    kern_ms = [s.elapsed_time(e) for s, e in zip(kstarts, kends)]

    n_int = interactions(n) * evals_per_step
    ms_per_step = wall * 1e3 / args.steps
    value = n_int * args.steps / wall / 1e9
    launch_s = float(np.mean(kern_ms)) / 1e3
    work = first_launch_work(n, eff, want_pot)
    achieved_tflops = work["flops"] / launch_s / 1e12
    conv_tflops = FLOPS_PER_INTERACTION * work["interactions"] / launch_s / 1e12
    khash = kernel_source_hash()
    traffic = measured_traffic(khash) if args.workload == "cube1m" and want_pot else None
    what = (f"{w.nsteps} Euler steps per call (nbody_step)" if stepping else
            ("acceleration + potential" if want_pot else "acceleration") +
            ", one evaluation per step (nbody_accel)")

    out = {
        "metric": "G body-body interactions/s & FP32 GFLOPS (20 flop/int) at N=1M, % of FP32 peak",
        "value": round(value, 3),
        "unit": "G interactions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{args.workload}: {workloads.CONFIGS[args.workload]['desc']}; timed: {what}",
            "N": n,
            "eps2": float(w.eps2),
            "potential": want_pot,
            "plan": eff.as_dict(),
            "device": torch.cuda.get_device_name(dev),
        },
        "gflops_at_20": round(FLOPS_PER_INTERACTION * value, 1),
        "pct_fp32_peak_at_20": round(100 * FLOPS_PER_INTERACTION * value / 1e3
                                     / FP32_VECTOR_PEAK_TFLOPS, 2),
        "sclk": clock.summary(achieved_tflops / FP32_VECTOR_PEAK_TFLOPS),
        "roofline": {
            "bound": "alu",
            "achieved": round(achieved_tflops, 3),
            "peak": FP32_VECTOR_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved_tflops / FP32_VECTOR_PEAK_TFLOPS, 4),
            "traffic": traffic,
            "kernel": work["kernel"],
            "timed": "the first pair-term kernel launch of each call, HIP events recorded by "
                     "the library on the launch stream (nbody_time_kernel)",
            "flops_per_launch": work["flops"],
            "units_per_launch": work["units"],
            "flops_per_unit": work["flops_per_unit"],
            "launch_ms_mean": round(launch_s * 1e3, 4),
            "call_ms_mean": round(float(np.mean(ev_ms)), 4),
            "achieved_at_20_flop_convention": round(conv_tflops, 3),
            "frac_at_20_flop_convention": round(conv_tflops / FP32_VECTOR_PEAK_TFLOPS, 4),
            "kernel_source_hash": khash,
        },
    }
    if stepping:
        # conserved quantities before the warm-up and after the timed steps, on the GPU
        # (nbody_diagnostics; outside the timed region)
        diag1 = nb.diagnostics(pos, vel, float(w.eps2))
        e0, e1 = diag0["total"], diag1["total"]
        out["config"]["energy_drift"] = {
            "steps": (args.warmup + args.steps) * w.nsteps,
            "relative": (e1 - e0) / abs(e0) if e0 else None,
            "momentum_change": [b - a for a, b in zip(diag0["momentum"], diag1["momentum"])],
        }
    if args.cpu_budget > 0:
        # the GPU results of the last timed evaluation, checked on the oracle's sample
        gpu_acc = acc.cpu().numpy() if not stepping else None
        gpu_pot = pot.cpu().numpy() if (pot is not None and not stepping) else None
        out["cpu_baseline"] = cpu_baseline(w.pos, w.eps2, gpu_acc, gpu_pot)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
