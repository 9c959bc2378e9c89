"""Several host threads calling the library at once, on one shared stream and on a stream each,
while the cached scratch areas grow between calls: every result equals the one-thread result
bit for bit (results are deterministic, so any mix-up of scratch between calls would show)."""

from __future__ import annotations

import threading

import numpy as np
import pytest

import workloads
from gpu_util import to_dev

pytestmark = pytest.mark.gpu

# small mode (no scratch), pair bands in one pass with growing slot arrays, and a step loop
SIZES = [3000, 9000, 24000, 70001, 131072]
THREADS = 4


@pytest.fixture(scope="module")
def nb():
    import direct_all_pairs_amd

    return direct_all_pairs_amd


def _inputs():
    out = {}
    for n in SIZES:
        pos, vel = workloads.random_bodies(n, seed=900 + n)
        out[n] = (to_dev(pos), to_dev(vel))
    return out


def _run(nb, n, pos, vel, stream, acc, pot, pos_out):
    """One evaluation and a two-step Euler loop on copies, all enqueued on `stream`."""
    import torch

    with torch.cuda.stream(stream):
        nb.nbody_accel(pos, n, 1e-4, acc, pot, stream=stream)
        pos_out.copy_(pos)
        v = vel.clone()
        nb.nbody_step(pos_out, v, n, 1e-3, 1e-4, 2, stream=stream)


@pytest.mark.parametrize("shared", [True, False], ids=["one_stream", "stream_each"])
def test_threads_match_single_thread(nb, shared):
    import torch

    data = _inputs()
    torch.cuda.synchronize()
    # one-thread reference, each size on a fresh scratch area
    ref = {}
    s0 = torch.cuda.Stream()
    for n in SIZES:
        nb.nbody_release_workspace()
        pos, vel = data[n]
        acc = torch.empty((n, 4), device="cuda")
        pot = torch.empty((n,), device="cuda")
        po = torch.empty_like(pos)
        _run(nb, n, pos, vel, s0, acc, pot, po)
        torch.cuda.synchronize()
        ref[n] = (acc.cpu().numpy(), pot.cpu().numpy(), po.cpu().numpy())

    nb.nbody_release_workspace()  # the threads start from empty scratch and grow it
    streams = [torch.cuda.Stream()] * THREADS if shared else [torch.cuda.Stream() for _ in range(THREADS)]
    outs = {}
    for t in range(THREADS):
        for n in SIZES:
            pos = data[n][0]
            outs[t, n] = (torch.full((n, 4), np.nan, device="cuda"),
                          torch.full((n,), np.nan, device="cuda"), torch.empty_like(pos))
    torch.cuda.synchronize()
    errors = []

    def work(t):
        try:
            order = SIZES[t % len(SIZES):] + SIZES[:t % len(SIZES)]  # a different growth order each
            for n in order:
                pos, vel = data[n]
                _run(nb, n, pos, vel, streams[t], *outs[t, n])
        except Exception as e:  # reported after the join
            errors.append(f"thread {t}: {e!r}")

    threads = [threading.Thread(target=work, args=(t,)) for t in range(THREADS)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for (t, n), (acc, pot, po) in outs.items():
        ra, rp, rpos = ref[n]
        assert np.array_equal(acc.cpu().numpy(), ra), f"thread {t} N={n} acceleration"
        assert np.array_equal(pot.cpu().numpy(), rp), f"thread {t} N={n} potential"
        assert np.array_equal(po.cpu().numpy(), rpos), f"thread {t} N={n} step positions"


def test_scratch_release_and_growth_with_queued_work(nb):
    """Scratch freed or grown while work that uses it is still queued: nbody_release_workspace
    and a larger call right behind a smaller one free the old block only after the device has
    finished with it, so every result equals its one-call-at-a-time reference bit for bit."""
    import torch

    sizes = [70001, 9000, 200003]
    data = {n: to_dev(workloads.random_bodies(n, seed=950 + n)[0]) for n in sizes}
    s = torch.cuda.Stream()
    ref = {}
    for n in sizes:
        nb.nbody_release_workspace()
        acc = torch.empty((n, 4), device="cuda")
        pot = torch.empty((n,), device="cuda")
        nb.nbody_accel(data[n], n, 1e-4, acc, pot, stream=s)
        torch.cuda.synchronize()
        ref[n] = (acc.cpu().numpy(), pot.cpu().numpy())

    nb.nbody_release_workspace()
    out = {n: (torch.full((n, 4), np.nan, device="cuda"), torch.full((n,), np.nan, device="cuda"))
           for n in sizes}
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        nb.nbody_accel(data[70001], 70001, 1e-4, *out[70001], stream=s)
        nb.nbody_release_workspace()  # the 70001-body evaluation may still be running
        nb.nbody_accel(data[9000], 9000, 1e-4, *out[9000], stream=s)
        nb.nbody_accel(data[200003], 200003, 1e-4, *out[200003], stream=s)  # grows the block
    torch.cuda.synchronize()
    for n in sizes:
        acc, pot = out[n]
        assert np.array_equal(acc.cpu().numpy(), ref[n][0]), f"N={n} acceleration"
        assert np.array_equal(pot.cpu().numpy(), ref[n][1]), f"N={n} potential"


@pytest.mark.parametrize("shared", [True, False], ids=["one_stream", "stream_each"])
def test_near_field_threads_match_single_thread(nb, shared):
    """nbody_near_tree (which waits on its stream part-way and keeps three scratch areas per
    stream) and nbody_near_grid from several threads at once, sizes in a different order per
    thread: every result equals the one-thread result bit for bit."""
    import torch

    sizes = [(5000, 16), (40000, 64), (150001, 32)]
    data = {n: to_dev(workloads.random_bodies(n, seed=970 + n)[0]) for n, _ in sizes}
    grid = ((-1.0, -1.0, -1.0), 0.25, (8, 8, 8))

    def run(n, leaf, stream, acc_t, pot_t, acc_g, pot_g):
        with torch.cuda.stream(stream):
            nb.nbody_near_tree(data[n], n, 1e-4, leaf, acc_t, pot_t, None, stream=stream)
            nb.nbody_near_grid(data[n], n, 1e-4, *grid, acc_g, pot_g, stream=stream)

    def bufs(n):
        return tuple(torch.full(shape, np.nan, device="cuda")
                     for shape in ((n, 4), (n,), (n, 4), (n,)))

    s0 = torch.cuda.Stream()
    ref = {}
    for n, leaf in sizes:
        nb.nbody_release_workspace()
        b = bufs(n)
        run(n, leaf, s0, *b)
        torch.cuda.synchronize()
        ref[n] = [x.cpu().numpy() for x in b]
    nb.nbody_release_workspace()
    streams = [torch.cuda.Stream()] * THREADS if shared else [torch.cuda.Stream() for _ in range(THREADS)]
    outs = {(t, n): bufs(n) for t in range(THREADS) for n, _ in sizes}
    torch.cuda.synchronize()
    errors = []

    def work(t):
        try:
            order = sizes[t % len(sizes):] + sizes[:t % len(sizes)]
            for n, leaf in order:
                run(n, leaf, streams[t], *outs[t, n])
        except Exception as e:  # reported after the join
            errors.append(f"thread {t}: {e!r}")

    threads = [threading.Thread(target=work, args=(t,)) for t in range(THREADS)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for (t, n), b in outs.items():
        for what, x, r in zip(("tree acc", "tree pot", "grid acc", "grid pot"), b, ref[n]):
            assert np.array_equal(x.cpu().numpy(), r), f"thread {t} N={n} {what}"
