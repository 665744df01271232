"""lin_bwd's host-side sizing decisions (csrc/dispatch.h), built with g++ and checked on the
CPU: the launch-length model against a plain tile-by-tile simulation, the dX range counts
against the fastest counts measured on the GPU with the count forced (the sweeps listed in
dispatch.h), the invariants every range count must keep (partials within the workspace,
ranges of whole 64-element pairs covering the reduction), the limits of the one-launch
small-M pair and of the small-M dX that sums whole reductions (no split partials).
"""
import heapq
import os
import shutil
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "linear_layer_backward_bwd_amd", "csrc")
CAP = 1 << 24            # dX partial floats in a workspace (64 MiB)
SMALL_CAP = 1 << 23      # ... of which the small-M kernels' splits use at most this
CUS, FIXED = 256, 4


@pytest.fixture(scope="module")
def probe(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not found")
    exe = str(tmp_path_factory.mktemp("dispatch") / "dispatch_probe")
    subprocess.run([gxx, "-std=c++17", "-O2", "-Wall", "-Werror", "-I", CSRC,
                    os.path.join(ROOT, "tests", "native", "dispatch_probe.cpp"), "-o", exe], check=True)

    def ask(lines):
        out = subprocess.run([exe], input="\n".join(lines) + "\n", capture_output=True, text=True, check=True)
        return [list(map(int, l.split())) for l in out.stdout.strip().splitlines()]
    return ask


def cdiv(a, b):
    return -(-a // b)


def simulate(jobs):
    """Tile-by-tile list schedule: each tile, in launch order, on the CU that frees first."""
    free = [0] * CUS
    heapq.heapify(free)
    end = 0
    for n, slabs in jobs:
        for _ in range(n):
            t = heapq.heappop(free) + slabs + FIXED
            end = max(end, t)
            heapq.heappush(free, t)
    return end


def test_launch_span_closed_forms(probe):
    cases = [(n, l) for n in (1, 255, 256, 257, 512, 1000) for l in (1, 64, 128)]
    got = probe(["span %d %d 0 0" % (n, l) for n, l in cases])
    for (n, l), (g,) in zip(cases, got):
        assert g == cdiv(n, CUS) * (l + FIXED), (n, l)
    # the M = 2048 launch: 128 dX tiles of 128 slabs, then 256 dW tiles of 64
    assert probe(["span 128 128 256 64"]) == [[2 * (64 + FIXED)]]


def test_launch_span_matches_a_tile_by_tile_simulation(probe):
    rng = np.random.default_rng(5)
    cases = [(int(rng.integers(0, 700)), int(rng.integers(1, 300)), int(rng.integers(0, 700)), int(rng.integers(1, 300)))
             for _ in range(200)]
    got = probe(["span %d %d %d %d" % c for c in cases])
    for c, (g,) in zip(cases, got):
        assert g == simulate([(c[0], c[1]), (c[2], c[3])]), c


def tile_query(M, K, N, both=True, cap=CAP):
    ntx = cdiv(M, 256) * cdiv(K, 256)
    ntw = cdiv(K, 256) * cdiv(N, 256) if both else 0
    return "tile %d %d %d %d %d %d %d" % (M, K, ntx, N, ntw, M if both else 0, cap)


# (M, K, N): the range count that measured fastest with the count forced (µs per call,
# both products, calls back to back on cold inputs; the sweeps dispatch.h lists)
MEASURED_BEST = [((1800, 4096, 4096), 1), ((1959, 2048, 2048), 1), ((200, 4096, 4096), 8),
                 ((1000, 520, 4104), 8), ((160, 2048, 2048), 8), ((2048, 1024, 16384), 4),
                 ((549, 8192, 1024), 1), ((200, 2048, 4104), 16), ((2048, 4096, 4096), 1)]


def test_tile_ranges_pick_the_fastest_measured_count(probe):
    got = probe([tile_query(M, K, N) for (M, K, N), _ in MEASURED_BEST])
    for ((M, K, N), best), (g,) in zip(MEASURED_BEST, got):
        assert g == best, (M, K, N, g)


def test_tile_ranges_keep_their_invariants(probe):
    rng = np.random.default_rng(9)
    shapes = [(int(rng.integers(1, 2049)), int(rng.integers(8, 20000)), int(rng.integers(8, 20000)),
               bool(rng.random() < 0.8), int(rng.choice([CAP, CAP // 7, 0]))) for _ in range(400)]
    sx = [g for (g,) in probe([tile_query(*s) for s in shapes])]
    lens = probe(["tlen %d %d" % (s[2], x) for s, x in zip(shapes, sx)])
    for (M, K, N, both, cap), x, (splits, ln) in zip(shapes, sx, lens):
        assert x in (1, 2, 4, 8, 16), x
        assert x * M * K <= max(cap, M * K), (M, K, N, x)      # one range needs no partials
        if x > 1:
            assert cdiv(N, 32) // x >= 8 - 1, (M, K, N, x)     # ranges of at least about 8 slabs
        assert ln % 64 == 0 and 1 <= splits <= x
        assert (splits - 1) * ln < N <= splits * ln            # the ranges cover the reduction once
        assert splits * M * K <= max(cap, M * K)


def test_small_m_splits_keep_their_invariants(probe):
    rng = np.random.default_rng(4)
    cases = []
    for _ in range(400):
        M, K, N = int(rng.integers(1, 1025)), int(rng.integers(8, 20000)), int(rng.integers(1, 20000))
        chunk = int(rng.choice([128, 256]))
        units = cdiv(K, 64) * cdiv(M, 256)
        cases.append((N, chunk, units, M, K, int(rng.choice([min(CAP, SMALL_CAP), 0]))))
    got = probe(["red %d %d %d %d %d %d" % c for c in cases])
    for (N, chunk, units, M, K, cap), (splits, ln) in zip(cases, got):
        assert 1 <= splits <= 16
        assert ln % chunk == 0 and (splits - 1) * ln < N <= splits * ln
        if cap == 0:
            assert splits == 1
        else:
            assert splits == 1 or splits * M * K <= cap
        # toward one block per CU: more splits only while the blocks are fewer than the CUs
        assert splits == 1 or (splits - 1) * units < CUS


def test_small_m_pair_limits(probe):
    cases = [((64, 4096, 4096), 1), ((65, 4096, 4096), 0), ((1, 8192, 4096), 1), ((1, 8200, 4096), 0),
             ((28, 2056, 8192), 1), ((32, 4096, 8192), 0), ((32, 1024, 8200), 0), ((12, 8192, 8192), 0),
             ((48, 2048, 16384), 0), ((16, 16384, 2048), 1), ((64, 8, 264), 1)]
    got = probe(["pair %d %d %d" % c for c, _ in cases])
    for (c, want), (g,) in zip(cases, got):
        assert g == want, c


def test_small_m_whole_reduction_limits(probe):
    cases = [((16, 1024, 2048), 1), ((17, 1024, 2048), 0), ((1, 1024, 1024), 1), ((16, 2056, 1024), 0),
             ((8, 4096, 4096), 0), ((16, 512, 2048), 1), ((16, 512, 2056), 0), ((16, 512, 4096), 0),
             ((4, 4096, 256), 1), ((4, 4096, 248), 0), ((4, 504, 2016), 0), ((3, 16, 8), 0),
             ((16, 8, 262144), 0)]
    got = probe(["r16 %d %d %d" % c for c, _ in cases])
    for (c, want), (g,) in zip(cases, got):
        assert g == want, c
