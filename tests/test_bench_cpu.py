"""Host-side behaviour of bench.py that needs no GPU: the one-GPU contract, and the
source hashing that keys the recorded HBM-traffic figures to each kernel's code."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and not r.stdout.strip()


def test_code_hash_ignores_comments_and_whitespace_only():
    src = "int f(int a) {\n    // add one\n    return a + 1; /* done */\n}\n"
    same = "int f(int a) { return a + 1; }  // reformatted, new comment\n"
    other = "int f(int a) {\n    // add one\n    return a + 2; /* done */\n}\n"
    assert bench.code_hash(src) == bench.code_hash(same)
    assert bench.code_hash(src) != bench.code_hash(other)


def test_every_traffic_record_names_a_known_kernel_and_matches_its_code():
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
        rec = json.load(f)
    for kernel, workloads in rec.items():
        assert kernel in bench.KERNEL_SOURCES, kernel
        for workload, r in workloads.items():
            assert r["hbm_bytes_per_launch"] > 0 and r["algorithmic_bytes_per_launch"] > 0
            # a record whose hash differs from the current code reads as absent
            got = bench.recorded_traffic(kernel, workload)
            assert got is None or got == r["hbm_bytes_per_launch"]


def test_a_changed_kernel_voids_its_record(monkeypatch):
    monkeypatch.setattr(bench, "source_hash", lambda kernel: "0" * 16)
    assert bench.recorded_traffic("k_adamw", "adamw_2p28_f16") is None


def test_tile_traffic_model_closed_forms():
    # M = K = N = 8192: 32 x 32 tiles per product, 128 per XCD; the 32 tiles an XCD
    # runs together are 4 tile rows x 8 tile columns, i.e. 12 panels of 256 rows
    # over the 8192-long reduction (4 MiB each) per 32 tiles
    M = K = N = 8192
    panel = 256 * 8192 * 2
    per_product = (1024 // 32) * 12 * panel
    out = 2 * M * K + 4 * K * N
    assert bench.lin_bwd_tiled_bytes(M, K, N) == 2 * per_product + out
    # one tile at a time per XCD shares nothing: two panels per tile
    assert bench.lin_bwd_tiled_bytes(M, K, N, cus_per_xcd=1) == 2 * 1024 * 2 * panel + out
    # one tile per product: each product reads its two operands once, so G is read
    # twice (once per product) and everything else as in the algorithmic bytes
    assert bench.lin_bwd_tiled_bytes(256, 256, 256) == bench.lin_bwd_min_bytes(256, 256, 256) + 2 * 256 * 256


def test_tile_traffic_model_rotation_splits_sharing():
    # rows 32 KiB apart (N = 16384): tiles of the four rotation groups (by tile
    # column) read the dX panels from different starting slabs, so an XCD's 16 dX
    # tiles (2 tile rows x 8 columns for a rotated job) fetch 2 x 4 + 8 panels instead
    # of 2 + 8
    M, K, N = 4096, 2048, 16384
    dx_tiles = (M // 256) * (K // 256)          # 128: 16 per XCD, fewer than 32
    assert dx_tiles % 8 == 0
    rotated = bench.lin_bwd_tiled_bytes(M, K, N)
    plain = bench.lin_bwd_tiled_bytes(M, K, N - 8)   # same tiles, no rotation
    assert rotated > plain
