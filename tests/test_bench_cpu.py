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
