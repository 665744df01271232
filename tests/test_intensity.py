"""The bench's roofline model reproduces the worked example the pages print.

"GPU 如何训练模型：从算子到 Kernel", section "Roofline：先判断“算不动”还是“搬不动”":
with bf16 and K = N = 4096, the ideal arithmetic intensity 2MKN / (b(MK+KN+MN))
is about 31.5 FLOP/B at M = 32 and 1024 FLOP/B at M = 2048 (fixture
tests/golden/intensity.json).
"""
import json
import os

import bench


def test_intensity_matches_the_pages_worked_example(golden_dir):
    data = json.load(open(os.path.join(golden_dir, "intensity.json")))
    for c in data["cases"]:
        got = bench.ideal_intensity(c["M"], c["K"], c["N"], c["bytes_per_elem"])
        assert abs(got - c["flop_per_byte"]) <= c["printed_precision"], (c, got)


def test_flop_and_byte_counts():
    assert bench.lin_bwd_flops(2048, 4096, 4096) == 4 * 2048 * 4096 * 4096
    # X, W, G read (bf16), dX written (bf16), dW written (fp32)
    assert bench.lin_bwd_min_bytes(32, 4096, 4096) == 2 * (32 * 4096 * 2 + 4096 * 4096) \
        + 2 * 32 * 4096 + 4 * 4096 * 4096
    assert bench.ADAMW_BYTES_16BIT_GRAD == 2 + 4 * 3 + 4 * 3


def test_multi_gpu_request_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err
