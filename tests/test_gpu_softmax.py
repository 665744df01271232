"""GPU parity of softmax_bwd (dX = P·(dY − Σ P·dY) per row) against the CPU oracle.

Bar (written in gpu_util): every element within softmax_bound — the first-order
error of an fp32 dot product over the row plus one rounding for the difference
and the product, and for bf16 output half an ulp of the result — and the
relative Frobenius error within SM_RELF.
"""
import numpy as np
import pytest
import torch

import linear_layer_backward_bwd_amd as lb
import oracle
import synth
from gpu_util import SM_RELF, bits, relf, softmax_bound

pytestmark = pytest.mark.gpu
DEV = "cuda"
TORCH = {"f32": torch.float32, "bf16": torch.bfloat16}


def place(t, offset):
    buf = torch.empty(t.numel() + offset, dtype=t.dtype, device=DEV)
    v = buf[offset:].view(t.shape)
    v.copy_(t.to(DEV))
    return v


def gpu_dx(P, dY, offset=0, inplace=None):
    Pg, Yg = place(P, offset), place(dY, offset)
    if inplace == "dY":
        out = Yg
    elif inplace == "P":
        out = Pg
    else:
        out = place(torch.full(P.shape, float("nan"), dtype=P.dtype), offset)
    lb.softmax_bwd(Pg, Yg, out)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


def check(got, P, dY, dtype):
    Pb, Yb = synth.bits(P.cpu()), synth.bits(dY.cpu())
    ref = oracle.softmax_bwd(Pb, Yb, dtype)
    cols = P.shape[1]
    bound = softmax_bound(oracle.decode(Pb, dtype), oracle.decode(Yb, dtype), cols, dtype)
    assert not np.isnan(got).any()
    err = np.abs(got - ref)
    assert (err <= bound + 1e-38).all(), float(np.max(err - bound))
    assert relf(got, ref) <= SM_RELF[dtype], relf(got, ref)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("rows,cols", [(1, 1), (5, 3), (7, 4), (3, 7), (33, 64), (9, 255), (9, 256),
                                       (9, 257), (20, 512), (17, 1000), (64, 2048), (5, 2049),
                                       (6, 4095), (8, 4096), (4, 4097), (3, 10000), (2, 65539)])
def test_matches_oracle(dtype, rows, cols):
    P, dY = synth.softmax_case(rows, cols, dtype, seed=rows * 131 + cols)
    check(gpu_dx(P, dY), P, dY, dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("offset", [1, 3])
@pytest.mark.parametrize("cols", [200, 2048, 6000])
def test_misaligned(dtype, offset, cols):
    P, dY = synth.softmax_case(11, cols, dtype, seed=offset + cols)
    check(gpu_dx(P, dY, offset=offset), P, dY, dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("inplace", ["dY", "P"])
@pytest.mark.parametrize("cols", [1000, 2048, 5000])
def test_in_place(dtype, inplace, cols):
    P, dY = synth.softmax_case(13, cols, dtype, seed=cols)
    check(gpu_dx(P, dY, inplace=inplace), P, dY, dtype)


def test_sharp_and_uniform_rows():
    """Near one-hot rows (logits of std 30) and exactly uniform rows."""
    P, dY = synth.softmax_case(64, 2048, "bf16", z_std=30.0, seed=3)
    check(gpu_dx(P, dY), P, dY, "bf16")
    U = torch.full((8, 1024), 1.0 / 1024, dtype=torch.float32)
    dY = synth.normal((8, 1024), 1.0, synth._gen(4))
    check(gpu_dx(U, dY), U, dY, "f32")


def test_empty():
    P = torch.empty(0, 16, device=DEV)
    lb.softmax_bwd(P, P)
    P = torch.empty(5, 0, device=DEV)
    lb.softmax_bwd(P, P)
    torch.cuda.synchronize()


def test_repeatable_bit_for_bit():
    P, dY = synth.softmax_case(4096, 2048, "bf16", seed=5, device=DEV)
    a = lb.softmax_bwd(P, dY)
    b = lb.softmax_bwd(P, dY)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_attention_workload_full():
    """8 x 32 heads x 2048 rows of 2048 probabilities (bf16): every row, in chunks of rows
    (the per-element bound in each chunk, the relative Frobenius error over the whole)."""
    rows, cols = synth.SOFTMAX_ROWS, synth.SOFTMAX_COLS
    P, dY = synth.softmax_case(rows, cols, "bf16", seed=0, device=DEV)
    dX = lb.softmax_bwd(P, dY)
    torch.cuda.synchronize()
    num = den = 0.0
    step = 1 << 15
    for lo in range(0, rows, step):
        Pb, Yb = synth.bits(P[lo:lo + step].cpu()), synth.bits(dY[lo:lo + step].cpu())
        got = dX[lo:lo + step].float().cpu().numpy().astype(np.float64)
        ref = oracle.softmax_bwd(Pb, Yb, "bf16")
        bound = softmax_bound(oracle.decode(Pb, "bf16"), oracle.decode(Yb, "bf16"), cols, "bf16")
        assert not np.isnan(got).any()
        err = np.abs(got - ref)
        assert (err <= bound + 1e-38).all(), "rows %d+: %g" % (lo, float(np.max(err - bound)))
        num += float(np.sum((got - ref) ** 2))
        den += float(np.sum(ref ** 2))
    assert (num / den) ** 0.5 <= SM_RELF["bf16"]
