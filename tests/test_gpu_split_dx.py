"""dX on the tile kernel with its reduction split over several tiles (where few, long dX
tiles would outlast the launch: from M = 257 up to 2048, and from M = 160 with both products
requested and K, N >= 2048).

In that range dW runs on the 256x256 tile kernel, and dX would give only (M/256)(K/256)
tiles, each over the whole reduction N: the launch would last as long as one such tile.
So dX's reduction is cut into ranges of whole 64-element pairs; the tiles of range s write
fp32 partial sums to the library's workspace, and a later launch adds the ranges in order
and rounds once to bf16.  These tests hold that path to the oracle's bars over every entry
and to the per-element bound on whole rows; check on integer inputs (exact in fp32 in any
summation order) that it gives the element-wise kernel's bits; and check that results
repeat, and agree between lin_bwd, lin_bwd_ex and lin_bwd_ex_noalloc, bit for bit (they
choose the same splits).  Outputs sit between NaN guard bands that must stay intact.

Every call goes through the C ABI of liblinbwd.so.
"""
import numpy as np
import pytest
import torch

import linear_layer_backward_bwd_amd as lb
import oracle
import synth
from gpu_util import DW_RELF, DX_RELF, Guarded, abs_bits, assert_within_bound, host_f64, relf

pytestmark = pytest.mark.gpu
DEV = "cuda"


def run(case, need_dw=True, path=lb.LB_PATH_AUTO):
    X, W, G = (t.to(DEV) for t in (case.X, case.W, case.G))
    gx = Guarded(case.M, case.K, torch.bfloat16)
    gw = Guarded(case.K, case.N, torch.float32) if need_dw else None
    with lb.lin_bwd_path(path):
        lb.lin_bwd(X, W, G, gx.t, gw.t if gw else None)
    torch.cuda.synchronize()
    for g in (gx, gw):
        if g is not None:
            g.check_guards()
    return gx.t, (gw.t if gw else None)


def check(case, dX, dW, bound_rows):
    """The bars over every entry; the per-element bound on `bound_rows` seeded whole rows of
    each output plus the first and the last."""
    Xb, Wb, Gb = synth.bits(case.X), synth.bits(case.W), synth.bits(case.G)
    rX, rW = oracle.lin_bwd(Xb, Wb, Gb, "bf16", need_dx=True, need_dw=dW is not None)
    aX, aW, aG = (abs_bits(b, "bf16") for b in (Xb, Wb, Gb))
    rng = np.random.default_rng(case.M * 7 + case.K + case.N)
    hx = host_f64(dX)
    assert relf(hx, rX) <= DX_RELF, "dX relF %.3g" % relf(hx, rX)
    rows = np.unique(np.concatenate([rng.integers(0, case.M, bound_rows), [0, case.M - 1]]))
    assert_within_bound(hx[rows], rX[rows], oracle.dx_rows(aG, aW, "bf16", rows), case.N, True, "dX")
    if dW is not None:
        hw = host_f64(dW)
        assert relf(hw, rW) <= DW_RELF, "dW relF %.3g" % relf(hw, rW)
        rows = np.unique(np.concatenate([rng.integers(0, case.K, bound_rows), [0, case.K - 1]]))
        assert_within_bound(hw[rows], rW[rows], oracle.dw_rows(aX, aG, "bf16", rows), case.M, False, "dW")


# (M, K, N, need_dw): both products on the tile kernel below M = 257 (large K and N); the
# first M that takes the split for any K and N; two and four ranges; ragged K and N (padded
# copies, then the split); N = 16384, where the rows of dY and W are 32 KiB apart and the
# tiles start their ranges at rotated pairs (eight ranges of 32 pairs here); M = 1024; above
# 1024 with small K, and (1280, 2048, 8192), whose four ranges of partials (40 MiB) need more
# than half the workspace
SHAPES = [(160, 2048, 2048, True), (200, 2048, 4100, True), (257, 256, 8192, True),
          (300, 1040, 2056, True), (600, 520, 4096, True), (1000, 520, 4100, True),
          (700, 777, 1030, True), (512, 1024, 16384, False), (1024, 1024, 4096, True),
          (1100, 264, 8192, True), (1500, 260, 4100, True), (1280, 2048, 8192, True)]


@pytest.mark.parametrize("M,K,N,need_dw", SHAPES)
def test_split_dx_matches_the_oracle(M, K, N, need_dw):
    case = synth.linear_case(M, K, N, "bf16", x_std=1.0, w_std=1.0, g_std=1.0, seed=M + K + N)
    dX, dW = run(case, need_dw=need_dw)
    check(case, dX, dW, bound_rows=48)


def int_case(M, K, N, seed):
    rng = np.random.default_rng(seed)
    mk = lambda *sh: torch.tensor(rng.integers(-2, 3, size=sh), dtype=torch.float32).to(torch.bfloat16)
    return synth.LinearCase(M, K, N, "bf16", mk(M, K), mk(K, N), mk(M, N))


@pytest.mark.parametrize("M,K,N", [(192, 2048, 2056), (600, 264, 4096), (512, 1024, 16384),
                                   (1024, 520, 2056), (1300, 520, 4096)])
def test_split_dx_integer_inputs_bitwise_against_the_element_wise_kernel(M, K, N):
    """Integer inputs in {-2..2}: every partial and every sum is exact in fp32, so the split
    path, the forced tile path and the element-wise kernel all give the same bits."""
    case = int_case(M, K, N, seed=M + N)
    ref = run(case, path=lb.LB_PATH_GENERAL)
    for path in (lb.LB_PATH_AUTO, lb.LB_PATH_TILE):
        dX, dW = run(case, path=path)
        assert torch.equal(dX.view(torch.int16), ref[0].view(torch.int16)), path
        assert torch.equal(dW, ref[1]), path


def test_split_dx_repeats_and_agrees_across_entry_points():
    """The same call twice, lin_bwd_ex with db and lin_bwd_ex_noalloc: dX and dW bit for bit
    (each entry point has the same workspace capacity, hence the same ranges)."""
    M, K, N = 640, 1024, 4096
    case = synth.linear_case(M, K, N, "bf16", x_std=1.0, w_std=1.0, g_std=1.0, seed=5)
    X, W, G = (t.to(DEV) for t in (case.X, case.W, case.G))
    outs = []
    for how in ("lin_bwd", "lin_bwd", "ex", "noalloc"):
        dX = torch.full((M, K), float("nan"), dtype=torch.bfloat16, device=DEV)
        dW = torch.full((K, N), float("nan"), device=DEV)
        db = torch.full((N,), float("nan"), device=DEV)
        if how == "lin_bwd":
            lb.lin_bwd(X, W, G, dX, dW)
        else:
            lb.lin_bwd_ex(X, W, G, dX, dW, db, no_alloc=how == "noalloc")
        torch.cuda.synchronize()
        outs.append((dX.view(torch.int16).clone(), dW.clone()))
    for dX, dW in outs[1:]:
        assert torch.equal(dX, outs[0][0]) and torch.equal(dW, outs[0][1])
    check(case, outs[0][0].view(torch.bfloat16), outs[0][1], bound_rows=16)
