"""Ragged and unaligned bf16 calls on the MFMA kernels.

The MFMA kernels read rows in 16-byte chunks.  A bf16 call whose K or N is not a multiple
of 8, or whose pointers are not 16-byte aligned, runs on zero-padded copies (the padded
call has the same sums; its extra output rows and columns are dropped on the way back).
Forced paths show that the tile kernel, the small-M kernels and the fused small-M kernel
take such calls; each result is held to the oracle's bars over every entry and to the
per-element bound on whole rows, and on integer inputs the MFMA paths agree bit for bit
with the element-wise kernel.  Outputs sit between NaN guard bands that must stay intact.

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
PATHS = {"auto": lb.LB_PATH_AUTO, "tile": lb.LB_PATH_TILE, "small_m": lb.LB_PATH_SMALL_M,
         "fused_small_m": lb.LB_PATH_FUSED_SMALL_M, "general": lb.LB_PATH_GENERAL}


def device_view(t, offset):
    """A copy of `t` on the device starting `offset` elements into its own buffer."""
    flat = torch.empty(t.numel() + offset, dtype=t.dtype, device=DEV)
    v = flat[offset:].view(t.shape)
    v.copy_(t.to(DEV))
    return v


def run(case, path, in_offset=0, out_offset=0, need_dx=True, need_dw=True):
    X, W, G = (device_view(t, in_offset) for t in (case.X, case.W, case.G))
    gx = Guarded(case.M, case.K, torch.bfloat16, offset=out_offset) if need_dx else None
    gw = Guarded(case.K, case.N, torch.float32, offset=out_offset) if need_dw else None
    with lb.lin_bwd_path(PATHS[path]):
        lb.lin_bwd(X, W, G, gx.t if gx else None, gw.t if gw else None)
    torch.cuda.synchronize()
    for g in (gx, gw):
        if g is not None:
            g.check_guards()
    return (gx.t if gx else None), (gw.t if gw else None)


def check(case, dX, dW, bound_rows):
    """The bars over every entry; the per-element bound on `bound_rows` seeded whole rows of
    each output (all rows when there are fewer)."""
    Xb, Wb, Gb = synth.bits(case.X), synth.bits(case.W), synth.bits(case.G)
    rX, rW = oracle.lin_bwd(Xb, Wb, Gb, "bf16", need_dx=dX is not None, need_dw=dW is not None)
    aX, aW, aG = (abs_bits(b, "bf16") for b in (Xb, Wb, Gb))
    rng = np.random.default_rng(case.M + case.K + case.N)
    if dX is not None:
        hx = host_f64(dX)
        assert relf(hx, rX) <= DX_RELF, "dX relF %.3g" % relf(hx, rX)
        rows = np.unique(np.concatenate([rng.integers(0, case.M, bound_rows), [0, case.M - 1]]))
        assert_within_bound(hx[rows], rX[rows], oracle.dx_rows(aG, aW, "bf16", rows), case.N, True, "dX")
    if dW is not None:
        hw = host_f64(dW)
        assert relf(hw, rW) <= DW_RELF, "dW relF %.3g" % relf(hw, rW)
        rows = np.unique(np.concatenate([rng.integers(0, case.K, bound_rows), [0, case.K - 1]]))
        assert_within_bound(hw[rows], rW[rows], oracle.dw_rows(aX, aG, "bf16", rows), case.M, False, "dW")


# (path, M, K, N): N = 4100 and K = 4100 beside the pages' K = N = 4096; K and N odd;
# every MFMA path; tiny shapes on the automatic path
RAGGED = [("tile", 2048, 4096, 4100), ("tile", 1100, 4100, 520), ("tile", 1040, 777, 1029),
          ("small_m", 32, 4100, 4096), ("small_m", 200, 1030, 1030), ("small_m", 700, 264, 1029),
          ("fused_small_m", 48, 1000, 4100), ("auto", 32, 4096, 4100), ("auto", 5, 7, 3),
          ("auto", 70, 9, 130), ("auto", 1, 1, 1)]


@pytest.mark.parametrize("path,M,K,N", RAGGED)
def test_ragged_shapes_on_the_mfma_kernels(path, M, K, N):
    case = synth.linear_case(M, K, N, "bf16", x_std=1.0, w_std=1.0, g_std=1.0, seed=M + K + N)
    need_dw = not (path == "small_m" and M > 256)
    dX, dW = run(case, path, need_dw=need_dw)
    check(case, dX, dW if need_dw else None, bound_rows=64)


def int_case(M, K, N, seed):
    rng = np.random.default_rng(seed)
    mk = lambda *sh: torch.tensor(rng.integers(-2, 3, size=sh), dtype=torch.float32).to(torch.bfloat16)
    return synth.LinearCase(M, K, N, "bf16", mk(M, K), mk(K, N), mk(M, N))


@pytest.mark.parametrize("M,K,N,paths", [(300, 1030, 1034, ["tile"]),
                                         (40, 1030, 1034, ["tile", "small_m", "fused_small_m"]),
                                         (1100, 263, 517, ["tile"])])
def test_ragged_integer_inputs_bitwise_against_the_element_wise_kernel(M, K, N, paths):
    case = int_case(M, K, N, seed=M + K)
    ref = run(case, "general")
    rX, rW = oracle.lin_bwd(synth.bits(case.X), synth.bits(case.W), synth.bits(case.G), "bf16")
    assert np.array_equal(ref[1].cpu().numpy(), rW.astype(np.float32))
    assert torch.equal(ref[0].cpu(), torch.from_numpy(rX.astype(np.float32)).to(torch.bfloat16))
    for path in paths:
        dX, dW = run(case, path)
        assert torch.equal(dX.view(torch.int16), ref[0].view(torch.int16)), path
        assert torch.equal(dW, ref[1]), path


@pytest.mark.parametrize("in_offset,out_offset", [(1, 0), (0, 1), (3, 5)])
def test_unaligned_buffers_on_the_tile_kernel(in_offset, out_offset):
    case = synth.linear_case(1100, 264, 520, "bf16", x_std=1.0, w_std=1.0, g_std=1.0, seed=17)
    dX, dW = run(case, "tile", in_offset=in_offset, out_offset=out_offset)
    check(case, dX, dW, bound_rows=32)


def test_one_product_at_a_time():
    case = synth.linear_case(1040, 1029, 777, "bf16", x_std=1.0, w_std=1.0, g_std=1.0, seed=23)
    dX, _ = run(case, "tile", need_dw=False)
    check(case, dX, None, bound_rows=32)
    _, dW = run(case, "tile", need_dx=False)
    check(case, None, dW, bound_rows=32)


def test_staged_calls_back_to_back_on_a_side_stream():
    """Several padded calls queued on one non-default stream with no synchronisation in
    between (each allocates and releases its copies in stream order), then each result
    against the oracle and against the same call repeated on the default stream."""
    cases = [synth.linear_case(M, K, N, "bf16", x_std=1.0, w_std=1.0, g_std=1.0, seed=i)
             for i, (M, K, N) in enumerate([(1100, 260, 1030), (40, 1030, 518), (300, 517, 263)])]
    dev = [[t.to(DEV) for t in (c.X, c.W, c.G)] for c in cases]
    outs = [(torch.full((c.M, c.K), float("nan"), dtype=torch.bfloat16, device=DEV),
             torch.full((c.K, c.N), float("nan"), device=DEV)) for c in cases]
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        for _ in range(3):
            for (X, W, G), (dX, dW) in zip(dev, outs):
                lb.lin_bwd(X, W, G, dX, dW)
    torch.cuda.synchronize()
    for c, (X, W, G), (dX, dW) in zip(cases, dev, outs):
        check(c, dX, dW, bound_rows=16)
        dX2, dW2 = torch.empty_like(dX), torch.empty_like(dW)
        lb.lin_bwd(X, W, G, dX2, dW2)
        torch.cuda.synchronize()
        assert torch.equal(dX, dX2) and torch.equal(dW, dW2)


def test_padded_copies_after_shutdown():
    """lb_shutdown() destroys the pool of the padded copies; the next ragged call makes a new
    one and gives the same bits."""
    case = synth.linear_case(300, 517, 263, "bf16", x_std=1.0, w_std=1.0, g_std=1.0, seed=29)
    before = run(case, "auto")
    torch.cuda.synchronize()
    lb.lb_shutdown()
    after = run(case, "auto")
    assert torch.equal(before[0], after[0]) and torch.equal(before[1], after[1])
    check(case, *after, bound_rows=16)


@pytest.mark.parametrize("M,K,N", [(0, 100, 70), (0, 4100, 8), (37, 9, 0), (37, 0, 13)])
def test_empty_sums_with_ragged_sizes(M, K, N):
    """M = 0: dW is the empty sum (zeros); N = 0: dX is; K = 0 leaves nothing to write.  These
    calls have nothing to pad and take the element-wise kernel."""
    X = torch.randn(M, K, device=DEV).to(torch.bfloat16)
    W = torch.randn(K, N, device=DEV).to(torch.bfloat16)
    G = torch.randn(M, N, device=DEV).to(torch.bfloat16)
    dX = torch.full((M, K), float("nan"), dtype=torch.bfloat16, device=DEV)
    dW = torch.full((K, N), float("nan"), device=DEV)
    lb.lin_bwd(X, W, G, dX, dW)
    torch.cuda.synchronize()
    if M == 0:
        assert bool((dW == 0).all())
    if N == 0:
        assert bool((dX == 0).all())
