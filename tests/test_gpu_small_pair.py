"""Both small-M products in one launch (M <= 64, N <= 8192, K*N up to 2^25 for N <= 4096 and
up to 5 * 2^22 above, both outputs requested).

There the library launches one grid whose first blocks compute dX (split-reduction blocks
with a ring of 128-element chunks) and whose other blocks compute dW (64x256 small tiles),
so that dX's read stream of W and dW's write stream overlap; dX's split partials are then
added in split order by a launch of their own.  Each block computes what the separate
dX and dW kernels compute, in the same order, so these tests check:

* the oracle's bars over every entry and the per-element bound on whole rows;
* bit-for-bit agreement with the two single-product calls (dX alone and dW alone take the
  separate kernels) on random inputs;
* on integer inputs (exact in fp32 in any order), the element-wise kernel's bits;
* both sides of the N = 8192 limit, ragged K and N, every row-block width (M <= 16, <= 32,
  <= 64), and a wide N beside a K*N above the wide limit (two launches there).

For M <= 16 on small calls (K >= 512, 256 <= N <= min(4096, 4K), K*N <= 2^21) the dX blocks
sum a whole reduction each instead (16 W rows per block, the four waves' quarter sums added in
order), with no partials and no summing launch, both in the one-launch pair and for dX alone,
so the same checks hold there.

Outputs sit between NaN-poisoned guard bands that must stay intact.  Every call goes
through the C ABI of liblinbwd.so.
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

# (M, K, N): one, two and four 16-row blocks (M = 1, 16 / 17, 32 / 40, 64); the bench's
# decode shape; ragged K and N (padded copies first); N at the limit and just past it (two
# launches there); K = 2056 and 4096 at N = 8192 (one launch, then two); small K (few dX
# groups, one dW row of tiles)
SHAPES = [(1, 4096, 4096), (16, 1024, 2048), (17, 2048, 1024), (32, 4096, 4096), (40, 520, 1032),
          (64, 4096, 4096), (64, 1040, 8192), (32, 1024, 8200), (5, 4100, 4100), (24, 64, 8192),
          (28, 2056, 8192), (8, 4096, 8192), (64, 8, 264),
          # M <= 16 on small calls: dX without partials; at and just past the K*N and N limits;
          # ragged (padded copies first); a tiny call just outside
          (1, 1024, 1024), (13, 520, 2056), (9, 1030, 1030), (16, 2048, 1024), (16, 2056, 1024),
          (4, 1024, 2048), (4, 512, 2056), (6, 4096, 256), (3, 16, 8)]


def run(case, need_dx=True, need_dw=True, path=lb.LB_PATH_AUTO):
    X, W, G = (t.to(DEV) for t in (case.X, case.W, case.G))
    gx = Guarded(case.M, case.K, torch.bfloat16) if need_dx else None
    gw = Guarded(case.K, case.N, torch.float32) if need_dw else None
    with lb.lin_bwd_path(path):
        lb.lin_bwd(X, W, G, gx.t if gx else None, gw.t if gw else None)
    torch.cuda.synchronize()
    for g in (gx, gw):
        if g is not None:
            g.check_guards()
    return (gx.t if gx else None), (gw.t if gw else None)


@pytest.mark.parametrize("M,K,N", SHAPES)
def test_pair_matches_the_oracle_and_the_single_product_calls(M, K, N):
    case = synth.linear_case(M, K, N, "bf16", x_std=1.0, w_std=1.0, g_std=1.0, seed=3 * M + K + N)
    dX, dW = run(case)
    Xb, Wb, Gb = synth.bits(case.X), synth.bits(case.W), synth.bits(case.G)
    rX, rW = oracle.lin_bwd(Xb, Wb, Gb, "bf16", need_dx=True, need_dw=True)
    aX, aW, aG = (abs_bits(b, "bf16") for b in (Xb, Wb, Gb))
    hx, hw = host_f64(dX), host_f64(dW)
    assert relf(hx, rX) <= DX_RELF, "dX relF %.3g" % relf(hx, rX)
    assert relf(hw, rW) <= DW_RELF, "dW relF %.3g" % relf(hw, rW)
    rng = np.random.default_rng(M + K + N)
    rows = np.unique(np.concatenate([rng.integers(0, M, 8), [0, M - 1]]))
    assert_within_bound(hx[rows], rX[rows], oracle.dx_rows(aG, aW, "bf16", rows), N, True, "dX")
    rows = np.unique(np.concatenate([rng.integers(0, K, 32), [0, K - 1]]))
    assert_within_bound(hw[rows], rW[rows], oracle.dw_rows(aX, aG, "bf16", rows), M, False, "dW")
    # the same sums in the same order as the separate kernels: the same bits
    dX1, _ = run(case, need_dw=False)
    _, dW1 = run(case, need_dx=False)
    assert torch.equal(dX.view(torch.int16), dX1.view(torch.int16))
    assert torch.equal(dW, dW1)


@pytest.mark.parametrize("M,K,N", [(32, 4096, 4096), (64, 1032, 8192), (9, 520, 2056), (16, 1024, 2048),
                                   (1, 8, 264), (5, 2048, 512)])
def test_pair_integer_inputs_bitwise_against_the_element_wise_kernel(M, K, N):
    """Integer inputs in {-2..2}: every product and sum is exact in fp32, so the one-launch
    pair, the forced small-M path and the element-wise kernel give the same bits."""
    rng = np.random.default_rng(M * 31 + N)
    mk = lambda *sh: torch.tensor(rng.integers(-2, 3, size=sh), dtype=torch.float32).to(torch.bfloat16)
    case = synth.LinearCase(M, K, N, "bf16", mk(M, K), mk(K, N), mk(M, N))
    ref = run(case, path=lb.LB_PATH_GENERAL)
    for path in (lb.LB_PATH_AUTO, lb.LB_PATH_SMALL_M):
        dX, dW = run(case, path=path)
        assert torch.equal(dX.view(torch.int16), ref[0].view(torch.int16)), path
        assert torch.equal(dW, ref[1]), path


def test_pair_repeats_and_agrees_across_entry_points():
    """lin_bwd twice, lin_bwd_ex with db and lin_bwd_ex_noalloc: the same bits."""
    M, K, N = 48, 2048, 4096
    case = synth.linear_case(M, K, N, "bf16", x_std=1.0, w_std=1.0, g_std=1.0, seed=11)
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
