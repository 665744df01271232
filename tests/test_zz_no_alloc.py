"""lin_bwd_ex_noalloc (temporaries in the library's static device array) against
lin_bwd_ex (temporaries in the stream's workspace): the same kernels and splits, so
the same bits; and both against the oracle's bars.  Two calls in a row, the second
smaller, so the second reuses the array with the first call's partials still in it.
Every call goes through the C ABI of liblinbwd.so.
"""
import ctypes

import numpy as np
import pytest
import torch

import linear_layer_backward_bwd_amd as lb
import oracle
import synth
from gpu_util import DB_RELF, DW_RELF, DX_RELF, host_f64, relf

pytestmark = pytest.mark.gpu
DEV = "cuda"


def call(entry, case, with_dx=True, with_dw=True, with_db=True):
    X, W, G = (t.to(DEV) for t in (case.X, case.W, case.G))
    dX = torch.full((case.M, case.K), float("nan"), dtype=torch.bfloat16, device=DEV) if with_dx else None
    dW = torch.full((case.K, case.N), float("nan"), device=DEV) if with_dw else None
    db = torch.full((case.N,), float("nan"), device=DEV) if with_db else None
    torch.cuda.synchronize()
    lib = lb.library()
    lib.lb_set_stream(ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    p = lambda t: None if t is None else t.data_ptr()
    rc = getattr(lib, entry)(p(X), p(W), p(G), p(dX), p(dW), p(db), case.M, case.K, case.N, lb.LB_BF16)
    assert rc == 0, lb.lb_last_error()
    torch.cuda.synchronize()
    return dX, dW, db


def check(case, got, ref):
    for a, b in zip(got, ref):
        if a is not None:
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32))
    Xb, Wb, Gb = synth.bits(case.X), synth.bits(case.W), synth.bits(case.G)
    rX, rW = oracle.lin_bwd(Xb, Wb, Gb, "bf16")
    dX, dW, db = got
    if dX is not None:
        assert relf(host_f64(dX), rX) <= DX_RELF
    if dW is not None:
        assert relf(host_f64(dW), rW) <= DW_RELF
    if db is not None:
        assert relf(db.cpu().numpy(), oracle.bias_grad(Gb, "bf16")) <= DB_RELF


# (M, K, N), each call smaller than the one before: M = 600 sums dX in 8 ranges on the tile
# kernel, M = 200 in 16 splits on the small-M kernel, and db in row splits, all through the
# array; M = 40 (4 splits) reads back only what it wrote
SHAPES = [(600, 1032, 4104), (200, 1032, 4104), (40, 520, 1032)]


def test_noalloc_matches_lin_bwd_ex_two_calls_in_a_row():
    for M, K, N in SHAPES:
        case = synth.linear_case(M, K, N, "bf16", x_std=1.0, w_std=1.0, g_std=1.0, seed=M + N)
        got = call("lin_bwd_ex_noalloc", case)
        ref = call("lin_bwd_ex", case)
        check(case, got, ref)


def test_noalloc_db_only_and_dx_only():
    case = synth.linear_case(300, 264, 2056, "bf16", seed=5)
    check(case, call("lin_bwd_ex_noalloc", case, with_dx=False, with_dw=False),
          call("lin_bwd_ex", case, with_dx=False, with_dw=False))
    case = synth.linear_case(24, 1032, 520, "bf16", seed=6)
    check(case, call("lin_bwd_ex_noalloc", case, with_dw=False, with_db=False),
          call("lin_bwd_ex", case, with_dw=False, with_db=False))


def test_noalloc_through_the_binding():
    case = synth.linear_case(64, 520, 1032, "bf16", seed=7)
    X, W, G = (t.to(DEV) for t in (case.X, case.W, case.G))
    outs = []
    for no_alloc in (True, False):
        dX = torch.empty(case.M, case.K, dtype=torch.bfloat16, device=DEV)
        dW = torch.empty(case.K, case.N, device=DEV)
        db = torch.empty(case.N, device=DEV)
        lb.lin_bwd_ex(X, W, G, dX, dW, db, no_alloc=no_alloc)
        outs.append((dX, dW, db))
    torch.cuda.synchronize()
    for a, b in zip(*outs):
        assert torch.equal(a, b)


@pytest.mark.parametrize("M", [200, 600])
def test_noalloc_replays_of_a_captured_graph(M):
    """lin_bwd_ex_noalloc captured into a HIP graph (its callers include graph capture),
    replayed on new inputs copied into the captured buffers, with eager work and
    synchronisations between replays; every replay bit for bit equal to lin_bwd_ex run
    eagerly on the same inputs.  M = 200 sums dX in 16 splits on the small-M kernel, M = 600
    in 8 ranges on the tile kernel (the split launch and the launch that adds the ranges),
    and db in row splits, all through the static array, so each replay reuses what the
    previous one left there."""
    K, N = 1032, 4104
    cases = [synth.linear_case(M, K, N, "bf16", x_std=1.0, w_std=1.0, g_std=1.0, seed=90 + i)
             for i in range(3)]
    X, W, G = (t.to(DEV) for t in (cases[0].X, cases[0].W, cases[0].G))
    dX = torch.empty(M, K, dtype=torch.bfloat16, device=DEV)
    dW = torch.empty(K, N, device=DEV)
    db = torch.empty(N, device=DEV)
    # the first call on the device looks up the array's address: outside the capture
    lb.lin_bwd_ex(X, W, G, dX, dW, db, no_alloc=True)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        lb.lin_bwd_ex(X, W, G, dX, dW, db, no_alloc=True)
    torch.cuda.synchronize()
    for rep in range(6):
        c = cases[rep % len(cases)]
        X.copy_(c.X.to(DEV))
        W.copy_(c.W.to(DEV))
        G.copy_(c.G.to(DEV))
        dX.fill_(float("nan"))
        dW.fill_(float("nan"))
        db.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        got = (dX.clone(), dW.clone(), db.clone())
        # eager work between replays: the allocating entry point on the same inputs
        ref = call("lin_bwd_ex", c)
        for a, b in zip(got, ref):
            assert torch.equal(a, b), "replay %d" % rep
    check(cases[-1], got, ref)
