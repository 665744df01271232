"""The Linear-backward kernels cross-checked against each other and against the oracle.

* Forced paths (lb_set_lin_bwd_path): the tile kernel, the small-M kernels and the
  element-wise kernel run the same calls; each meets the bars against the oracle, and
  on integer-valued inputs (exact fp32 sums) all three agree bit for bit.
* The transposition identity: dW(X, G) = Xᵀ·G is also dX of the call with dY := Xᵀ and
  W := Gᵀ, so the dX kernels compute the dW product from transposed copies.
* Streams: calls that use the library's workspace (small-M dX partials, the bias
  gradient's row partials, the gradient norm's block partials) issued on two streams at
  once, each checked against the oracle.

Every call goes through the C ABI of liblinbwd.so.
"""
import numpy as np
import pytest
import torch

import linear_layer_backward_bwd_amd as lb
import oracle
import synth
from gpu_util import (DB_RELF, DW_RELF, DX_RELF, NORM_ULP, abs_bits, assert_within_bound,
                      host_f64, relf, ulp_distance_f32)

pytestmark = pytest.mark.gpu
DEV = "cuda"
PATHS = {"tile": lb.LB_PATH_TILE, "small_m": lb.LB_PATH_SMALL_M, "general": lb.LB_PATH_GENERAL,
         "fused_small_m": lb.LB_PATH_FUSED_SMALL_M}


def runs_on(name, M):
    """Whether a forced path takes this M with both outputs requested (dW on the small-M
    path needs M <= 256; the fused path needs M <= 64)."""
    return not ((name == "small_m" and M > 256) or (name == "fused_small_m" and M > 64))


def run_path(case, path, need_dx=True, need_dw=True):
    X, W, G = (t.to(DEV) for t in (case.X, case.W, case.G))
    dX = torch.full((case.M, case.K), float("nan"), dtype=case.X.dtype, device=DEV) if need_dx else None
    dW = torch.full((case.K, case.N), float("nan"), dtype=torch.float32, device=DEV) if need_dw else None
    with lb.lin_bwd_path(path):
        lb.lin_bwd(X, W, G, dX, dW)
    torch.cuda.synchronize()
    return dX, dW


def int_case(M, K, N, seed):
    rng = np.random.default_rng(seed)
    mk = lambda *sh: torch.tensor(rng.integers(-2, 3, size=sh), dtype=torch.float32).to(torch.bfloat16)
    return synth.LinearCase(M, K, N, "bf16", mk(M, K), mk(K, N), mk(M, N))


# M <= 256 runs every product on every path; 256 < M <= 1024 runs dX only on the small-M
# path; M <= 64 also on the fused path (K = 264 / 520: a partial last group of 16 rows;
# N = 264 / 2056: a partial last chunk of 256 columns; N = 520 with K = 264: several splits)
CROSS_SHAPES = [(1, 264, 520), (17, 4104, 264), (32, 1032, 2056), (48, 264, 4104), (64, 520, 264),
                (100, 264, 1032), (256, 1032, 520), (384, 520, 1032), (1024, 264, 520)]


@pytest.mark.parametrize("M,K,N", CROSS_SHAPES)
def test_each_path_meets_the_bars(M, K, N):
    case = synth.linear_case(M, K, N, "bf16", x_std=1.0, w_std=1.0, g_std=1.0, seed=M + 2 * K + N)
    rX, rW = oracle.lin_bwd(synth.bits(case.X), synth.bits(case.W), synth.bits(case.G), "bf16")
    aX, aW, aG = (abs_bits(synth.bits(t), "bf16") for t in (case.X, case.W, case.G))
    SX = oracle.lin_bwd(aX, aW, aG, "bf16")
    for name, path in PATHS.items():
        if name == "fused_small_m" and M > 64:
            continue
        need_dw = runs_on(name, M)
        dX, dW = run_path(case, path, need_dw=need_dw)
        e = relf(host_f64(dX), rX)
        assert e <= DX_RELF, "%s dX relF %.3g" % (name, e)
        seq = name == "general"
        assert_within_bound(host_f64(dX), rX, SX[0], N, True, name + " dX", sequential=seq)
        if need_dw:
            e = relf(host_f64(dW), rW)
            assert e <= DW_RELF, "%s dW relF %.3g" % (name, e)
            assert_within_bound(host_f64(dW), rW, SX[1], M, False, name + " dW", sequential=seq)


@pytest.mark.parametrize("M,K,N", [(48, 264, 2056), (64, 4096, 1032), (200, 1032, 520),
                                   (700, 264, 1032)])
def test_paths_agree_bitwise_on_integer_inputs(M, K, N):
    case = int_case(M, K, N, seed=M)
    outs = {}
    for name, path in PATHS.items():
        if name == "fused_small_m" and M > 64:
            continue
        outs[name] = run_path(case, path, need_dw=runs_on(name, M))
    for name in [n for n in outs if n != "tile"]:
        assert torch.equal(outs[name][0].view(torch.int16), outs["tile"][0].view(torch.int16)), name
        if outs[name][1] is not None:
            assert torch.equal(outs[name][1], outs["tile"][1]), name


def test_forced_path_refusal_leaves_outputs_untouched():
    """A forced path that cannot run the call is refused before anything is enqueued."""
    case = synth.linear_case(300, 264, 520, "bf16", seed=3)
    with pytest.raises(RuntimeError, match="forced kernel path"):
        run_path(case, lb.LB_PATH_SMALL_M)          # dW on the small-M path needs M <= 256
    X, W, G = (t.to(DEV) for t in (case.X, case.W, case.G))
    dW = torch.full((case.K, case.N), 7.0, device=DEV)
    with lb.lin_bwd_path(lb.LB_PATH_SMALL_M):
        with pytest.raises(RuntimeError):
            lb.lin_bwd(X, W, G, None, dW)
    torch.cuda.synchronize()
    assert bool((dW == 7.0).all())


# ---- the transposition identity ------------------------------------------------------

@pytest.mark.parametrize("path", ["auto", "tile"])
@pytest.mark.parametrize("M,K,N", [(296, 520, 264), (1096, 264, 1032), (96, 2056, 520)])
def test_dw_equals_dx_of_transposed_operands(M, K, N, path):
    """dW[k,n] = Σ_m X[m,k]·G[m,n] is dX' = dY'·W'ᵀ of the call with M' = K, K' = N, N' = M,
    dY' = Xᵀ [K,M] and W' = Gᵀ [N,M]: the dW kernels (outer-contiguous operands, transposing
    LDS reads) against the dX kernels (reduction-contiguous operands) on the same sums.
    dX' is rounded to bf16: one rounding apart from dW plus both kernels' fp32 error."""
    case = synth.linear_case(M, K, N, "bf16", x_std=1.0, w_std=1.0, g_std=1.0, seed=K + N)
    forced = lb.LB_PATH_TILE if path == "tile" else lb.LB_PATH_AUTO
    _, dW = run_path(case, forced, need_dx=False)
    tcase = synth.LinearCase(K, N, M, "bf16", torch.zeros(K, N, dtype=torch.bfloat16),
                             case.G.t().contiguous(), case.X.t().contiguous())
    dXt, _ = run_path(tcase, forced, need_dw=False)
    aX, aG = abs_bits(synth.bits(case.X), "bf16"), abs_bits(synth.bits(case.G), "bf16")
    S = oracle.dw_rows(aX, aG, "bf16", np.arange(K))                    # Σ_m |X[m,k]·G[m,n]|
    d = host_f64(dXt)
    w = host_f64(dW)
    assert relf(d, w) <= DX_RELF
    # both are within gamma(M)·S of the exact sum; dX' adds one bf16 rounding
    assert_within_bound(d, w, 2.0 * S, M, True, "dX of the transposed operands")


def test_transposition_identity_is_exact_on_integer_inputs():
    case = int_case(520, 264, 1032, seed=9)
    _, dW = run_path(case, lb.LB_PATH_AUTO, need_dx=False)
    tcase = synth.LinearCase(264, 1032, 520, "bf16", torch.zeros(264, 1032, dtype=torch.bfloat16),
                             case.G.t().contiguous(), case.X.t().contiguous())
    dXt, _ = run_path(tcase, lb.LB_PATH_AUTO, need_dw=False)
    assert torch.equal(dXt.cpu(), dW.cpu().to(torch.bfloat16))


# ---- two streams -----------------------------------------------------------------------

def test_workspace_users_on_two_streams_at_once():
    """Small-M lin_bwd (fp32 dX partials), lin_bwd_ex with db (row partials) and grad_norm
    (block partials), each on two streams, issued back to back several times without a
    synchronisation in between; every result against the oracle, and equal bit for bit to
    the same calls on one stream."""
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    # M = 200: dX sums over n in 16 splits whose fp32 partials go to the workspace
    cases = [synth.linear_case(200, 1032, 4104, "bf16", seed=60 + i) for i in range(2)]
    grads = [synth.adamw_case(1 << 21, "bf16", seed=70 + i).g for i in range(2)]
    dev = []
    for c, g in zip(cases, grads):
        X, W, G = (t.to(DEV) for t in (c.X, c.W, c.G))
        dev.append(dict(X=X, W=W, G=G, g=g.to(DEV),
                        dX=torch.empty(c.M, c.K, dtype=torch.bfloat16, device=DEV),
                        dW=torch.empty(c.K, c.N, device=DEV), db=torch.empty(c.N, device=DEV),
                        dX2=torch.empty(c.M, c.K, dtype=torch.bfloat16, device=DEV),
                        out=torch.empty(2, device=DEV), found=torch.empty(1, dtype=torch.int32,
                                                                         device=DEV)))
    torch.cuda.synchronize()

    def issue(d):
        lb.lin_bwd(d["X"], d["W"], d["G"], d["dX"], d["dW"])
        lb.grad_norm(d["g"], 1.0 / 1024, 0.0, out=d["out"], found_inf=d["found"])
        lb.lin_bwd_ex(d["X"], d["W"], d["G"], d["dX2"], None, d["db"])

    for _ in range(4):
        for s, d in zip(streams, dev):
            with torch.cuda.stream(s):
                issue(d)
    torch.cuda.synchronize()
    results = [{k: d[k].clone() for k in ("dX", "dW", "db", "dX2", "out")} for d in dev]
    for c, g, r in zip(cases, grads, results):
        Xb, Wb, Gb = synth.bits(c.X), synth.bits(c.W), synth.bits(c.G)
        rX, rW = oracle.lin_bwd(Xb, Wb, Gb, "bf16")
        assert relf(host_f64(r["dX"]), rX) <= DX_RELF
        assert relf(host_f64(r["dW"]), rW) <= DW_RELF
        assert torch.equal(r["dX"], r["dX2"])
        assert relf(r["db"].cpu().numpy(), oracle.bias_grad(Gb, "bf16")) <= DB_RELF
        norm = oracle.grad_norm(synth.bits(g), "bf16", 1.0 / 1024)[0]
        assert ulp_distance_f32(np.float32([r["out"][0].item()]), np.float32([norm]))[0] <= NORM_ULP
    # the same calls on one stream, one after the other
    for d in dev:
        issue(d)
    torch.cuda.synchronize()
    for d, r in zip(dev, results):
        for k in ("dX", "dW", "db", "dX2", "out"):
            assert torch.equal(d[k], r[k]), k
