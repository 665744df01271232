"""GPU parity of lin_bwd (dX = dY·Wᵀ, dW = Xᵀ·dY) against the CPU oracle.

Every call goes through the C ABI of liblinbwd.so.  Bars (written in
gpu_util): bf16 dX relative Frobenius error <= 4e-3, fp32 dW <= 1e-5, fp32
dX (fp32 operands) <= 1e-5; integer-valued and identity cases bitwise.
"""
import numpy as np
import pytest
import torch

import linear_layer_backward_bwd_amd as lb
import oracle
import synth
from gpu_util import (DW_RELF, DX_RELF, F32_OUT_RELF, Guarded, abs_bits, assert_within_bound,
                      bits, host_f64, relf)

pytestmark = pytest.mark.gpu
DEV = "cuda"
TDT = {"bf16": torch.bfloat16, "f32": torch.float32}


def run(case, need_dx=True, need_dw=True, stream=None, offset=0, path=lb.LB_PATH_AUTO):
    X, W, G = (t.to(DEV) for t in (case.X, case.W, case.G))
    gx = Guarded(case.M, case.K, TDT[case.dtype], offset=offset) if need_dx else None
    gw = Guarded(case.K, case.N, torch.float32, offset=offset) if need_dw else None
    with lb.lin_bwd_path(path):
        if stream is not None:
            with torch.cuda.stream(stream):
                lb.lin_bwd(X, W, G, gx.t if gx else None, gw.t if gw else None)
        else:
            lb.lin_bwd(X, W, G, gx.t if gx else None, gw.t if gw else None)
    torch.cuda.synchronize()
    for g in (gx, gw):
        if g is not None:
            g.check_guards()
    return (gx.t if gx else None), (gw.t if gw else None)


def check_full(case, dX, dW):
    rX, rW = oracle.lin_bwd(synth.bits(case.X), synth.bits(case.W), synth.bits(case.G), case.dtype,
                            need_dx=dX is not None, need_dw=dW is not None)
    if dX is not None:
        hx = host_f64(dX)
        assert not np.isnan(hx).any(), "dX has unwritten (NaN) entries"
        bar = DX_RELF if case.dtype == "bf16" else F32_OUT_RELF
        e = relf(hx, rX)
        assert e <= bar, "dX relF %.3g > %.3g" % (e, bar)
    if dW is not None:
        hw = host_f64(dW)
        assert not np.isnan(hw).any(), "dW has unwritten (NaN) entries"
        e = relf(hw, rW)
        assert e <= DW_RELF, "dW relF %.3g > %.3g" % (e, DW_RELF)
    return rX, rW


SHAPES = [
    # (M, K, N): MFMA tiles with ragged edges and a partial reduction slab
    (300, 520, 264), (257, 264, 520), (96, 64, 4104), (200, 256, 256), (512, 512, 512),
    (65, 128, 384),
    # small-M dX path (M <= 64), with the MFMA dW path
    (64, 384, 520), (32, 1024, 1032), (17, 40, 8), (1, 264, 72), (48, 8, 1000),
    # sizes not multiples of 8: zero-padded copies on the MFMA kernels
    (33, 100, 70), (5, 7, 3), (70, 9, 130),
]


@pytest.mark.parametrize("M,K,N", SHAPES)
def test_bf16_shapes_match_oracle(M, K, N):
    case = synth.linear_case(M, K, N, "bf16", x_std=1.0, w_std=1.0, g_std=1.0, seed=M + K + N)
    dX, dW = run(case)
    check_full(case, dX, dW)


# The small-M kernels: dW (M <= 64) in 64x256 tiles with one or two 32-row
# reduction slabs; dX (M <= 1024, in row groups of 256 above 256) over
# 64-column groups with the reduction split
# across blocks (fp32 partials summed in split order) in chunks of 256 (M <= 64)
# or 128.  Shapes: M in each of the 16/32/64/128/256-row variants and across
# their boundaries, ragged k groups, n tiles and chunks, several chunks per
# split (K = 4096, N = 8192), M*K above the 2^23-float partial workspace (runs
# unsplit and stores bf16 directly), and M > 64, where dW takes the tile kernel
# and the partials are summed by a launch of their own.
SMALL_M_SHAPES = [
    (1, 264, 1544), (16, 4104, 520), (17, 1032, 2056), (32, 640, 3080), (33, 200, 3080),
    (48, 72, 264), (63, 520, 1032), (64, 8, 40), (32, 4096, 8192), (64, 33792, 64),
    (65, 264, 1032), (128, 520, 2056), (129, 1032, 392), (200, 4104, 520), (256, 1032, 3080),
    (256, 33792, 8), (257, 264, 1032), (384, 1032, 520), (512, 520, 2056), (513, 264, 392),
    (768, 1032, 520), (1024, 264, 1032), (1025, 136, 264),
]


@pytest.mark.parametrize("M,K,N", SMALL_M_SHAPES)
def test_small_m_shapes_match_oracle(M, K, N):
    case = synth.linear_case(M, K, N, "bf16", x_std=1.0, w_std=1.0, g_std=1.0, seed=3 * M + K + N)
    dX, dW = run(case)
    check_full(case, dX, dW)


@pytest.mark.parametrize("M", [32, 384])
def test_small_m_repeatable(M):
    """The split reduction adds partials in a fixed order: two runs agree bit for bit
    (M = 384 also has two row groups)."""
    case = synth.linear_case(M, 4096, 4096, "bf16", seed=11)
    a = [t.clone() for t in run(case)]
    b = run(case)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("M,K,N", [(24, 520, 2056), (200, 264, 3080)])
def test_small_m_one_output_at_a_time(M, K, N):
    """dX alone (its split partials then get a summing launch of their own) and dW alone."""
    case = synth.linear_case(M, K, N, "bf16", x_std=1.0, w_std=1.0, g_std=1.0, seed=M + 5)
    dX, _ = run(case, need_dw=False)
    check_full(case, dX, None)
    _, dW = run(case, need_dx=False)
    check_full(case, None, dW)


@pytest.mark.parametrize("M,K,N", [(40, 264, 2056), (200, 520, 1032), (384, 136, 1544)])
def test_small_m_integer_inputs_are_exact(M, K, N):
    """Values in {-2..2}: every partial and their sum are exact in fp32, so dW is bitwise and
    dX = RNE(exact) whatever the split (small-M dW, tile-kernel dW, row groups)."""
    rng = np.random.default_rng(M + 1)
    mk = lambda *sh: torch.tensor(rng.integers(-2, 3, size=sh), dtype=torch.float32).to(torch.bfloat16)
    case = synth.LinearCase(M, K, N, "bf16", mk(M, K), mk(K, N), mk(M, N))
    dX, dW = run(case)
    rX, rW = oracle.lin_bwd(synth.bits(case.X), synth.bits(case.W), synth.bits(case.G), "bf16")
    assert np.array_equal(dW.cpu().numpy(), rW.astype(np.float32))
    assert torch.equal(dX.cpu(), torch.from_numpy(rX.astype(np.float32)).to(torch.bfloat16))


def test_small_m_non_default_stream():
    case = synth.linear_case(48, 1032, 2056, "bf16", seed=12)
    s = torch.cuda.Stream()
    dX, dW = run(case, stream=s)
    check_full(case, dX, dW)


# Reduction lengths around the 32-deep slab, the 64-deep dX slab pair (a
# partial last pair when R % 64 != 0) and the padding of the slab count to a
# multiple of four.
REDUCTIONS = [8, 24, 32, 40, 64, 72, 96, 128, 136, 200, 256, 264, 392]


@pytest.mark.parametrize("R", REDUCTIONS)
def test_short_and_ragged_reductions(R):
    # dX, reduction over n = R: on the split-reduction kernel (M = 96) and on the
    # tile kernel (M = 1040 > 1024: four whole tile rows and a 16-row one)
    for M in (96, 1040):
        case = synth.linear_case(M, 72, R, "bf16", x_std=1.0, w_std=1.0, g_std=1.0, seed=R + M)
        dX, _ = run(case, need_dw=False)
        check_full(case, dX, None)
    # dW: reduction over m = R
    case = synth.linear_case(R, 72, 80, "bf16", x_std=1.0, w_std=1.0, g_std=1.0, seed=R + 1)
    _, dW = run(case, need_dx=False)
    check_full(case, None, dW)


# Both products on the tile kernel (M > 1024) with ragged output edges: each
# 256x256 tile's four 128x128 quadrants are whole, partial or wholly outside the
# output (M = 1152: dX rows 1152..1279 of the last tile row; N = 96: dW columns
# 128..255), and the reductions end in partial slab pairs.
@pytest.mark.parametrize("M,K,N", [(1152, 384, 200), (1100, 264, 520), (2000, 520, 96), (1300, 136, 1032)])
def test_tile_kernel_ragged_edges(M, K, N):
    case = synth.linear_case(M, K, N, "bf16", x_std=1.0, w_std=1.0, g_std=1.0, seed=M ^ K ^ N)
    dX, dW = run(case)
    check_full(case, dX, dW)


def test_shutdown_then_calls_allocate_again():
    # M = 48 keeps its dX split partials in the library's workspace
    case = synth.linear_case(48, 1032, 2056, "bf16", seed=21)
    dX0, dW0 = run(case)
    lb.lb_shutdown()
    lb.lb_shutdown()  # nothing left to free
    dX1, dW1 = run(case)
    assert torch.equal(dX0.view(torch.int16), dX1.view(torch.int16))
    assert torch.equal(dW0.view(torch.int32), dW1.view(torch.int32))
    check_full(case, dX1, dW1)


@pytest.mark.parametrize("M,K,N", [(64, 64, 64), (33, 100, 70), (130, 264, 96)])
def test_f32_shapes_match_oracle(M, K, N):
    case = synth.linear_case(M, K, N, "f32", x_std=1.0, w_std=1.0, g_std=1.0, seed=7)
    dX, dW = run(case)
    check_full(case, dX, dW)


def test_tiny_f32_workload_then_adamw():
    """64x64x64 fp32 backward, then one AdamW step on W with g = dW (GPU chain vs oracle chain)."""
    case, hp = synth.tiny_f32(seed=0)
    dX, dW = run(case)
    rX, rW = check_full(case, dX, dW)
    W = case.W.to(DEV).clone()
    m = torch.zeros_like(W)
    v = torch.zeros_like(W)
    lb.adamw_step(W, dW.contiguous(), m, v, hp["lr"], hp["b1"], hp["b2"], hp["eps"], hp["wd"],
                  hp["step"], hp["inv_scale"])
    torch.cuda.synchronize()
    z = np.zeros((64, 64), np.float32)
    oW, om, ov = oracle.adamw(synth.bits(case.W), rW.astype(np.float32), z, z, "f32", hp["lr"],
                              hp["b1"], hp["b2"], hp["eps"], hp["wd"], hp["step"], hp["inv_scale"])
    from gpu_util import adamw_ok
    for got, ref in ((W, oW), (m, om), (v, ov)):
        ok, err = adamw_ok(got.cpu().numpy(), ref)
        assert ok, err


def test_skip_outputs_and_empty_sums():
    case = synth.linear_case(100, 72, 80, "bf16", seed=3)
    dX, dW = run(case, need_dx=False)
    assert dX is None
    check_full(case, None, dW)
    dX, dW = run(case, need_dw=False)
    check_full(case, dX, None)
    # M = 0: dW is the empty sum, zeros
    e = synth.linear_case(0, 72, 80, "bf16", seed=4)
    _, dW = run(e, need_dx=False)
    assert bool((dW == 0).all())
    # N = 0: dX is zeros
    e = synth.linear_case(40, 72, 0, "bf16", seed=5)
    dX, _ = run(e, need_dw=False)
    assert bool((dX == 0).all())
    # N = 0 on the tile path (M > 64): a reduction of padding slabs only
    e = synth.linear_case(100, 72, 0, "bf16", seed=5)
    dX, _ = run(e, need_dw=False)
    assert bool((dX == 0).all())
    # small-M shape with N = 0, and fp32 with M = 0
    e = synth.linear_case(0, 9, 7, "f32", seed=6)
    _, dW = run(e, need_dx=False)
    assert bool((dW == 0).all())


def test_misaligned_pointers_take_a_correct_path():
    case = synth.linear_case(64, 136, 136, "bf16", x_std=1.0, w_std=1.0, g_std=1.0, seed=8)
    dX, dW = run(case, offset=1)
    check_full(case, dX, dW)


@pytest.mark.parametrize("M,K,N", [(96, 256, 264), (24, 264, 256), (300, 520, 136)])
def test_integer_inputs_are_exact(M, K, N):
    """Values in {-2..2}: products exact, fp32 sums exact; dW bitwise, dX = RNE(exact)."""
    rng = np.random.default_rng(M)
    mk = lambda *s: torch.tensor(rng.integers(-2, 3, size=s), dtype=torch.float32).to(torch.bfloat16)
    case = synth.LinearCase(M, K, N, "bf16", mk(M, K), mk(K, N), mk(M, N))
    dX, dW = run(case)
    rX, rW = oracle.lin_bwd(synth.bits(case.X), synth.bits(case.W), synth.bits(case.G), "bf16")
    assert np.array_equal(dW.cpu().numpy(), rW.astype(np.float32))
    want = torch.from_numpy(rX.astype(np.float32)).to(torch.bfloat16)
    assert torch.equal(dX.cpu(), want)


def test_identity_operands_are_bitwise():
    n = 256
    G = synth.to_storage(synth.normal((n, n), 1.0, synth._gen(9)), "bf16")
    eye = torch.eye(n, dtype=torch.bfloat16)
    # W = I: dX = G exactly;  X = I: dW = G exactly
    case = synth.LinearCase(n, n, n, "bf16", eye, eye, G)
    dX, dW = run(case)
    assert torch.equal(dX.cpu(), G)
    assert torch.equal(dW.cpu(), G.float())


def test_scaling_and_determinism():
    case = synth.linear_case(384, 512, 520, "bf16", x_std=1.0, w_std=1.0, g_std=1.0, seed=10)
    dX1, dW1 = run(case)
    dX2, dW2 = run(case)
    assert torch.equal(dX1, dX2) and torch.equal(dW1, dW2)
    twice = synth.LinearCase(case.M, case.K, case.N, "bf16", (case.X.float() * 2).bfloat16(),
                             case.W, case.G)
    _, dW3 = run(twice, need_dx=False)
    assert torch.equal(dW3, dW1 * 2)


def test_non_default_stream():
    case = synth.linear_case(160, 264, 200, "bf16", seed=11)
    s = torch.cuda.Stream()
    dX, dW = run(case, stream=s)
    check_full(case, dX, dW)


def test_decode_like_m32_full_compare():
    """bf16 X[32,4096], W[4096,4096], G[32,4096]: every entry against the oracle."""
    case = synth.linear_m32(seed=0)
    dX, dW = run(case)
    check_full(case, dX, dW)


def check_full_with_bounds(case, dX, dW, bound_rows=256, seed=0):
    """Every entry against the oracle (the relative Frobenius bars over the whole tensors),
    then the per-element bound on `bound_rows` seeded whole rows of each output."""
    rX, rW = check_full(case, dX, dW)
    Xb, Wb, Gb = synth.bits(case.X), synth.bits(case.W), synth.bits(case.G)
    aX, aW, aG = (abs_bits(b, case.dtype) for b in (Xb, Wb, Gb))
    rng = np.random.default_rng(seed)
    if dX is not None:
        rows = np.unique(np.concatenate([rng.integers(0, case.M, bound_rows), [0, case.M - 1]]))
        assert_within_bound(host_f64(dX[torch.from_numpy(rows)]), rX[rows],
                            oracle.dx_rows(aG, aW, case.dtype, rows), case.N,
                            case.dtype == "bf16", "dX")
    if dW is not None:
        rows = np.unique(np.concatenate([rng.integers(0, case.K, bound_rows), [0, case.K - 1]]))
        assert_within_bound(host_f64(dW[torch.from_numpy(rows)]), rW[rows],
                            oracle.dw_rows(aX, aG, case.dtype, rows), case.M, False, "dW")
    return rX, rW


def test_large_m2048_full():
    """bf16 X[2048,4096], W[4096,4096], G[2048,4096]: every entry of dX and dW against the
    oracle, per-element bounds on 256 rows of each, and a second run bit for bit."""
    case = synth.linear_m2048(seed=0)
    dX, dW = run(case)
    check_full_with_bounds(case, dX, dW)
    dX2, dW2 = run(case)
    assert torch.equal(dX, dX2) and torch.equal(dW, dW2)


# The tile kernel starts the reduction of four groups of dX tiles (by tile column) 32
# slabs apart when the rows of dY and W are a multiple of 32 KiB apart (N = 16384):
# M > 1024 puts dX on the tile kernel, K > 512 gives tile columns with a nonzero start.
def test_rotated_dx_reduction_full():
    case = synth.linear_case(1040, 2056, 16384, "bf16", x_std=1.0, w_std=1.0, g_std=1.0, seed=41)
    dX, dW = run(case)
    check_full_with_bounds(case, dX, dW, bound_rows=64)


def test_rotated_dx_reduction_integer_inputs_are_exact():
    rng = np.random.default_rng(42)
    M, K, N = 1040, 776, 16384
    mk = lambda *sh: torch.tensor(rng.integers(-2, 3, size=sh), dtype=torch.float32).to(torch.bfloat16)
    case = synth.LinearCase(M, K, N, "bf16", mk(M, K), mk(K, N), mk(M, N))
    dX, dW = run(case)
    rX, rW = oracle.lin_bwd(synth.bits(case.X), synth.bits(case.W), synth.bits(case.G), "bf16")
    assert np.array_equal(dW.cpu().numpy(), rW.astype(np.float32))
    assert torch.equal(dX.cpu(), torch.from_numpy(rX.astype(np.float32)).to(torch.bfloat16))


def _rows_check(case, dX, dW, rows, seed):
    """Whole sampled rows of dX and dW against the oracle: the bars over the sample and the
    per-element bound of every entry."""
    Xb, Wb, Gb = synth.bits(case.X), synth.bits(case.W), synth.bits(case.G)
    aX, aW, aG = (abs_bits(b, "bf16") for b in (Xb, Wb, Gb))
    rng = np.random.default_rng(seed)
    r = np.unique(np.concatenate([rng.integers(0, case.M, rows), [0, case.M - 1]]))
    got = host_f64(dX[torch.from_numpy(r).to(dX.device)])
    ref = oracle.dx_rows(Gb, Wb, "bf16", r)
    assert relf(got, ref) <= DX_RELF, "dX rows relF %.3g" % relf(got, ref)
    assert_within_bound(got, ref, oracle.dx_rows(aG, aW, "bf16", r), case.N, True, "dX")
    r = np.unique(np.concatenate([rng.integers(0, case.K, rows), [0, case.K - 1]]))
    got = host_f64(dW[torch.from_numpy(r).to(dW.device)])
    ref = oracle.dw_rows(Xb, Gb, "bf16", r)
    assert relf(got, ref) <= DW_RELF, "dW rows relF %.3g" % relf(got, ref)
    assert_within_bound(got, ref, oracle.dw_rows(aX, aG, "bf16", r), case.M, False, "dW")


# Operands and outputs of 2 GiB and more stay on the MFMA kernels: every buffer
# descriptor covers only the rows its block reads or writes.  The path is forced,
# so a call that could not run there would be refused, not moved to the
# element-wise kernel.
#   (8, 32768, 32768)    W 2 GiB, dW 4 GiB: split-reduction dX and small-tile dW
#   (1040, 8, 2^20 + 8)  dY > 2 GiB: both products on the tile kernel
#   (65536, 16384, 8)    X 2 GiB and dX 2 GiB: the tile kernel
#   (1040, 32768, 32768) W 2 GiB, dW 4 GiB: the tile kernel
BIG_SHAPES = [(8, 32768, 32768), (1040, 8, (1 << 20) + 8), (65536, 16384, 8), (1040, 32768, 32768)]


@pytest.mark.parametrize("M,K,N", BIG_SHAPES)
def test_operands_of_2gib_and_more_stay_on_the_mfma_kernels(M, K, N):
    case = synth.linear_case(M, K, N, "bf16", x_std=1.0, w_std=0.02, g_std=1e-4, seed=31 + M)
    dX, dW = run(case, path=lb.LB_PATH_SMALL_M if M <= 256 else lb.LB_PATH_TILE)
    assert not torch.isnan(dX).any() and not torch.isnan(dW).any()
    if M * K * N <= (1 << 34):
        check_full_with_bounds(case, dX, dW, bound_rows=32)
    else:
        _rows_check(case, dX, dW, 32, M)


@pytest.mark.parametrize("proj", range(4))
def test_block_projection_full(proj):
    """One Transformer block's projections at M = 16384 (QKV, out, up, down): every entry of
    dX and dW against the oracle, per-element bounds on 64 rows of each."""
    name, k, n = synth.BLOCK_PROJECTIONS[proj]
    case = synth.linear_case(synth.BLOCK_TOKENS, k, n, "bf16", x_std=1.0, w_std=0.02,
                             g_std=1e-4, seed=1 + proj, name=name)
    dX, dW = run(case)
    check_full_with_bounds(case, dX, dW, bound_rows=64, seed=proj)
