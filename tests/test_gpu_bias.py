"""GPU parity of the bias gradient (lin_bwd_ex's db = Σ_m dY[m,:]) against the CPU oracle.

Bar (written in gpu_util): relative Frobenius error ≤ DB_RELF against the fp64
oracle, and per column |gpu − oracle| ≤ DB_ABS · Σ_m |dY[m,n]| (fp32 sums of
a few dozen terms, then fp64); bitwise on integer-valued inputs, whose sums
are exact in fp32.
"""
import numpy as np
import pytest
import torch

import linear_layer_backward_bwd_amd as lb
import oracle
import synth
from gpu_util import DB_ABS, DB_RELF, Guarded, bits, relf

pytestmark = pytest.mark.gpu
DEV = "cuda"


def gpu_db(G, offset=0):
    """db of a device copy of G placed offset elements into a buffer, into a guarded output."""
    M, N = G.shape
    buf = torch.empty(M * N + offset, dtype=G.dtype, device=DEV)
    g = buf[offset:].view(M, N)
    g.copy_(G.to(DEV))
    out = Guarded(1, N, torch.float32)
    lb.lin_bwd_ex(None, None, g, db=out.t.view(N))
    torch.cuda.synchronize()
    out.check_guards()
    return out.t.view(N).cpu().numpy()


def check(got, G, dtype):
    Gb = synth.bits(G.cpu())
    ref = oracle.bias_grad(Gb, dtype)
    colabs = np.abs(oracle.decode(Gb, dtype)).sum(axis=0)
    assert not np.isnan(got).any()
    assert relf(got, ref) <= DB_RELF, relf(got, ref)
    err = np.abs(got.astype(np.float64) - ref)
    assert (err <= DB_ABS * colabs + 1e-30).all(), float((err / np.maximum(colabs, 1e-30)).max())


@pytest.mark.parametrize("M,N", [(1, 1), (3, 7), (64, 512), (65, 513), (100, 4104), (1000, 1000),
                                 (1000, 1001), (2048, 4096), (4097, 520), (300, 16)])
def test_bf16_matches_oracle(M, N):
    G = synth.to_storage(synth.normal((M, N), 1e-4, synth._gen(M * 7 + N)), "bf16")
    check(gpu_db(G), G, "bf16")


@pytest.mark.parametrize("M,N", [(7, 5), (300, 260), (1000, 1028), (129, 3)])
def test_f32_matches_oracle(M, N):
    G = synth.normal((M, N), 1.0, synth._gen(M + N))
    check(gpu_db(G), G, "f32")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("offset", [1, 3])
def test_misaligned(dtype, offset):
    G = synth.to_storage(synth.normal((333, 1024), 1.0, synth._gen(offset)), dtype)
    check(gpu_db(G, offset=offset), G, dtype)


@pytest.mark.parametrize("M,N", [(5000, 4096), (1, 77), (16384, 520)])
def test_integer_values_exact(M, N):
    rng = np.random.default_rng(M + N)
    G = torch.tensor(rng.integers(-8, 9, size=(M, N)), dtype=torch.float32).to(torch.bfloat16)
    got = gpu_db(G)
    ref = oracle.bias_grad(synth.bits(G), "bf16")
    assert np.array_equal(got.astype(np.float64), ref)


def test_single_row_is_the_row():
    G = synth.to_storage(synth.normal((1, 4096), 1.0, synth._gen(5)), "bf16")
    assert np.array_equal(gpu_db(G), G.float().numpy()[0])


def test_empty_sum_writes_zeros():
    G = torch.empty(0, 300, dtype=torch.bfloat16)
    assert np.array_equal(gpu_db(G), np.zeros(300, np.float32))


@pytest.mark.parametrize("M,N", [(3, (1 << 20) + 8), (400, 200000)])
def test_wide_outputs(M, N):
    """Past 2^20 columns one row split remains and the first pass writes db itself;
    200000 columns: 391 strips of 512 columns, 3 row splits (the most partials a launch writes)."""
    G = synth.to_storage(synth.normal((M, N), 1.0, synth._gen(9)), "bf16")
    check(gpu_db(G), G, "bf16")


def test_repeatable_bit_for_bit():
    G = synth.to_storage(synth.normal((4096, 12288), 1e-4, synth._gen(10), ), "bf16").to(DEV)
    a = torch.empty(12288, device=DEV)
    b = torch.empty(12288, device=DEV)
    lb.lin_bwd_ex(None, None, G, db=a)
    lb.lin_bwd_ex(None, None, G, db=b)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))


def test_with_dx_dw_equals_lin_bwd():
    """lin_bwd_ex's dX and dW are lin_bwd's, bit for bit; db alongside them is right."""
    c = synth.linear_case(1000, 512, 1024, "bf16", seed=12, device=DEV)
    dX1 = torch.empty(1000, 512, dtype=torch.bfloat16, device=DEV)
    dW1 = torch.empty(512, 1024, device=DEV)
    dX2, dW2 = torch.empty_like(dX1), torch.empty_like(dW1)
    db = torch.full((1024,), float("nan"), device=DEV)
    lb.lin_bwd(c.X, c.W, c.G, dX1, dW1)
    lb.lin_bwd_ex(c.X, c.W, c.G, dX2, dW2, db)
    torch.cuda.synchronize()
    assert torch.equal(bits_t(dX1), bits_t(dX2)) and torch.equal(bits_t(dW1), bits_t(dW2))
    check(db.cpu().numpy(), c.G, "bf16")


# db requested together with dW (and dX or not), on the shapes where dW runs on the tile
# kernel (M > 256): partial last slab (M % 32), partial tile columns (N % 256), one and
# several tile columns.
@pytest.mark.parametrize("M,K,N,with_dx", [(300, 264, 1032, True), (1100, 520, 776, False),
                                           (4097, 264, 520, True), (2048, 4096, 4096, True),
                                           (257, 8, 8, False), (1000, 1024, 16, True)])
def test_db_with_dw(M, K, N, with_dx):
    c = synth.linear_case(M, K, N, "bf16", seed=M + N, device=DEV)
    dW = torch.empty(K, N, device=DEV)
    dX = torch.empty(M, K, dtype=torch.bfloat16, device=DEV) if with_dx else None
    db = Guarded(1, N, torch.float32)
    lb.lin_bwd_ex(c.X, c.W, c.G, dX, dW, db.t.view(N))
    torch.cuda.synchronize()
    db.check_guards()
    check(db.t.view(N).cpu().numpy(), c.G, "bf16")
    # and db requested alone
    alone = torch.empty(N, device=DEV)
    lb.lin_bwd_ex(None, None, c.G, db=alone)
    torch.cuda.synchronize()
    check(alone.cpu().numpy(), c.G, "bf16")


def test_db_with_dw_integer_inputs_exact():
    rng = np.random.default_rng(77)
    M, K, N = 5000, 264, 4104
    mk = lambda *sh: torch.tensor(rng.integers(-3, 4, size=sh), dtype=torch.float32).to(torch.bfloat16)
    c = synth.LinearCase(M, K, N, "bf16", mk(M, K), mk(K, N), mk(M, N))
    dW = torch.empty(K, N, device=DEV)
    db = torch.empty(N, device=DEV)
    lb.lin_bwd_ex(c.X.to(DEV), c.W.to(DEV), c.G.to(DEV), None, dW, db)
    torch.cuda.synchronize()
    ref = oracle.bias_grad(synth.bits(c.G), "bf16")
    assert np.array_equal(db.cpu().numpy(), ref.astype(np.float32))


def test_db_with_dw_block_projections():
    """The block's four projections (M = 16384) with dW and db: every column of db."""
    cases, _ = synth.block_case(seed=0, device=DEV)
    for c in cases:
        dW = torch.empty(c.K, c.N, device=DEV)
        db = torch.empty(c.N, device=DEV)
        lb.lin_bwd_ex(c.X, c.W, c.G, None, dW, db)
        torch.cuda.synchronize()
        check(db.cpu().numpy(), c.G, "bf16")


def bits_t(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def test_block_projections_full():
    """The block's four dY (M = 16384; N = 12288, 4096, 16384, 4096): every column."""
    cases, _ = synth.block_case(seed=0, device=DEV)
    for c in cases:
        db = torch.empty(c.N, device=DEV)
        lb.lin_bwd_ex(None, None, c.G, db=db)
        torch.cuda.synchronize()
        check(db.cpu().numpy(), c.G, "bf16")


def test_after_shutdown_the_workspace_is_allocated_again():
    G = synth.to_storage(synth.normal((3000, 2056), 1e-4, synth._gen(99)), "bf16")
    before = gpu_db(G)
    torch.cuda.synchronize()
    lb.lb_shutdown()
    after = gpu_db(G)
    check(after, G, "bf16")
    assert np.array_equal(np.asarray(before), np.asarray(after))
