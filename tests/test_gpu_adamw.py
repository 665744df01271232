"""GPU parity of the fused unscale + AdamW entry points against the CPU oracle.

Bar (written in gpu_util): |gpu - oracle| <= 2e-6·max(1, |oracle|) for each of
W, m, v.  Both sides evaluate the same fp32 operation sequence with IEEE
division and square root and no contraction, so the distance in ulps is
reported and held to 16.
"""
import numpy as np
import pytest
import torch

import linear_layer_backward_bwd_amd as lb
import oracle
import synth
from gpu_util import adamw_ok, bits, ulp_distance_f32

pytestmark = pytest.mark.gpu
DEV = "cuda"


def gpu_steps(case, steps, offset=0):
    """Run the steps on the GPU; returns host copies of W, m, v."""
    def place(t):
        if offset == 0:
            return t.to(DEV).clone()
        buf = torch.empty(t.numel() + offset, dtype=t.dtype, device=DEV)
        view = buf[offset:]
        view.copy_(t.to(DEV))
        return view
    W, m, v, g = (place(t) for t in (case.W, case.m, case.v, case.g))
    for t in steps:
        lb.adamw_step(W, g, m, v, case.lr, case.b1, case.b2, case.eps, case.wd, t, case.inv_scale)
    torch.cuda.synchronize()
    return W.cpu().numpy(), m.cpu().numpy(), v.cpu().numpy()


def oracle_steps(case, steps, idx=None):
    W, m, v, g = case.W.numpy(), case.m.numpy(), case.v.numpy(), synth.bits(case.g)
    if idx is not None:
        W, m, v, g = W[idx], m[idx], v[idx], g[idx]
    for t in steps:
        W, m, v = oracle.adamw(W, g, m, v, case.gdtype, case.lr, case.b1, case.b2, case.eps,
                               case.wd, t, case.inv_scale)
    return W, m, v


def compare(got, ref):
    worst_ulp = 0
    for name, a, b in zip("Wmv", got, ref):
        ok, err = adamw_ok(a, b)
        assert ok, "%s: max scaled error %.3g" % (name, err)
        keep = ~(np.isnan(a) & np.isnan(b))   # NaN payloads differ between CPU and GPU
        if keep.any():
            worst_ulp = max(worst_ulp, int(ulp_distance_f32(a[keep], b[keep]).max()))
    assert worst_ulp <= 16, "max ulp distance %d" % worst_ulp
    return worst_ulp


@pytest.mark.parametrize("gdtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("n", [1, 7, 8, 4096 + 5, 1000003])
def test_grad_types_and_ragged_sizes(gdtype, n):
    g_scale = 1.0 if gdtype == "f32" else 1024.0
    case = synth.adamw_case(n, gdtype, g_scale=g_scale, seed=n % 97)
    steps = [1, 2, 3]
    compare(gpu_steps(case, steps), oracle_steps(case, steps))


@pytest.mark.parametrize("gdtype", ["f32", "f16"])
def test_misaligned_buffers(gdtype):
    case = synth.adamw_case(100003, gdtype, g_scale=1.0 if gdtype == "f32" else 1024.0, seed=3)
    compare(gpu_steps(case, [1, 2], offset=1), oracle_steps(case, [1, 2]))


def test_zero_moments_step1():
    case = synth.adamw_case(65536, "bf16", seed=4, zero_moments=True, lr=1e-3, b2=0.999, wd=0.01)
    compare(gpu_steps(case, [1]), oracle_steps(case, [1]))


def test_lr_zero_keeps_W_and_grad_untouched():
    case = synth.adamw_case(50000, "f16", seed=5, lr=0.0)
    g_dev = case.g.to(DEV)
    W = case.W.to(DEV).clone()
    m, v = case.m.to(DEV).clone(), case.v.to(DEV).clone()
    lb.adamw_step(W, g_dev, m, v, 0.0, case.b1, case.b2, case.eps, case.wd, 4, case.inv_scale)
    torch.cuda.synchronize()
    assert torch.equal(W.cpu(), case.W)
    assert torch.equal(g_dev.cpu(), case.g)


def test_nan_and_inf_propagate():
    case = synth.adamw_case(64, "f32", g_scale=1.0, seed=6)
    case.g[3] = float("nan")
    case.g[5] = float("inf")
    got = gpu_steps(case, [1])
    ref = oracle_steps(case, [1])
    compare(got, ref)
    assert np.isnan(got[0][3]) and np.isnan(ref[0][3])


def test_explicit_typed_entry_points():
    case = synth.adamw_case(4099, "f16", seed=7)
    W, m, v, g = (t.to(DEV).clone() for t in (case.W, case.m, case.v, case.g))
    lb.adamw_step_f16(W, g, m, v, case.lr, case.b1, case.b2, case.eps, case.wd, 1, case.inv_scale)
    torch.cuda.synchronize()
    compare((W.cpu().numpy(), m.cpu().numpy(), v.cpu().numpy()), oracle_steps(case, [1]))
    with pytest.raises(TypeError):
        lb.adamw_step_bf16(W, g, m, v, 1e-3, 0.9, 0.95, 1e-8, 0.0, 1)


def compare_large(got, ref, chunk=1 << 24):
    """compare() for arrays of hundreds of millions of entries: equal bit patterns pass at
    once; otherwise the bar and the ulp distance are checked chunk by chunk."""
    worst_ulp = 0
    for name, a, b in zip("Wmv", got, ref):
        if np.array_equal(a.view(np.uint32), b.view(np.uint32)):
            continue
        for lo in range(0, a.size, chunk):
            x, y = a[lo:lo + chunk], b[lo:lo + chunk]
            ok, err = adamw_ok(x, y)
            assert ok, "%s[%d:]: max scaled error %.3g" % (name, lo, err)
            keep = ~(np.isnan(x) & np.isnan(y))
            if keep.any():
                worst_ulp = max(worst_ulp, int(ulp_distance_f32(x[keep], y[keep]).max()))
    assert worst_ulp <= 16, "max ulp distance %d" % worst_ulp
    return worst_ulp


def test_adamw_2p28_ten_steps_full():
    """2^28 fp32 params, fp16 grads x1024, t = 1..10: every parameter of W, m and v after each
    step against the oracle's own ten steps."""
    n = 1 << 28
    case = synth.adamw_2p28(seed=0, n=n, device=DEV)
    W, m, v, g = case.W, case.m, case.v, case.g
    rW, rm, rv, gb = W.cpu().numpy(), m.cpu().numpy(), v.cpu().numpy(), synth.bits(g.cpu())
    for t in case.steps:
        lb.adamw_step(W, g, m, v, case.lr, case.b1, case.b2, case.eps, case.wd, t, case.inv_scale)
        rW, rm, rv = oracle.adamw(rW, gb, rm, rv, case.gdtype, case.lr, case.b1, case.b2, case.eps,
                                  case.wd, t, case.inv_scale)
        got = tuple(x.cpu().numpy() for x in (W, m, v))
        compare_large(got, (rW, rm, rv))


def test_block_optimizer_full():
    """The block's 201,326,592 params, bf16 grads x1024, step 100: every parameter."""
    cases, opt = synth.block_case(seed=0, device=DEV)
    del cases
    rW, rm, rv, gb = (opt.W.cpu().numpy(), opt.m.cpu().numpy(), opt.v.cpu().numpy(),
                      synth.bits(opt.g.cpu()))
    for t in opt.steps:
        lb.adamw_step(opt.W, opt.g, opt.m, opt.v, opt.lr, opt.b1, opt.b2, opt.eps, opt.wd, t,
                      opt.inv_scale)
        rW, rm, rv = oracle.adamw(rW, gb, rm, rv, opt.gdtype, opt.lr, opt.b1, opt.b2, opt.eps,
                                  opt.wd, t, opt.inv_scale)
    got = tuple(x.cpu().numpy() for x in (opt.W, opt.m, opt.v))
    compare_large(got, (rW, rm, rv))


def test_resume_from_host_copy_is_bitwise():
    """Ten steps in one go equal five steps, the state copied to the host and back into fresh
    device buffers (a checkpoint and restore), then five more -- bit for bit, for each
    gradient type."""
    for gdtype in ("f32", "f16", "bf16"):
        case = synth.adamw_case(100003, gdtype, g_scale=1.0 if gdtype == "f32" else 1024.0,
                                seed=12, steps=range(1, 11))
        straight = gpu_steps(case, range(1, 11))
        W, m, v = gpu_steps(case, range(1, 6))
        resumed = synth.AdamWCase(torch.from_numpy(W), torch.from_numpy(m), torch.from_numpy(v),
                                  case.g, case.gdtype, case.lr, case.b1, case.b2, case.eps,
                                  case.wd, case.inv_scale)
        again = gpu_steps(resumed, range(6, 11))
        for a, b in zip(straight, again):
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), gdtype
        compare(again, oracle_steps(case, range(1, 11)))


def test_run_twice_is_bitwise():
    case = synth.adamw_case(300001, "bf16", seed=8)
    a = gpu_steps(case, [1, 2])
    b = gpu_steps(case, [1, 2])
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


# ---- adamw_step_ex: clip factor, skip flag, 16-bit copy of the updated W ----

W16T = {"bf16": torch.bfloat16, "f16": torch.float16}


def _ex_gpu(case, step, clip=None, skip=None, w16=None, offset=0, w16_fill=0x1234):
    def place(t, dt=None):
        t = t.to(DEV)
        buf = torch.empty(t.numel() + offset, dtype=t.dtype, device=DEV)
        view = buf[offset:]
        view.copy_(t)
        return view
    W, m, v, g = (place(t) for t in (case.W, case.m, case.v, case.g))
    h = None
    if w16 is not None:
        hb = torch.full((W.numel() + offset,), w16_fill, dtype=torch.int16, device=DEV)
        h = hb[offset:].view(W16T[w16])
    c = torch.tensor([clip], dtype=torch.float32, device=DEV) if clip is not None else None
    s = torch.tensor([skip], dtype=torch.int32, device=DEV) if skip is not None else None
    lb.adamw_step_ex(W, g, m, v, case.lr, case.b1, case.b2, case.eps, case.wd, step,
                     case.inv_scale, clip=c, skip=s, w16=h)
    torch.cuda.synchronize()
    return (W.cpu().numpy(), m.cpu().numpy(), v.cpu().numpy(),
            None if h is None else bits(h))


def _ex_ref(case, step, clip=None, skip=False, w16=None):
    return oracle.adamw_ex(case.W.numpy(), synth.bits(case.g), case.m.numpy(), case.v.numpy(),
                           case.gdtype, case.lr, case.b1, case.b2, case.eps, case.wd, step,
                           case.inv_scale, clip=clip, skip=skip, w16=w16)


def _check_shadow(W_gpu, h_gpu, w16):
    """The 16-bit copy is the GPU's own updated W rounded to nearest even."""
    ref = oracle.round16(W_gpu, w16)
    nan = np.isnan(W_gpu)
    assert np.array_equal(h_gpu[~nan], ref[~nan])
    expm = 0x7F80 if w16 == "bf16" else 0x7C00
    assert ((h_gpu[nan].astype(np.int64) & expm) == expm).all()


@pytest.mark.parametrize("w16", [None, "bf16", "f16"])
@pytest.mark.parametrize("gdtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("clip", [None, 0.37, 1.0])
def test_ex_matches_oracle(gdtype, w16, clip):
    n = 100003
    case = synth.adamw_case(n, gdtype, g_scale=1.0 if gdtype == "f32" else 1024.0, seed=21)
    got = _ex_gpu(case, 4, clip=clip, skip=0 if clip == 1.0 else None, w16=w16)
    ref = _ex_ref(case, 4, clip=clip, w16=w16)
    compare(got[:3], ref[:3])
    if w16 is not None:
        _check_shadow(got[0], got[3], w16)
        assert np.array_equal(got[3], ref[3])  # GPU and oracle W agree bit for bit here


def test_ex_clip_one_equals_plain_step():
    case = synth.adamw_case(65539, "bf16", seed=22)
    a = _ex_gpu(case, 2, clip=1.0)
    b = gpu_steps(case, [2])
    for x, y in zip(a[:3], b):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("w16", [None, "bf16"])
def test_ex_skip_writes_nothing(w16):
    case = synth.adamw_case(70001, "f16", seed=23)
    got = _ex_gpu(case, 3, clip=0.5, skip=1, w16=w16, w16_fill=0x5A5A)
    assert np.array_equal(got[0], case.W.numpy())
    assert np.array_equal(got[1], case.m.numpy())
    assert np.array_equal(got[2], case.v.numpy())
    if w16 is not None:
        assert (got[3] == 0x5A5A).all()


@pytest.mark.parametrize("w16", ["bf16", "f16"])
@pytest.mark.parametrize("n", [1, 3, 4, 5, 4099])
def test_ex_ragged_and_misaligned(w16, n):
    case = synth.adamw_case(n, "bf16", seed=24 + n)
    for offset in (0, 1):
        got = _ex_gpu(case, 1, clip=0.8, w16=w16, offset=offset)
        ref = _ex_ref(case, 1, clip=0.8, w16=w16)
        compare(got[:3], ref[:3])
        _check_shadow(got[0], got[3], w16)


def test_ex_shadow_overflow_and_nan():
    case = synth.adamw_case(64, "f32", g_scale=1.0, seed=25)
    case.W[0] = 70000.0      # beyond fp16: the copy is inf
    case.W[1] = 65504.0
    case.g[2] = float("nan")
    got = _ex_gpu(case, 1, w16="f16")
    ref = _ex_ref(case, 1, w16="f16")
    compare(got[:3], ref[:3])
    _check_shadow(got[0], got[3], "f16")
    assert got[3][0] == 0x7C00


def test_ex_large_full():
    """2^26 params, fp16 gradients x1024, clip 0.61, bf16 copy: every parameter of W, m, v and
    every entry of the copy against the oracle."""
    n = 1 << 26
    case = synth.adamw_2p28(seed=1, n=n, device=DEV)
    before = tuple(t.cpu() for t in (case.W, case.m, case.v, case.g))
    h = torch.empty(n, dtype=torch.bfloat16, device=DEV)
    c = torch.tensor([0.61], dtype=torch.float32, device=DEV)
    lb.adamw_step_ex(case.W, case.g, case.m, case.v, case.lr, case.b1, case.b2, case.eps, case.wd,
                     5, case.inv_scale, clip=c, w16=h)
    torch.cuda.synchronize()
    ref = oracle.adamw_ex(before[0].numpy(), synth.bits(before[3]), before[1].numpy(),
                          before[2].numpy(), case.gdtype, case.lr, case.b1, case.b2, case.eps,
                          case.wd, 5, case.inv_scale, clip=0.61, w16="bf16")
    got = tuple(t.cpu().numpy() for t in (case.W, case.m, case.v))
    compare_large(got, ref[:3])
    _check_shadow(got[0], bits(h), "bf16")
