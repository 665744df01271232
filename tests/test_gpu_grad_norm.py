"""GPU parity of grad_norm (norm of the unscaled gradient, clip factor, inf/NaN
flag) against the CPU oracle, and its use as the clip factor and skip flag of
adamw_step_ex.

Bar (written in gpu_util): the norm within NORM_ULP fp32 ulps of the oracle's
(both sum exact fp64 squares and round once, so only the fp64 summation order
differs); the clip factor equal, bit for bit, to the fp32 quotient of max_norm
by the GPU's own norm (or 1) and within CLIP_ULP ulps of the oracle's; the flag
identical.
"""
import math

import numpy as np
import pytest
import torch

import linear_layer_backward_bwd_amd as lb
import oracle
import synth
from gpu_util import CLIP_ULP, NORM_ULP, adamw_ok, ulp_distance_f32

pytestmark = pytest.mark.gpu
DEV = "cuda"


def gpu_norm(g, inv_scale, max_norm, offset=0):
    """grad_norm on a device copy of g placed offset elements into a buffer."""
    t = g.to(DEV)
    buf = torch.empty(t.numel() + offset, dtype=t.dtype, device=DEV)
    view = buf[offset:]
    view.copy_(t)
    out = torch.full((2,), float("nan"), dtype=torch.float32, device=DEV)
    found = torch.full((1,), -7, dtype=torch.int32, device=DEV)
    lb.grad_norm(view, inv_scale, max_norm, out=out, found_inf=found)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    return float(o[0]), float(o[1]), int(found.cpu().item())


def expected_clip(norm, max_norm):
    if max_norm > 0 and norm > np.float32(max_norm):
        return float(np.float32(max_norm) / np.float32(norm))
    return 1.0


def check(got, ref, max_norm):
    norm_g, clip_g, found_g = got
    norm_r, clip_r, found_r = ref
    assert found_g == int(found_r)
    if math.isnan(norm_r) or math.isinf(norm_r):
        assert (math.isnan(norm_g) and math.isnan(norm_r)) or norm_g == norm_r, (norm_g, norm_r)
    else:
        d = int(ulp_distance_f32(np.float32(norm_g), np.float32(norm_r)))
        assert d <= NORM_ULP, "norm %r vs oracle %r: %d ulps" % (norm_g, norm_r, d)
    assert clip_g == expected_clip(norm_g, max_norm)
    assert int(ulp_distance_f32(np.float32(clip_g), np.float32(clip_r))) <= CLIP_ULP


@pytest.mark.parametrize("gdtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("n", [0, 1, 7, 8, 9, 4096 + 5, 8192 * 3 + 1, 1000003])
def test_matches_oracle(gdtype, n):
    case = synth.adamw_case(n, gdtype, g_scale=1.0 if gdtype == "f32" else 1024.0, seed=31 + n)
    ref0 = oracle.grad_norm(synth.bits(case.g), gdtype, case.inv_scale)
    max_norm = 0.5 * ref0[0]
    got = gpu_norm(case.g, case.inv_scale, max_norm)
    ref = oracle.grad_norm(synth.bits(case.g), gdtype, case.inv_scale, max_norm)
    check(got, ref, max_norm)
    if n > 0:
        assert got[1] < 1.0


def test_clip_thresholds():
    case = synth.adamw_case(30011, "bf16", seed=32)
    g = synth.bits(case.g)
    norm = gpu_norm(case.g, case.inv_scale, 0.0)[0]
    below = float(np.nextafter(np.float32(norm), np.float32(0)))
    for max_norm in (0.0, -1.0, 2.0 * norm, norm, below, 1e-30, float("inf")):
        got = gpu_norm(case.g, case.inv_scale, max_norm)
        check(got, oracle.grad_norm(g, "bf16", case.inv_scale, max_norm), max_norm)
        if max_norm == below:
            assert got[1] < 1.0
        if max_norm in (0.0, -1.0, 2.0 * norm, norm, float("inf")):
            assert got[1] == 1.0


@pytest.mark.parametrize("gdtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("where", ["first", "middle", "last"])
@pytest.mark.parametrize("bad", [float("inf"), float("-inf"), float("nan")])
def test_found_inf(gdtype, where, bad):
    n = 50001
    case = synth.adamw_case(n, gdtype, seed=33)
    pos = {"first": 0, "middle": n // 2 + 3, "last": n - 1}[where]
    case.g[pos] = bad
    got = gpu_norm(case.g, case.inv_scale, 1.0)
    ref = oracle.grad_norm(synth.bits(case.g), gdtype, case.inv_scale, 1.0)
    assert ref[2] and got[2] == 1
    check(got, ref, 1.0)


def test_overflow_by_the_unscale_factor_is_flagged():
    g = torch.full((1000,), 1e-3, dtype=torch.float32)
    g[123] = 3e38
    got = gpu_norm(g, 4.0, 1.0)           # 3e38 * 4 is inf in fp32
    ref = oracle.grad_norm(synth.bits(g), "f32", 4.0, 1.0)
    assert ref[2] and got[2] == 1 and math.isinf(got[0])
    check(got, ref, 1.0)
    h = torch.full((4099,), 65504.0, dtype=torch.float16)  # largest finite fp16: no flag
    got = gpu_norm(h, 1.0, 0.0)
    check(got, oracle.grad_norm(synth.bits(h), "f16", 1.0, 0.0), 0.0)
    assert got[2] == 0


@pytest.mark.parametrize("value", [1e30, 1e-30])
def test_squares_beyond_fp32_range(value):
    """Squares of 1e30 overflow fp32 and of 1e-30 underflow it; the norm does neither."""
    n = 100000
    g = torch.full((n,), value, dtype=torch.float32)
    got = gpu_norm(g, 1.0, 0.0)
    check(got, oracle.grad_norm(synth.bits(g), "f32", 1.0, 0.0), 0.0)
    assert got[2] == 0
    assert abs(got[0] / (value * math.sqrt(n)) - 1.0) < 1e-6


@pytest.mark.parametrize("gdtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("offset", [1, 2, 3])
def test_misaligned(gdtype, offset):
    case = synth.adamw_case(10007, gdtype, seed=34)
    got = gpu_norm(case.g, case.inv_scale, 0.25, offset=offset)
    check(got, oracle.grad_norm(synth.bits(case.g), gdtype, case.inv_scale, 0.25), 0.25)


def test_repeatable_bit_for_bit():
    case = synth.adamw_case((1 << 24) + 77, "f16", seed=35, device=DEV)
    outs = []
    for _ in range(3):
        out, found = lb.grad_norm(case.g, case.inv_scale, 1e-3)
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy().view(np.uint32).copy())
    assert (outs[0] == outs[1]).all() and (outs[0] == outs[2]).all()


def test_2p28_fp16_full():
    """The 2^28-parameter fp16 gradient of the AdamW workload: many full grids."""
    case = synth.adamw_2p28(seed=1, device=DEV)
    out, found = lb.grad_norm(case.g, case.inv_scale, 1.0)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    ref = oracle.grad_norm(synth.bits(case.g.cpu()), "f16", case.inv_scale, 1.0)
    check((float(o[0]), float(o[1]), int(found.cpu().item())), ref, 1.0)


def test_several_rounds_per_block_f32():
    """2^27 + 2^20 + 5 fp32 gradients: more than one round of loads per block, ragged end."""
    n = (1 << 27) + (1 << 20) + 5
    case = synth.adamw_case(n, "f32", g_scale=1.0, seed=38, device=DEV)
    out, found = lb.grad_norm(case.g, 1.0, 0.5)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    ref = oracle.grad_norm(synth.bits(case.g.cpu()), "f32", 1.0, 0.5)
    check((float(o[0]), float(o[1]), int(found.cpu().item())), ref, 0.5)


@pytest.mark.parametrize("w16", [None, "bf16"])
def test_feeds_adamw_step_ex(w16):
    """grad_norm's clip factor and flag drive adamw_step_ex with no host round trip."""
    n = 200003
    case = synth.adamw_case(n, "f16", seed=36)
    ref_norm = oracle.grad_norm(synth.bits(case.g), "f16", case.inv_scale)[0]
    max_norm = 0.3 * ref_norm
    W, m, v, g = (t.to(DEV).clone() for t in (case.W, case.m, case.v, case.g))
    h = torch.empty(n, dtype=torch.bfloat16, device=DEV) if w16 else None
    out, found = lb.grad_norm(g, case.inv_scale, max_norm)
    lb.adamw_step_ex(W, g, m, v, case.lr, case.b1, case.b2, case.eps, case.wd, 2, case.inv_scale,
                     clip=out[1:2], skip=found, w16=h)
    torch.cuda.synchronize()
    clip = float(out[1].item())
    check((float(out[0].item()), clip, int(found.item())),
          oracle.grad_norm(synth.bits(case.g), "f16", case.inv_scale, max_norm), max_norm)
    ref = oracle.adamw_ex(case.W.numpy(), synth.bits(case.g), case.m.numpy(), case.v.numpy(),
                          "f16", case.lr, case.b1, case.b2, case.eps, case.wd, 2, case.inv_scale,
                          clip=clip, w16=w16)
    for name, a, b in zip("Wmv", (W, m, v), ref[:3]):
        ok, err = adamw_ok(a.cpu().numpy(), b)
        assert ok, "%s: max scaled error %.3g" % (name, err)


def test_found_inf_skips_adamw_step_ex():
    n = 4099
    case = synth.adamw_case(n, "bf16", seed=37)
    case.g[1000] = float("nan")
    W, m, v, g = (t.to(DEV).clone() for t in (case.W, case.m, case.v, case.g))
    out, found = lb.grad_norm(g, case.inv_scale, 1.0)
    lb.adamw_step_ex(W, g, m, v, case.lr, case.b1, case.b2, case.eps, case.wd, 1, case.inv_scale,
                     clip=out[1:2], skip=found)
    torch.cuda.synchronize()
    assert int(found.item()) == 1
    assert np.array_equal(W.cpu().numpy(), case.W.numpy())
    assert np.array_equal(m.cpu().numpy(), case.m.numpy())
    assert np.array_equal(v.cpu().numpy(), case.v.numpy())


def test_after_shutdown_the_workspace_is_allocated_again():
    case = synth.adamw_case(1 << 20, "f16", g_scale=1024.0, seed=77)
    ref = oracle.grad_norm(synth.bits(case.g), "f16", case.inv_scale, 1.0)
    before = gpu_norm(case.g, case.inv_scale, 1.0)
    torch.cuda.synchronize()
    lb.lb_shutdown()
    after = gpu_norm(case.g, case.inv_scale, 1.0)
    check(after, ref, 1.0)
    assert list(before) == list(after)
