"""Pins for the oracle's 16-bit roundings and its extended AdamW step.

The roundings are pinned to values fixed by IEEE 754 (binary16 and the
bfloat16 truncation of binary32, round to nearest, ties to even), then
cross-checked against library conversions the oracle does not use (numpy's
float32 -> float16 cast and torch's CPU float32 -> bfloat16 cast, both round
to nearest even).  The extended step is pinned to the plain step through its
definition: the clip factor multiplies the unscaled gradient, the skip flag
changes nothing, and the 16-bit copy is the rounding of the updated W.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

F = np.float32


def f32(bits):
    return np.array([bits], dtype=np.uint32).view(np.float32)[0]


# binary16: 1 sign, 5 exponent bits (bias 15), 10 fraction bits.
F16_GOLDEN = [
    (1.0, 0x3C00), (-2.0, 0xC000), (0.5, 0x3800), (0.1, 0x2E66),
    (65504.0, 0x7BFF),                 # largest finite
    (65519.0, 0x7BFF),                 # below the midpoint to 65536
    (65520.0, 0x7C00),                 # midpoint, 65504 has an odd fraction: ties to even = inf
    (2.0 ** -14, 0x0400),              # smallest normal
    (2.0 ** -24, 0x0001),              # smallest subnormal
    (2.0 ** -25, 0x0000),              # half of it: tie to even (0)
    (1.5 * 2.0 ** -25, 0x0001),
    (3 * 2.0 ** -25, 0x0002),          # 1.5 ulp: tie between 1 and 2, even is 2
    (1 + 2.0 ** -11, 0x3C00),          # tie, 1.0 is even
    (1 + 3 * 2.0 ** -11, 0x3C02),      # tie between 0x3C01 and 0x3C02: even
    (-0.0, 0x8000), (0.0, 0x0000),
    (float("inf"), 0x7C00), (float("-inf"), 0xFC00),
    (1e-9, 0x0000), (-1e10, 0xFC00),
]

# bfloat16: the upper half of binary32.
BF16_GOLDEN = [
    (1.0, 0x3F80), (-1.0, 0xBF80), (0.1, 0x3DCD), (3.140625, 0x4049),
    (1 + 2.0 ** -8, 0x3F80),           # tie, 0x3F80 even
    (1 + 3 * 2.0 ** -8, 0x3F82),       # tie, 0x3F81 odd: up
    (1 + 2.0 ** -8 + 2.0 ** -20, 0x3F81),  # just above the tie
    (f32(0x7F7FFFFF), 0x7F80),         # largest float rounds to inf
    (f32(0x7F7F7FFF), 0x7F7F),
    (f32(0x00000001), 0x0000),         # subnormal binary32
    (f32(0x00008000), 0x0000),         # tie, even
    (f32(0x00018000), 0x0002),         # tie, odd: up
    (-0.0, 0x8000), (float("inf"), 0x7F80), (float("-inf"), 0xFF80),
]


@pytest.mark.parametrize("x,bits", F16_GOLDEN)
def test_f16_golden(x, bits):
    assert int(oracle.round16(np.array([x], F), "f16")[0]) == bits


@pytest.mark.parametrize("x,bits", BF16_GOLDEN)
def test_bf16_golden(x, bits):
    assert int(oracle.round16(np.array([x], F), "bf16")[0]) == bits


def test_nan_stays_nan():
    x = np.array([np.nan, -np.nan, f32(0x7F800001), f32(0xFFC00001)], F)
    for dt, exp_mask, frac_mask in (("f16", 0x7C00, 0x03FF), ("bf16", 0x7F80, 0x007F)):
        b = oracle.round16(x, dt).astype(np.int64)
        assert ((b & exp_mask) == exp_mask).all() and ((b & frac_mask) != 0).all()


def _edge_and_random(seed):
    rng = np.random.default_rng(seed)
    parts = [
        rng.standard_normal(200000).astype(F),
        (rng.standard_normal(50000) * 1e4).astype(F),
        (rng.standard_normal(50000) * 1e-5).astype(F),
        rng.integers(0, 2 ** 32, 200000, dtype=np.uint64).astype(np.uint32).view(F),  # any pattern
    ]
    x = np.concatenate(parts)
    return x[~np.isnan(x)]


def test_f16_matches_numpy_cast():
    x = _edge_and_random(1)
    with np.errstate(over="ignore"):  # the cast overflows to inf, as intended
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(oracle.round16(x, "f16"), ref)


def test_bf16_matches_torch_cast():
    x = _edge_and_random(2)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.round16(x, "bf16"), ref)


# ---- the extended AdamW step -------------------------------------------------

def _case(n, gdtype, seed):
    return synth.adamw_case(n, gdtype, g_scale=1.0 if gdtype == "f32" else 1024.0, seed=seed)


def _plain(case):
    return (case.W.numpy(), synth.bits(case.g), case.m.numpy(), case.v.numpy())


@pytest.mark.parametrize("gdtype", ["f32", "f16", "bf16"])
def test_clip_multiplies_the_unscaled_gradient(gdtype):
    """clip c equals the plain step on the fp32 gradient fp32(fp32(g·inv_scale)·c)."""
    case = _case(4099, gdtype, 11)
    W, g, m, v = _plain(case)
    clip = 0.3718
    g32 = oracle.decode(g, gdtype).astype(F) if gdtype != "f32" else g.astype(F)
    g_eff = (g32 * F(case.inv_scale)) * F(clip)  # numpy float32: one IEEE rounding per op
    a = oracle.adamw_ex(W, g, m, v, gdtype, case.lr, case.b1, case.b2, case.eps, case.wd, 3,
                        case.inv_scale, clip=clip)
    b = oracle.adamw(W, g_eff, m, v, "f32", case.lr, case.b1, case.b2, case.eps, case.wd, 3, 1.0)
    for x, y in zip(a[:3], b):
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32))


def test_no_options_is_the_plain_step():
    case = _case(3001, "bf16", 12)
    W, g, m, v = _plain(case)
    a = oracle.adamw_ex(W, g, m, v, "bf16", case.lr, case.b1, case.b2, case.eps, case.wd, 5,
                        case.inv_scale)
    b = oracle.adamw(W, g, m, v, "bf16", case.lr, case.b1, case.b2, case.eps, case.wd, 5,
                     case.inv_scale)
    assert a[3] is None
    for x, y in zip(a[:3], b):
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32))


def test_skip_changes_nothing():
    case = _case(1001, "f16", 13)
    W, g, m, v = _plain(case)
    a = oracle.adamw_ex(W, g, m, v, "f16", case.lr, case.b1, case.b2, case.eps, case.wd, 2,
                        case.inv_scale, clip=0.5, skip=True, w16="bf16")
    for x, y in zip(a[:3], (W, m, v)):
        assert np.array_equal(x, y)
    assert not a[3].any()  # the 16-bit buffer was not written


@pytest.mark.parametrize("w16", ["bf16", "f16"])
def test_shadow_is_the_rounded_update(w16):
    case = _case(5003, "bf16", 14)
    W, g, m, v = _plain(case)
    Wn, _, _, W16 = oracle.adamw_ex(W, g, m, v, "bf16", case.lr, case.b1, case.b2, case.eps,
                                    case.wd, 7, case.inv_scale, w16=w16)
    ref = (torch.from_numpy(Wn).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
           if w16 == "bf16" else Wn.astype(np.float16).view(np.uint16))  # |W| < 65504 here
    assert np.array_equal(W16, ref)


def test_shadow_with_lr_zero_is_the_old_weight():
    W = np.array([1.0, -2.0, 0.1, 65504.0, 3.0e5], F)
    z = np.zeros(5, F)
    g = np.ones(5, F)
    _, _, _, h = oracle.adamw_ex(W, g, z, z, "f32", 0.0, 0.9, 0.999, 1e-8, 0.1, 1, 1.0, w16="f16")
    assert [int(x) for x in h] == [0x3C00, 0xC000, 0x2E66, 0x7BFF, 0x7C00]


def test_invalid_shadow_type_rejected():
    W = np.zeros(4, F)
    with pytest.raises(ValueError):
        oracle.adamw_ex(W, W, W, W, "f32", 1e-3, 0.9, 0.999, 1e-8, 0.0, 1, 1.0, w16="f32")
