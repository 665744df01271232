"""Pins for the oracle's gradient norm, clip factor and inf/NaN flag.

Closed forms (constant vectors, 3-4-5), the pages' clipping rule written out
(factor max_norm/norm only when the norm exceeds max_norm), and the fp64
accumulation checked against math.fsum of the same squares (an exactly
rounded sum) on inputs where an fp32 running sum would drift.
"""
import math

import numpy as np
import pytest

import oracle

F = np.float32


def test_three_four_five():
    norm, clip, bad = oracle.grad_norm(np.array([3, 4], F), "f32")
    assert (norm, clip, bad) == (5.0, 1.0, False)


@pytest.mark.parametrize("gtype", ["f32", "f16", "bf16"])
def test_constant_vector(gtype):
    n = 1 << 16                      # sqrt(n) = 256 exactly
    c = 0.75                         # exact in every format
    x = np.full(n, c, F)
    g = x if gtype == "f32" else oracle.round16(x, gtype)
    norm, clip, bad = oracle.grad_norm(g, gtype, inv_scale=1.0 / 1024)
    assert norm == np.float32(c / 1024 * 256)
    assert clip == 1.0 and not bad


def test_clip_factor_rule():
    g = np.array([3, 4], F)          # norm 5
    assert oracle.grad_norm(g, "f32", max_norm=2.5)[1] == 0.5
    assert oracle.grad_norm(g, "f32", max_norm=5.0)[1] == 1.0      # not above: no clipping
    assert oracle.grad_norm(g, "f32", max_norm=7.0)[1] == 1.0
    assert oracle.grad_norm(g, "f32", max_norm=0.0)[1] == 1.0      # disabled
    assert oracle.grad_norm(g, "f32", max_norm=-1.0)[1] == 1.0
    clip = oracle.grad_norm(np.array([1, 1, 1], F), "f32", max_norm=1.0)[1]
    assert clip == np.float32(1.0) / np.float32(math.sqrt(3))


def test_empty_gradient():
    assert oracle.grad_norm(np.zeros(0, F), "f32", max_norm=1.0) == (0.0, 1.0, False)


@pytest.mark.parametrize("bad", [np.inf, -np.inf, np.nan])
def test_found_inf(bad):
    g = np.ones(1000, F)
    g[517] = bad
    norm, _, found = oracle.grad_norm(g, "f32")
    assert found and not math.isfinite(norm)


def test_found_inf_after_unscale_only():
    # finite in fp16, but the unscaled value overflows fp32 only if inv_scale were huge:
    g = oracle.round16(np.array([65504.0, 1.0], F), "f16")
    assert not oracle.grad_norm(g, "f16", inv_scale=1.0)[2]
    assert oracle.grad_norm(g, "f16", inv_scale=1e36)[2]


def test_fp64_accumulation_against_fsum():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(1 << 20) * 1e-3).astype(F)
    x[::97] *= 1e3                                # a wide dynamic range
    inv = F(1.0 / 1024)
    g32 = x * inv                                 # the fp32 unscale, as the oracle does it
    ref = np.float32(math.sqrt(math.fsum(float(v) * float(v) for v in g32)))
    norm = oracle.grad_norm(x, "f32", inv_scale=float(inv))[0]
    assert abs(norm - ref) <= 1e-6 * ref          # fp64 vs exactly rounded: well inside an fp32 ulp
    f32_running = np.float32(0)
    for v in g32[:1 << 16]:
        f32_running = np.float32(f32_running + v * v)   # what the oracle must not do
    assert f32_running != np.float32(math.fsum(float(v) * float(v) for v in g32[:1 << 16]))


@pytest.mark.parametrize("x", [1e30, -1e30, 1e-30])
def test_squares_outside_fp32_range(x):
    """fp32 squares of 1e30 overflow and of 1e-30 underflow; the fp64 sum of four
    exact squares is 4x², whose root 2|x| is exact in fp32."""
    g = np.full(4, x, F)
    norm, clip, bad = oracle.grad_norm(g, "f32")
    assert norm == 2 * abs(float(np.float32(x)))
    assert not bad
    with np.errstate(over="ignore", under="ignore"):
        naive = np.sqrt(np.sum(g * g, dtype=np.float32))
    assert naive != np.float32(norm)
