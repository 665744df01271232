"""Pins for the oracle's softmax backward dX = P·(dY − Σ_j P_j·dY_j), CPU only.

P is the forward softmax of logits z ("GPU 优化实战 Part 2", section "Softmax 和
LayerNorm 的梯度（自定义内核）").  Each check ties the oracle to something other
than its own formula:

* finite differences of L(z) = Σ dY ⊙ softmax(z) with respect to every logit,
  the softmax evaluated forward in fp64 (the backward formula is never used);
* invariants: Σ_i dX_i = dot·(1 − Σ P), so rows of exact probabilities sum to
  zero; a constant dY gives zero; a one-hot P gives zero;
* a missing factor P or a flipped sign fails the finite difference.
"""
import numpy as np
import pytest

import oracle


def _softmax(z):
    e = np.exp(z - z.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def _fd_logits(z, dY, h=1e-5):
    """Central differences of L(z) = Σ dY·softmax(z) for every entry of z."""
    g = np.empty_like(z)
    for r in range(z.shape[0]):
        for i in range(z.shape[1]):
            zp, zm = z.copy(), z.copy()
            zp[r, i] += h
            zm[r, i] -= h
            g[r, i] = (np.sum(dY[r] * _softmax(zp[r])) - np.sum(dY[r] * _softmax(zm[r]))) / (2 * h)
    return g


@pytest.mark.parametrize("rows,cols", [(1, 1), (3, 5), (4, 17), (2, 64)])
def test_finite_difference_every_logit(rows, cols):
    rng = np.random.default_rng(rows * 100 + cols)
    z = rng.standard_normal((rows, cols)) * 2.0
    dY = rng.standard_normal((rows, cols))
    P = _softmax(z)
    # the oracle reads fp32 inputs: take P and dY as fp32 and difference those exact values
    P32, dY32 = P.astype(np.float32), dY.astype(np.float32)
    dX = oracle.softmax_bwd(P32, dY32, "f32")
    fd = _fd_logits(z, dY32.astype(np.float64))
    # the fd sees the fp64 P; the oracle sees P rounded to fp32 (relative 6e-8)
    scale = np.abs(P) * (np.abs(dY32) + np.sum(np.abs(P * dY32), axis=1, keepdims=True))
    assert np.all(np.abs(dX - fd) <= 1e-6 * scale + 1e-9), float(np.max(np.abs(dX - fd) - 1e-6 * scale))


def test_finite_difference_catches_planted_mistakes():
    rng = np.random.default_rng(1)
    z = rng.standard_normal((1, 6))
    dY = rng.standard_normal((1, 6))
    P = _softmax(z)
    fd = _fd_logits(z, dY)
    dot = np.sum(P * dY)
    assert np.max(np.abs((dY - dot) - fd)) > 1e-3           # factor P dropped
    assert np.max(np.abs(P * (dY + dot) - fd)) > 1e-3       # sign of the dot flipped
    assert np.max(np.abs(P * dY - fd)) > 1e-3               # dot term dropped
    assert np.max(np.abs(oracle.softmax_bwd(P.astype(np.float32), dY.astype(np.float32), "f32")
                         - fd)) < 1e-6


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_row_sums_follow_the_probability_mass(dtype):
    rng = np.random.default_rng(2)
    P = _softmax(rng.standard_normal((8, 300)))
    dY = rng.standard_normal((8, 300))
    import torch
    conv = {"f32": lambda a: a.astype(np.float32),
            "bf16": lambda a: torch.tensor(a, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16),
            "f16": lambda a: a.astype(np.float16).view(np.uint16)}[dtype]
    Pb, dYb = conv(P), conv(dY)
    Pd, dYd = oracle.decode(Pb, dtype), oracle.decode(dYb, dtype)
    dX = oracle.softmax_bwd(Pb, dYb, dtype)
    dot = np.sum(Pd * dYd, axis=1)
    expect = dot * (1.0 - Pd.sum(axis=1))
    assert np.allclose(dX.sum(axis=1), expect, rtol=0, atol=1e-12)


def test_constant_upstream_gradient_and_one_hot_rows():
    P = np.array([[0.25, 0.5, 0.125, 0.125], [0.0, 1.0, 0.0, 0.0]], np.float32)  # exact mass 1
    dY = np.full((2, 4), 3.0, np.float32)
    assert np.array_equal(oracle.softmax_bwd(P, dY, "f32"), np.zeros((2, 4)))
    dY2 = np.array([[1, 2, 3, 4], [5, -6, 7, 8]], np.float32)
    dX = oracle.softmax_bwd(P[1:], dY2[1:], "f32")
    assert np.array_equal(dX, np.zeros((1, 4)))


def test_empty():
    assert oracle.softmax_bwd(np.zeros((0, 5), np.float32), np.zeros((0, 5), np.float32), "f32").shape == (0, 5)
    assert oracle.softmax_bwd(np.zeros((3, 0), np.float32), np.zeros((3, 0), np.float32), "f32").shape == (3, 0)
