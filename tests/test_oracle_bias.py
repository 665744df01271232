"""Pins for the oracle's bias gradient db[n] = Σ_m G[m,n], CPU only.

The forward with a bias is Y = X·W + b with b added to every row ("GPU 优化实战
Part 2", section "反向传播——Linear 层的梯度").  Each check ties the oracle to
something other than its own formula:

* finite differences of the forward loss L(b) = Σ G ⊙ (X·W + 1·bᵀ), which is
  linear in b, so the central difference is the gradient up to the rounding of L;
  only the forward is evaluated;
* the bias as the weight row of an extra input column of ones: db equals the
  row of dW = Xᵀ·G that belongs to a column of X holding 1 in every row (a
  different oracle function, the dW product);
* brute force with Python integers on integer-valued inputs, and constant G;
* an axis mistake (summing over the columns) fails the finite difference;
* the empty sum (M = 0) is zero.
"""
import numpy as np
import pytest
import torch

import oracle
import synth


def _loss(X, W, b, G):
    Y = X @ W + b[None, :]
    return float(np.sum(G * Y)), float(np.sum(np.abs(G) * (np.abs(X) @ np.abs(W) + np.abs(b)[None, :])))


@pytest.mark.parametrize("M,K,N,dtype", [(3, 5, 4, "f32"), (8, 12, 16, "bf16"), (7, 3, 9, "f16"),
                                         (6, 4, 6, "bf16")])
def test_finite_difference_every_entry(M, K, N, dtype):
    case = synth.linear_case(M, K, N, dtype, x_std=1.0, w_std=1.0, g_std=1.0, seed=7 * M + N)
    Gb = synth.bits(case.G)
    db = oracle.bias_grad(Gb, dtype)
    assert db.shape == (N,)
    X = oracle.decode(synth.bits(case.X), dtype)
    W = oracle.decode(synth.bits(case.W), dtype)
    G = oracle.decode(Gb, dtype)
    b = np.random.default_rng(M).standard_normal(N)
    for n in range(N):
        e = np.zeros(N)
        e[n] = 1.0
        lp, s1 = _loss(X, W, b + e, G)
        lm, s2 = _loss(X, W, b - e, G)
        fd = (lp - lm) / 2.0
        assert abs(fd - db[n]) <= 1e-13 * max(s1, s2), (n, fd, db[n])


def test_finite_difference_catches_the_wrong_axis():
    """Summing a square G over its columns instead of its rows fails the pin (planted here)."""
    case = synth.linear_case(5, 3, 5, "f32", x_std=1.0, w_std=1.0, g_std=1.0, seed=11)
    X, W, G = (synth.bits(t).astype(np.float64) for t in (case.X, case.W, case.G))
    wrong = G.sum(axis=1)
    b = np.zeros(5)
    e = np.zeros(5)
    e[2] = 1.0
    fd = (_loss(X, W, b + e, G)[0] - _loss(X, W, b - e, G)[0]) / 2.0
    assert abs(fd - wrong[2]) > 1e-6
    assert abs(fd - oracle.bias_grad(synth.bits(case.G), "f32")[2]) < 1e-12


@pytest.mark.parametrize("M,N,dtype", [(9, 13, "bf16"), (64, 32, "f32"), (33, 7, "f16")])
def test_equals_dw_row_of_a_ones_column(M, N, dtype):
    case = synth.linear_case(M, 3, N, dtype, x_std=1.0, w_std=1.0, g_std=1.0, seed=M + N)
    X = synth.bits(case.X).copy()
    one = {"f32": np.float32(1.0), "bf16": np.uint16(0x3F80), "f16": np.uint16(0x3C00)}[dtype]
    X[:, 1] = one
    _, dW = oracle.lin_bwd(X, synth.bits(case.W), synth.bits(case.G), dtype, need_dx=False)
    db = oracle.bias_grad(synth.bits(case.G), dtype)
    assert np.array_equal(dW[1], db)


@pytest.mark.parametrize("M,N", [(5, 3), (17, 11), (1, 9)])
def test_integer_inputs_brute_force(M, N):
    rng = np.random.default_rng(M * N)
    Gi = rng.integers(-100, 101, size=(M, N))
    Gb = synth.bits(torch.tensor(Gi, dtype=torch.float32).to(torch.bfloat16))
    db = oracle.bias_grad(Gb, "bf16")
    for n in range(N):
        assert db[n] == sum(int(Gi[m, n]) for m in range(M))


def test_constant_gradient():
    G = np.full((1000, 6), 0.375, dtype=np.float32)
    assert np.array_equal(oracle.bias_grad(G, "f32"), np.full(6, 375.0))


def test_empty_sum_and_empty_output():
    assert np.array_equal(oracle.bias_grad(np.zeros((0, 4), np.float32), "f32"), np.zeros(4))
    assert oracle.bias_grad(np.zeros((3, 0), np.float32), "f32").shape == (0,)
