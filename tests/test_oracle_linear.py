"""Pins for the oracle's Linear backward (dX = G·Wᵀ, dW = Xᵀ·G), CPU only.

Each check ties the oracle to something other than its own formula:

* finite differences of the forward loss L(X, W) = Σ G ⊙ (X·W).  L is linear
  in X and in W, so the central difference equals the gradient exactly in exact
  arithmetic for any step h; in fp64 the only error is rounding of L.  Only the
  forward product is evaluated here, never the backward formulas.  This is the
  check the pages' definition calls for ("GPU 优化实战 Part 2", section
  "反向传播——Linear 层的梯度": dX and dW are the gradients of the forward
  product with respect to its two operands).
* brute force with Python integers on integer-valued inputs (exact);
* the exact bf16 / fp16 decoders against torch's and numpy's conversions over
  all 65536 bit patterns;
* empty sums (M = 0 gives dW = 0; N = 0 gives dX = 0).
"""
import numpy as np
import pytest
import torch

import oracle
import synth


def _loss(X, W, G):
    """Forward loss L = Σ_{m,n} G[m,n]·(X·W)[m,n] in fp64, plus a rounding scale."""
    Y = X @ W
    return float(np.sum(G * Y)), float(np.sum(np.abs(G) * (np.abs(X) @ np.abs(W))))


def _fd_dense(X, W, G, wrt, D, h=1.0):
    """Central difference of L along direction D in X (wrt='X') or W (wrt='W')."""
    if wrt == "X":
        lp, s1 = _loss(X + h * D, W, G)
        lm, s2 = _loss(X - h * D, W, G)
    else:
        lp, s1 = _loss(X, W + h * D, G)
        lm, s2 = _loss(X, W - h * D, G)
    return (lp - lm) / (2 * h), max(s1, s2)


@pytest.mark.parametrize("M,K,N,dtype", [(3, 5, 4, "f32"), (8, 12, 16, "bf16"),
                                         (7, 3, 9, "bf16"), (1, 6, 2, "f32")])
def test_finite_difference_every_entry(M, K, N, dtype):
    case = synth.linear_case(M, K, N, dtype, x_std=1.0, w_std=1.0, g_std=1.0, seed=M * 100 + K)
    Xb, Wb, Gb = synth.bits(case.X), synth.bits(case.W), synth.bits(case.G)
    dX, dW = oracle.lin_bwd(Xb, Wb, Gb, dtype)
    X, W, G = oracle.decode(Xb, dtype), oracle.decode(Wb, dtype), oracle.decode(Gb, dtype)
    for i in range(M):
        for j in range(K):
            E = np.zeros_like(X)
            E[i, j] = 1.0
            fd, scale = _fd_dense(X, W, G, "X", E)
            assert abs(fd - dX[i, j]) <= 1e-13 * scale + 1e-300, (i, j, fd, dX[i, j])
    for i in range(K):
        for j in range(N):
            E = np.zeros_like(W)
            E[i, j] = 1.0
            fd, scale = _fd_dense(X, W, G, "W", E)
            assert abs(fd - dW[i, j]) <= 1e-13 * scale + 1e-300, (i, j, fd, dW[i, j])


def test_finite_difference_tiny_f32_config():
    """The 64x64x64 fp32 workload: 64 random entries of each gradient, 16 dense directions."""
    case, _ = synth.tiny_f32(seed=0)
    Xb, Wb, Gb = synth.bits(case.X), synth.bits(case.W), synth.bits(case.G)
    dX, dW = oracle.lin_bwd(Xb, Wb, Gb, "f32")
    X, W, G = (a.astype(np.float64) for a in (Xb, Wb, Gb))
    rng = np.random.default_rng(1)
    for _ in range(64):
        i, j = rng.integers(0, 64, size=2)
        E = np.zeros_like(X)
        E[i, j] = 1.0
        fd, s = _fd_dense(X, W, G, "X", E)
        assert abs(fd - dX[i, j]) <= 1e-13 * s
        fd, s = _fd_dense(X, W, G, "W", E)
        assert abs(fd - dW[i, j]) <= 1e-13 * s
    for _ in range(16):
        D = rng.standard_normal((64, 64))
        fd, s = _fd_dense(X, W, G, "X", D)
        assert abs(fd - float(np.sum(dX * D))) <= 1e-12 * s * 8
        fd, s = _fd_dense(X, W, G, "W", D)
        assert abs(fd - float(np.sum(dW * D))) <= 1e-12 * s * 8


def test_finite_difference_catches_a_transposed_operand():
    """The pin is sharp: a transposed W in the dX product fails it (planted in a copy, on the CPU)."""
    case = synth.linear_case(4, 4, 4, "f32", x_std=1.0, w_std=1.0, g_std=1.0, seed=3)
    X, W, G = (synth.bits(t).astype(np.float64) for t in (case.X, case.W, case.G))
    wrong = G @ W          # should be G @ W.T
    E = np.zeros_like(X)
    E[1, 2] = 1.0
    fd, _ = _fd_dense(X, W, G, "X", E)
    assert abs(fd - wrong[1, 2]) > 1e-6


@pytest.mark.parametrize("M,K,N", [(5, 7, 3), (16, 9, 11)])
def test_integer_inputs_brute_force(M, K, N):
    """Integer values in {-2..2} are exact in bf16; Python ints give the exact sums."""
    rng = np.random.default_rng(M + K + N)
    Xi = rng.integers(-2, 3, size=(M, K))
    Wi = rng.integers(-2, 3, size=(K, N))
    Gi = rng.integers(-2, 3, size=(M, N))
    to_bf16 = lambda a: synth.bits(torch.tensor(a, dtype=torch.float32).to(torch.bfloat16))
    dX, dW = oracle.lin_bwd(to_bf16(Xi), to_bf16(Wi), to_bf16(Gi), "bf16")
    for m in range(M):
        for k in range(K):
            assert dX[m, k] == sum(int(Gi[m, n]) * int(Wi[k, n]) for n in range(N))
    for k in range(K):
        for n in range(N):
            assert dW[k, n] == sum(int(Xi[m, k]) * int(Gi[m, n]) for m in range(M))


def test_sampled_entries_match_full():
    case = synth.linear_case(37, 29, 41, "bf16", x_std=1.0, w_std=1.0, g_std=1.0, seed=5)
    Xb, Wb, Gb = synth.bits(case.X), synth.bits(case.W), synth.bits(case.G)
    dX, dW = oracle.lin_bwd(Xb, Wb, Gb, "bf16")
    rng = np.random.default_rng(0)
    r, c = rng.integers(0, 37, 50), rng.integers(0, 29, 50)
    assert np.array_equal(oracle.dx_at(Gb, Wb, "bf16", r, c), dX[r, c])
    r, c = rng.integers(0, 29, 50), rng.integers(0, 41, 50)
    assert np.array_equal(oracle.dw_at(Xb, Gb, "bf16", r, c), dW[r, c])


def test_empty_sums():
    z = lambda *s: np.zeros(s, dtype=np.float32)
    dX, dW = oracle.lin_bwd(z(0, 4), np.ones((4, 3), np.float32), z(0, 3), "f32")
    assert dX.shape == (0, 4) and dW.shape == (4, 3) and np.all(dW == 0.0)
    dX, dW = oracle.lin_bwd(np.ones((2, 4), np.float32), z(4, 0), z(2, 0), "f32")
    assert dX.shape == (2, 4) and np.all(dX == 0.0) and dW.shape == (4, 0)


def test_skip_flags():
    case = synth.linear_case(4, 5, 6, "f32", seed=9)
    Xb, Wb, Gb = synth.bits(case.X), synth.bits(case.W), synth.bits(case.G)
    dX, dW = oracle.lin_bwd(Xb, Wb, Gb, "f32", need_dx=False)
    assert dX is None and dW.shape == (5, 6)
    dX, dW = oracle.lin_bwd(Xb, Wb, Gb, "f32", need_dw=False)
    assert dW is None and dX.shape == (4, 5)


def test_bf16_decoder_all_patterns():
    allbits = np.arange(65536, dtype=np.uint16)
    got = oracle.decode(allbits, "bf16")
    ref = torch.from_numpy(allbits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_f16_decoder_all_patterns():
    allbits = np.arange(65536, dtype=np.uint16)
    got = oracle.decode(allbits, "f16")
    ref = allbits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_rejects_bad_shapes_and_samples():
    a = np.zeros((2, 3), np.float32)
    with pytest.raises(ValueError):
        oracle.lin_bwd(a, np.zeros((4, 3), np.float32), np.zeros((2, 3), np.float32), "f32")
    with pytest.raises(ValueError):
        oracle.dx_at(np.zeros((2, 3), np.float32), np.zeros((4, 3), np.float32), "f32", [2], [0])
    with pytest.raises(TypeError):
        oracle.lin_bwd(a.astype(np.float64), a, a, "f32")


@pytest.mark.parametrize("dtype", ["bf16", "f32", "f16"])
def test_whole_rows_equal_entry_by_entry_dot_products(dtype):
    """The whole-row functions (terms of one output row added side by side, used for the
    full tensors) against the entry-by-entry dot products: the same fp64 operations in the
    same order, so every entry must agree bit for bit -- at every position of a ragged shape
    and for each element type."""
    M, K, N = 23, 37, 31
    case = synth.linear_case(M, K, N, dtype, x_std=1.0, w_std=1.0, g_std=1.0, seed=17)
    Xb, Wb, Gb = synth.bits(case.X), synth.bits(case.W), synth.bits(case.G)
    dX, dW = oracle.lin_bwd(Xb, Wb, Gb, dtype)
    r, c = np.meshgrid(np.arange(M), np.arange(K), indexing="ij")
    assert np.array_equal(oracle.dx_at(Gb, Wb, dtype, r.ravel(), c.ravel()).reshape(M, K), dX)
    r, c = np.meshgrid(np.arange(K), np.arange(N), indexing="ij")
    assert np.array_equal(oracle.dw_at(Xb, Gb, dtype, r.ravel(), c.ravel()).reshape(K, N), dW)


def test_row_subsets_equal_the_full_tensors():
    """dx_rows / dw_rows on a shuffled subset with a repeated row give those rows of the full
    tensors, bit for bit; an out-of-range row is refused."""
    M, K, N = 19, 26, 33
    case = synth.linear_case(M, K, N, "bf16", x_std=1.0, w_std=1.0, g_std=1.0, seed=18)
    Xb, Wb, Gb = synth.bits(case.X), synth.bits(case.W), synth.bits(case.G)
    dX, dW = oracle.lin_bwd(Xb, Wb, Gb, "bf16")
    rows = np.array([M - 1, 0, 7, 7, 3])
    assert np.array_equal(oracle.dx_rows(Gb, Wb, "bf16", rows), dX[rows])
    rows = np.array([K - 1, 2, 2, 11])
    assert np.array_equal(oracle.dw_rows(Xb, Gb, "bf16", rows), dW[rows])
    assert oracle.dx_rows(Gb, Wb, "bf16", []).shape == (0, K)
    with pytest.raises(ValueError):
        oracle.dx_rows(Gb, Wb, "bf16", [M])
    with pytest.raises(ValueError):
        oracle.dw_rows(Xb, Gb, "bf16", [-1])
