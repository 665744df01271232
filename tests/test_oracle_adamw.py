"""Pins for the oracle's unscale + AdamW update, CPU only.

The update rule (pages: "GPU 优化实战 Part 2", section "AdamW 优化器——融合内核";
"Mastering LLM Training with CUDA and ROCm", section "AdamW Algorithm"):

    m_t = b1·m + (1-b1)·g          v_t = b2·v + (1-b2)·g²
    m̂ = m_t/(1-b1^t)               v̂ = v_t/(1-b2^t)
    W ← W − lr·( m̂/(√v̂+ε) + λ·W )

Independent pins used here, none of which re-runs the oracle's own loop:

* step-1 closed form from m = v = 0: m̂ = g, v̂ = g², so W₁ = W₀ − lr·(g/(|g|+ε) + λW₀);
* the two written forms of the decoupled update, and the factored form
  (1−lr·λ)W − lr·m̂/(√v̂+ε), agree in fp64 and with the oracle; the sign-flipped
  decay of the host C++ listing on the second page grows W and is rejected;
* constant-gradient trajectory: m_t = b1ᵗm₀ + (1−b1ᵗ)g, v_t = b2ᵗv₀ + (1−b2ᵗ)g²
  in closed form, W_T by the fp64 recurrence;
* special cases: lr = 0, wd = 0, b1 = b2 = 0, g = 0, ε placement, v ≥ 0;
* unscale by 2⁻¹⁰ of a 16-bit gradient equals the pre-scaled fp32 gradient bitwise
  ("GPU 优化实战 Part 2", section "混合精度训练（FP16 / BF16）");
* resume: 10 steps equal 5 + 5 with the state carried over, bitwise.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

F32_EPS = np.finfo(np.float32).eps


def _state(n, seed, g_std=1e-3, zero=False):
    c = synth.adamw_case(n, "f32", g_scale=1.0, g_std=g_std, seed=seed, zero_moments=zero)
    return c.W.numpy(), c.m.numpy(), c.v.numpy(), synth.bits(c.g)


def _close(a, b, rel):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return np.all(np.abs(a - b) <= rel * np.maximum(np.abs(b), 1e-30))


def _within(a, b, bound):
    """|a - b| <= bound elementwise (bound: the fp32 rounding budget of each entry)."""
    return np.all(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64)) <= bound)


def test_step1_closed_form():
    W0, m0, v0, g = _state(4096, seed=11, zero=True)
    lr, b1, b2, eps, wd = 1e-3, 0.9, 0.999, 1e-8, 0.01
    W1, m1, v1 = oracle.adamw(W0, g, m0, v0, "f32", lr, b1, b2, eps, wd, 1, 1.0)
    g64, W064 = g.astype(np.float64), W0.astype(np.float64)
    f = lambda x: float(np.float32(x))
    assert _close(m1, (1 - f(b1)) * g64, 4 * F32_EPS)
    assert _close(v1, (1 - f(b2)) * g64 * g64, 8 * F32_EPS)
    ref = W064 - f(lr) * (g64 / (np.abs(g64) + f(eps)) + f(wd) * W064)
    # W ≈ 0.02 and the step ≈ 1e-3: compare the change, relative
    assert _close(W1.astype(np.float64) - W064, ref - W064, 1e-4)
    assert np.max(np.abs(W1 - ref)) <= 4 * F32_EPS * np.max(np.abs(W064))


def _fp64_step(W, g, m, v, lr, b1, b2, eps, wd, t):
    m = b1 * m + (1 - b1) * g
    v = b2 * v + (1 - b2) * g * g
    mh, vh = m / (1 - b1 ** t), v / (1 - b2 ** t)
    u = mh / (np.sqrt(vh) + eps)
    forms = {
        "first_page": W - lr * (u + wd * W),
        "second_page_equation": W - lr * u - lr * wd * W,
        "factored": (1 - lr * wd) * W - lr * u,
        "sign_flipped_listing": W - (lr * u - lr * wd * W),
    }
    return forms, m, v


def test_written_forms_agree_and_sign_flip_is_rejected():
    W0, m0, v0, g = _state(8192, seed=12)
    hp = dict(lr=3e-4, b1=0.9, b2=0.95, eps=1e-8, wd=0.1)
    h = {k: float(np.float32(x)) for k, x in hp.items()}
    t = 7
    forms, m64, v64 = _fp64_step(W0.astype(np.float64), g.astype(np.float64), m0.astype(np.float64),
                                 v0.astype(np.float64), h["lr"], h["b1"], h["b2"], h["eps"], h["wd"], t)
    a, b, c = forms["first_page"], forms["second_page_equation"], forms["factored"]
    assert np.max(np.abs(a - b)) <= 1e-16 and np.max(np.abs(a - c)) <= 1e-16
    W1, m1, v1 = oracle.adamw(W0, g, m0, v0, "f32", step=t, inv_scale=1.0, **hp)
    # fp32 evaluation of b·x + (1-b)·y errs by a few ulps of the terms, not of the result
    g64 = g.astype(np.float64)
    m_terms = h["b1"] * np.abs(m0) + (1 - h["b1"]) * np.abs(g64)
    v_terms = h["b2"] * np.abs(v0) + (1 - h["b2"]) * g64 * g64
    assert _within(m1, m64, 4 * F32_EPS * m_terms) and _within(v1, v64, 4 * F32_EPS * v_terms)
    # change of W agrees with all three forms to fp32 rounding of W
    assert np.max(np.abs(W1 - a)) <= 2 * F32_EPS * np.max(np.abs(W0))
    # the flipped decay moves W by 2·lr·λ·W ≈ 1e-6 more: far outside fp32 rounding of W
    bad = forms["sign_flipped_listing"]
    assert np.max(np.abs(bad - a)) > 50 * np.max(np.abs(W1 - a))


def test_constant_gradient_trajectory_closed_form():
    W0, m0, v0, g = _state(4096, seed=13)
    lr, b1, b2, eps, wd = (float(np.float32(x)) for x in (3e-4, 0.9, 0.95, 1e-8, 0.1))
    W, m, v = W0, m0, v0
    T = 10
    for t in range(1, T + 1):
        W, m, v = oracle.adamw(W, g, m, v, "f32", lr, b1, b2, eps, wd, t, 1.0)
    g64, m064, v064 = g.astype(np.float64), m0.astype(np.float64), v0.astype(np.float64)
    mT = b1 ** T * m064 + (1 - b1 ** T) * g64
    vT = b2 ** T * v064 + (1 - b2 ** T) * g64 * g64
    # T steps of fp32 rounding, each a few ulps of the terms
    assert _within(m, mT, 4 * T * F32_EPS * (np.abs(m064) + np.abs(g64)))
    assert _within(v, vT, 4 * T * F32_EPS * (np.abs(v064) + g64 * g64))
    Wr = W0.astype(np.float64)
    for t in range(1, T + 1):
        mt = b1 ** t * m064 + (1 - b1 ** t) * g64
        vt = b2 ** t * v064 + (1 - b2 ** t) * g64 * g64
        u = (mt / (1 - b1 ** t)) / (np.sqrt(vt / (1 - b2 ** t)) + eps)
        Wr = (1 - lr * wd) * Wr - lr * u
    assert np.max(np.abs(W - Wr)) <= 2e-6 * max(1.0, float(np.max(np.abs(Wr))))
    # and sharper: within a few fp32 ulps of |W| per step
    assert np.max(np.abs(W - Wr)) <= 4 * T * F32_EPS * float(np.max(np.abs(Wr)))


def test_swapped_betas_are_caught_by_the_trajectory():
    """Planted on the CPU: exchanging b1 and b2 moves m far off the closed form."""
    W0, m0, v0, g = _state(1024, seed=14)
    _, m, _ = oracle.adamw(W0, g, m0, v0, "f32", 3e-4, 0.95, 0.9, 1e-8, 0.1, 1, 1.0)
    b1 = float(np.float32(0.9))
    m1 = b1 * m0.astype(np.float64) + (1 - b1) * g.astype(np.float64)
    assert not _close(m, m1, 1e-3)


def test_lr_zero_leaves_W_bitwise():
    W0, m0, v0, g = _state(2048, seed=15)
    W1, m1, v1 = oracle.adamw(W0, g, m0, v0, "f32", 0.0, 0.9, 0.95, 1e-8, 0.1, 3, 1.0)
    assert np.array_equal(W1, W0)
    assert not np.array_equal(m1, m0)


def test_wd_zero_is_plain_adam_and_betas_zero():
    W0, m0, v0, g = _state(2048, seed=16)
    lr, eps = float(np.float32(1e-3)), float(np.float32(1e-8))
    # b1 = b2 = 0: m = g, v = g², bias corrections 1
    W1, m1, v1 = oracle.adamw(W0, g, m0, v0, "f32", lr, 0.0, 0.0, eps, 0.0, 5, 1.0)
    assert np.array_equal(m1, g) and np.array_equal(v1, g * g)
    g64 = g.astype(np.float64)
    ref = W0.astype(np.float64) - lr * g64 / (np.abs(g64) + eps)
    assert np.max(np.abs(W1 - ref)) <= 2 * F32_EPS * np.max(np.abs(W0))


def test_zero_gradient_only_decays():
    W0, _, _, g = _state(2048, seed=17, zero=True)
    z = np.zeros_like(W0)
    lr, wd = 1e-2, 0.5
    W1, m1, v1 = oracle.adamw(W0, np.zeros_like(g), z, z, "f32", lr, 0.9, 0.95, 1e-8, wd, 1, 1.0)
    assert np.all(m1 == 0) and np.all(v1 == 0)
    f = lambda x: float(np.float32(x))
    ref = W0.astype(np.float64) * (1 - f(lr) * f(wd))
    assert _close(W1, ref, 2 * F32_EPS)


def test_decay_uses_the_old_weight():
    """With large lr·λ, decaying the new W instead of the old one is visibly different."""
    W0, m0, v0, g = _state(512, seed=18)
    lr, wd = 0.25, 0.5
    W1, _, _ = oracle.adamw(W0, g, m0, v0, "f32", lr, 0.9, 0.95, 1e-8, wd, 1, 1.0)
    forms, _, _ = _fp64_step(W0.astype(np.float64), g.astype(np.float64), m0.astype(np.float64),
                             v0.astype(np.float64), lr, float(np.float32(0.9)),
                             float(np.float32(0.95)), float(np.float32(1e-8)), wd, 1)
    assert _close(W1, forms["first_page"], 1e-5)


def test_eps_outside_the_square_root():
    """Tiny gradients make √v̂ comparable to ε: ε inside the root would differ by orders."""
    n = 256
    W0 = np.full(n, 0.5, np.float32)
    z = np.zeros(n, np.float32)
    g = np.full(n, 1e-8, np.float32)
    eps = 1e-8
    W1, _, _ = oracle.adamw(W0, g, z, z, "f32", 1e-3, 0.9, 0.999, eps, 0.0, 1, 1.0)
    f = lambda x: float(np.float32(x))
    outside = 0.5 - f(1e-3) * (f(1e-8) / (f(1e-8) + f(eps)))
    inside = 0.5 - f(1e-3) * (f(1e-8) / np.sqrt(f(1e-8) ** 2 + f(eps)))
    assert abs(float(W1[0]) - outside) <= 2 * F32_EPS
    assert abs(outside - inside) > 1e-4


def test_second_moment_stays_nonnegative():
    W0, m0, v0, g = _state(4096, seed=19, g_std=10.0)
    for t in range(1, 4):
        W0, m0, v0 = oracle.adamw(W0, g, m0, v0, "f32", 3e-4, 0.9, 0.95, 1e-8, 0.1, t, 1.0)
        assert np.all(v0 >= 0)


@pytest.mark.parametrize("gdtype", ["f16", "bf16"])
def test_unscale_is_exact_for_power_of_two(gdtype):
    n = 4096
    c = synth.adamw_case(n, gdtype, g_std=1e-3, g_scale=1024.0, seed=20)
    W0, m0, v0 = c.W.numpy(), c.m.numpy(), c.v.numpy()
    g16 = synth.bits(c.g)
    g32 = (c.g.to(torch.float32) * (1.0 / 1024.0)).numpy()   # exact: power-of-two scale
    a = oracle.adamw(W0, g16, m0, v0, gdtype, 3e-4, 0.9, 0.95, 1e-8, 0.1, 1, 1.0 / 1024.0)
    b = oracle.adamw(W0, g32, m0, v0, "f32", 3e-4, 0.9, 0.95, 1e-8, 0.1, 1, 1.0)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_resume_is_bitwise():
    W, m, v, g = _state(4096, seed=21)
    hp = (3e-4, 0.9, 0.95, 1e-8, 0.1)
    A = (W, m, v)
    for t in range(1, 11):
        A = oracle.adamw(A[0], g, A[1], A[2], "f32", *hp, t, 1.0)
    B = (W, m, v)
    for t in range(1, 6):
        B = oracle.adamw(B[0], g, B[1], B[2], "f32", *hp, t, 1.0)
    B = tuple(np.array(x, copy=True) for x in B)   # "checkpoint" and restore
    for t in range(6, 11):
        B = oracle.adamw(B[0], g, B[1], B[2], "f32", *hp, t, 1.0)
    for x, y in zip(A, B):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("bad", [dict(step=0), dict(b1=1.0), dict(b2=1.5), dict(b1=-0.1)])
def test_rejects_undefined_updates(bad):
    W, m, v, g = _state(16, seed=22)
    hp = dict(lr=1e-3, b1=0.9, b2=0.95, eps=1e-8, wd=0.0, step=1, inv_scale=1.0)
    hp.update(bad)
    with pytest.raises(ValueError):
        oracle.adamw(W, g, m, v, "f32", **hp)
