"""Seeded synthetic inputs for the Linear backward + AdamW path.

This module holds no arithmetic of the method: it only draws normal variates
and rounds them to the storage dtype.  Both the HIP path (through the tests
and the bench) and the CPU oracle receive the same bytes from it.

Recipe (every workload):

* one ``torch.Generator`` seeded with ``seed`` (0 by default), on the CPU
  unless a ``device`` is named (the bench draws its large inputs on the GPU
  for speed: same distributions, a different stream of numbers);
* float32 standard-normal draws with ``torch.randn``, in the documented
  order, each multiplied by its standard deviation ``s`` ("N(0, s)" means
  standard deviation s throughout);
* rounding to bf16 / fp16 by torch's float32 -> 16-bit conversion, which
  rounds to nearest even.

The shapes and scales follow the pages' workload: a Transformer-training
Linear layer with batch and sequence flattened into M ("GPU 如何训练模型：从算子到
Kernel", section "一个线性层，前向和反向到底在算什么"; its roofline example uses
bf16 with K = N = 4096 at M = 32 and M = 2048), and a loss scale of 1024
("GPU 优化实战 Part 2", section "混合精度训练（FP16 / BF16）").
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

LOSS_SCALE = 1024.0


def _gen(seed: int, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def normal(shape, std: float, gen: torch.Generator) -> torch.Tensor:
    """float32 N(0, std) draws of the given shape (std is a standard deviation)."""
    return torch.randn(tuple(shape), generator=gen, dtype=torch.float32,
                       device=gen.device) * std


def to_storage(t: torch.Tensor, dtype: str) -> torch.Tensor:
    """Round float32 values to the storage dtype (round-to-nearest-even)."""
    return {"f32": lambda x: x.contiguous(),
            "bf16": lambda x: x.to(torch.bfloat16),
            "f16": lambda x: x.to(torch.float16)}[dtype](t)


def bits(t: torch.Tensor):
    """numpy view of a CPU tensor's raw elements: float32, or 16-bit patterns as uint16."""
    t = t.contiguous()
    if t.dtype == torch.float32:
        return t.numpy()
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16).numpy().view("uint16")
    raise TypeError("unsupported dtype %s" % t.dtype)


@dataclass
class LinearCase:
    """One Linear-backward problem: X[M,K], W[K,N], G[M,N] in the storage dtype."""
    M: int
    K: int
    N: int
    dtype: str
    X: torch.Tensor
    W: torch.Tensor
    G: torch.Tensor
    W_master: torch.Tensor | None = None   # fp32 master of W when W is 16-bit
    name: str = ""


def linear_case(M, K, N, dtype="bf16", x_std=1.0 / 4096, w_std=1.0 / 4096,
                g_std=1e-4, seed=0, name="", w_master=False, device="cpu") -> LinearCase:
    """Draw order: X, W, G."""
    gen = _gen(seed, device)
    X = to_storage(normal((M, K), x_std, gen), dtype)
    Wm = normal((K, N), w_std, gen)
    W = to_storage(Wm, dtype)
    G = to_storage(normal((M, N), g_std, gen), dtype)
    return LinearCase(M, K, N, dtype, X, W, G, Wm if w_master else None, name)


@dataclass
class AdamWCase:
    """Optimizer state and one gradient buffer; hyper-parameters for steps 1..T."""
    W: torch.Tensor          # fp32 master weights
    m: torch.Tensor          # fp32
    v: torch.Tensor          # fp32, >= 0
    g: torch.Tensor          # loss-scaled gradient in gdtype
    gdtype: str
    lr: float
    b1: float
    b2: float
    eps: float
    wd: float
    inv_scale: float
    steps: list = field(default_factory=lambda: [1])


def adamw_case(n, gdtype="f16", w_std=0.02, m_std=1e-3, v_std=1e-6, g_std=1e-3,
               g_scale=LOSS_SCALE, lr=3e-4, b1=0.9, b2=0.95, eps=1e-8, wd=0.1,
               steps=(1,), seed=0, zero_moments=False, W=None, device="cpu") -> AdamWCase:
    """Draw order: W (unless given), m, v (absolute value), g (times g_scale, then rounded)."""
    gen = _gen(seed, device)
    W = normal((n,), w_std, gen) if W is None else W.reshape(-1).to(torch.float32)
    if zero_moments:
        m = torch.zeros(n, dtype=torch.float32, device=gen.device)
        v = torch.zeros(n, dtype=torch.float32, device=gen.device)
    else:
        m = normal((n,), m_std, gen)
        v = normal((n,), v_std, gen).abs()
    g = to_storage(normal((n,), g_std, gen) * g_scale, gdtype)
    return AdamWCase(W, m, v, g, gdtype, lr, b1, b2, eps, wd, 1.0 / g_scale, list(steps))


# ---- the five named workloads ------------------------------------------------

#: one Transformer block's projections (in_features, out_features), in draw order
BLOCK_PROJECTIONS = (("qkv", 4096, 12288), ("out", 4096, 4096),
                     ("up", 4096, 16384), ("down", 16384, 4096))
BLOCK_TOKENS = 16384  # B = 8, S = 2048 flattened


def tiny_f32(seed=0):
    """64x64x64 fp32 Linear backward, then one AdamW step on W with g = dW."""
    case = linear_case(64, 64, 64, "f32", x_std=1.0 / 64, w_std=1.0 / 64, g_std=0.01,
                       seed=seed, name="tiny_f32_64")
    hp = dict(lr=1e-3, b1=0.9, b2=0.999, eps=1e-8, wd=0.01, inv_scale=1.0, step=1)
    return case, hp


def adamw_2p28(seed=0, n=1 << 28, device="cpu"):
    """AdamW over n fp32 params (2^28 by default), fp16 grads scaled by 1024, t = 1..10."""
    return adamw_case(n, "f16", lr=3e-4, b1=0.9, b2=0.95, eps=1e-8, wd=0.1,
                      steps=range(1, 11), seed=seed, device=device)


def linear_m32(seed=0, device="cpu"):
    return linear_case(32, 4096, 4096, "bf16", seed=seed, name="lin_bwd_M32_K4096_N4096",
                       device=device)


def linear_m2048(seed=0, device="cpu"):
    return linear_case(2048, 4096, 4096, "bf16", seed=seed, name="lin_bwd_M2048_K4096_N4096",
                       device=device)


def block_case(seed=0, tokens=BLOCK_TOKENS, projections=BLOCK_PROJECTIONS, device="cpu"):
    """One block's four projections (X ~ N(0,1), W master ~ N(0,0.02), G ~ N(0,1e-4)),
    then the AdamW state over all their parameters, concatenated in projection order.

    Each projection draws from its own generator seeded ``seed + 1 + index``;
    the AdamW m, v and g draw from ``seed``; its W is the projections' fp32
    masters, concatenated.  The bf16 gradients are a synthetic
    draw with the scale of these dW (std sqrt(M)·1e-4) times the loss scale 1024.
    """
    cases = [linear_case(tokens, k, n, "bf16", x_std=1.0, w_std=0.02, g_std=1e-4,
                         seed=seed + 1 + i, name=name, w_master=True, device=device)
             for i, (name, k, n) in enumerate(projections)]
    n_params = sum(k * n for _, k, n in projections)
    dw_std = (tokens ** 0.5) * 1e-4
    # the optimizer's master weights are the projections' masters, concatenated
    masters = torch.cat([c.W_master.reshape(-1) for c in cases])
    opt = adamw_case(n_params, "bf16", m_std=1e-3, v_std=1e-6, g_std=dw_std,
                     lr=3e-4, b1=0.9, b2=0.95, eps=1e-8, wd=0.1, steps=[100], seed=seed,
                     W=masters, device=device)
    return cases, opt


# ---- softmax backward --------------------------------------------------------

#: attention probabilities of one block: batch 8 x 32 heads x 2048 query rows, 2048 keys
SOFTMAX_ROWS = 8 * 32 * 2048
SOFTMAX_COLS = 2048


def softmax_case(rows, cols, dtype="bf16", z_std=1.0, dy_std=1.0, seed=0, device="cpu"):
    """(P, dY): P = row softmax of logits z ~ N(0, z_std) computed in fp32, dY ~ N(0, dy_std),
    both rounded to dtype.  Draw order: z, dY.  (No causal mask: every row is dense.)"""
    gen = _gen(seed, device)
    z = normal((rows, cols), z_std, gen)
    P = to_storage(torch.softmax(z, dim=1), dtype)
    del z
    dY = to_storage(normal((rows, cols), dy_std, gen), dtype)
    return P, dY
