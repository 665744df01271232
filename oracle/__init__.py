"""CPU oracle for the Linear-layer backward and the fused unscale + AdamW update.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may import this package; the product path never
does.  It shares no code with the HIP library.  The arithmetic lives in
``oracle.c`` (plain C, gcc, ``-O2 -ffp-contract=off``); this module only loads
it and moves numpy arrays in and out.

Definitions followed (cited by page title and section):

* dX = G·Wᵀ and dW = Xᵀ·G for a Linear layer Y = X·W -- "GPU 优化实战 Part 2",
  section "反向传播——Linear 层的梯度"; "GPU 如何训练模型：从算子到 Kernel",
  section "一个线性层，前向和反向到底在算什么".  Evaluated in fp64 on the exact
  decoded inputs.
* db = sum of G over rows for the bias of Y = X·W + b -- "GPU 优化实战 Part 2",
  section "反向传播——Linear 层的梯度" (the forward with a bias).  fp64.
* softmax backward dX = P·(dY − Σ P·dY) per row -- "GPU 优化实战 Part 2", section
  "Softmax 和 LayerNorm 的梯度（自定义内核）".  fp64.
* unscale + AdamW with decoupled weight decay -- "GPU 优化实战 Part 2", sections
  "AdamW 优化器——融合内核" and "混合精度训练（FP16 / BF16）"; "Mastering LLM
  Training with CUDA and ROCm", section "AdamW Algorithm".  Scalar fp32 loop.

Every function is pinned by the ``-m "not gpu"`` tests in ``tests/test_oracle_*.py``
(finite differences, closed forms, special cases, exact integer cases).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

F32, BF16, F16 = 0, 1, 2
_DTYPES = {"f32": F32, "bf16": BF16, "f16": F16}

_lib = None


def build() -> str:
    """Compile oracle.c with gcc into liboracle.so (IEEE scalar float, no contraction)."""
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-ftree-vectorize", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-std=c11", "-Wall", "-Wextra", "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
    lib.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_f64.restype = ctypes.c_double
    lib.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
    lib.oracle_f16_to_f64.restype = ctypes.c_double
    lib.oracle_decode.argtypes = [vp, i32, i64, vp]
    lib.oracle_decode.restype = None
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = i32
    for name in ("oracle_dx", "oracle_dw"):
        fn = getattr(lib, name)
        fn.argtypes = [vp, vp, i32, i64, i64, i64, vp]
    lib.oracle_dx.restype = i32
    lib.oracle_dw.restype = None
    for name in ("oracle_dx_rows", "oracle_dw_rows"):
        fn = getattr(lib, name)
        fn.argtypes = [vp, vp, i32, i64, i64, i64, vp, i64, vp]
    lib.oracle_dx_rows.restype = i32
    lib.oracle_dw_rows.restype = None
    for name in ("oracle_dx_at", "oracle_dw_at"):
        fn = getattr(lib, name)
        fn.argtypes = [vp, vp, i32, i64, i64, i64, vp, vp, i64, vp]
        fn.restype = None
    lib.oracle_adamw.argtypes = [vp, vp, i32, vp, vp, i64,
                                 f32, f32, f32, f32, f32, i32, f32]
    lib.oracle_adamw.restype = i32
    lib.oracle_adamw_ex.argtypes = [vp, vp, i32, vp, vp, i64, f32, f32, f32, f32, f32, i32, f32,
                                    vp, i32, vp, i32]
    lib.oracle_adamw_ex.restype = i32
    lib.oracle_f32_to_bf16.argtypes = [f32]
    lib.oracle_f32_to_bf16.restype = ctypes.c_uint16
    lib.oracle_f32_to_f16.argtypes = [f32]
    lib.oracle_f32_to_f16.restype = ctypes.c_uint16
    lib.oracle_grad_norm.argtypes = [vp, i32, i64, f32, f32, vp, vp]
    lib.oracle_db.argtypes = [vp, i32, i64, i64, vp]
    lib.oracle_db.restype = None
    lib.oracle_softmax_bwd.argtypes = [vp, vp, i32, i64, i64, vp]
    lib.oracle_softmax_bwd.restype = None
    lib.oracle_grad_norm.restype = None
    lib.oracle_round16.argtypes = [vp, i64, i32, vp]
    lib.oracle_round16.restype = None
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _as_input(a, dtype: str) -> np.ndarray:
    """The caller's raw element buffer: float32 values, or 16-bit patterns as uint16."""
    a = np.ascontiguousarray(a)
    if dtype == "f32":
        if a.dtype != np.float32:
            raise TypeError("f32 input must be a float32 array")
    else:
        if a.dtype != np.uint16:
            raise TypeError("%s input must hold the 16-bit patterns as uint16" % dtype)
    return a


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def bf16_to_f64(bits: int) -> float:
    return float(_load().oracle_bf16_to_f64(bits))


def f16_to_f64(bits: int) -> float:
    return float(_load().oracle_f16_to_f64(bits))


def decode(a, dtype: str) -> np.ndarray:
    """Exact widening of an f32 / bf16 / f16 buffer to float64."""
    a = _as_input(a, dtype)
    out = np.empty(a.shape, dtype=np.float64)
    _load().oracle_decode(_ptr(a), _DTYPES[dtype], a.size, _ptr(out))
    return out


def lin_bwd(X, W, G, dtype: str, need_dx: bool = True, need_dw: bool = True):
    """(dX, dW) in float64 for X[M,K], W[K,N], G[M,N]; either may be skipped (None)."""
    X, W, G = (_as_input(a, dtype) for a in (X, W, G))
    M, K = X.shape
    K2, N = W.shape
    if K2 != K or G.shape != (M, N):
        raise ValueError("shape mismatch: X%s W%s G%s" % (X.shape, W.shape, G.shape))
    lib = _load()
    dX = dW = None
    if need_dx:
        dX = np.empty((M, K), dtype=np.float64)
        if lib.oracle_dx(_ptr(G), _ptr(W), _DTYPES[dtype], M, K, N, _ptr(dX)) != 0:
            raise MemoryError("oracle_dx: no host memory for the copy of W")
    if need_dw:
        dW = np.empty((K, N), dtype=np.float64)
        lib.oracle_dw(_ptr(X), _ptr(G), _DTYPES[dtype], M, K, N, _ptr(dW))
    return dX, dW


def bias_grad(G, dtype: str) -> np.ndarray:
    """db[n] = sum over rows m of G[m, n], in float64, for G[M,N]."""
    G = _as_input(G, dtype)
    if G.ndim != 2:
        raise ValueError("G must be 2-D")
    M, N = G.shape
    db = np.empty(N, dtype=np.float64)
    _load().oracle_db(_ptr(G), _DTYPES[dtype], M, N, _ptr(db))
    return db


def softmax_bwd(P, dY, dtype: str) -> np.ndarray:
    """dX = P * (dY - rowsum(P * dY)) in float64 for row-major P, dY [rows, cols]."""
    P, dY = _as_input(P, dtype), _as_input(dY, dtype)
    if P.ndim != 2 or P.shape != dY.shape:
        raise ValueError("P and dY must be 2-D of one shape")
    rows, cols = P.shape
    dX = np.empty((rows, cols), dtype=np.float64)
    _load().oracle_softmax_bwd(_ptr(P), _ptr(dY), _DTYPES[dtype], rows, cols, _ptr(dX))
    return dX


def _row_list(rows, limit):
    rows = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1)
    if rows.size and (rows.min() < 0 or rows.max() >= limit):
        raise ValueError("row index out of range")
    return rows


def dx_rows(G, W, dtype: str, rows) -> np.ndarray:
    """Whole rows of dX = G·Wᵀ in float64: out[i, :] = dX[rows[i], :] (shape len(rows) x K)."""
    G, W = _as_input(G, dtype), _as_input(W, dtype)
    M, N = G.shape
    K = W.shape[0]
    if W.shape[1] != N:
        raise ValueError("shape mismatch: G%s W%s" % (G.shape, W.shape))
    rows = _row_list(rows, M)
    out = np.empty((rows.size, K), dtype=np.float64)
    if _load().oracle_dx_rows(_ptr(G), _ptr(W), _DTYPES[dtype], M, K, N, _ptr(rows), rows.size,
                              _ptr(out)) != 0:
        raise MemoryError("oracle_dx_rows: no host memory for the copy of W")
    return out


def dw_rows(X, G, dtype: str, rows) -> np.ndarray:
    """Whole rows of dW = Xᵀ·G in float64: out[i, :] = dW[rows[i], :] (shape len(rows) x N)."""
    X, G = _as_input(X, dtype), _as_input(G, dtype)
    M, K = X.shape
    N = G.shape[1]
    if G.shape[0] != M:
        raise ValueError("shape mismatch: X%s G%s" % (X.shape, G.shape))
    rows = _row_list(rows, K)
    out = np.empty((rows.size, N), dtype=np.float64)
    _load().oracle_dw_rows(_ptr(X), _ptr(G), _DTYPES[dtype], M, K, N, _ptr(rows), rows.size,
                           _ptr(out))
    return out


def dx_at(G, W, dtype: str, rows, cols) -> np.ndarray:
    """dX[rows[i], cols[i]] in float64, each computed on its own."""
    G, W = _as_input(G, dtype), _as_input(W, dtype)
    M, N = G.shape
    K = W.shape[0]
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    if rows.shape != cols.shape or (rows.size and (rows.min() < 0 or rows.max() >= M
                                                   or cols.min() < 0 or cols.max() >= K)):
        raise ValueError("sample positions out of range")
    out = np.empty(rows.shape, dtype=np.float64)
    _load().oracle_dx_at(_ptr(G), _ptr(W), _DTYPES[dtype], M, K, N,
                         _ptr(rows), _ptr(cols), rows.size, _ptr(out))
    return out


def dw_at(X, G, dtype: str, rows, cols) -> np.ndarray:
    """dW[rows[i], cols[i]] in float64 (rows index K, cols index N)."""
    X, G = _as_input(X, dtype), _as_input(G, dtype)
    M, K = X.shape
    N = G.shape[1]
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    if rows.shape != cols.shape or (rows.size and (rows.min() < 0 or rows.max() >= K
                                                   or cols.min() < 0 or cols.max() >= N)):
        raise ValueError("sample positions out of range")
    out = np.empty(rows.shape, dtype=np.float64)
    _load().oracle_dw_at(_ptr(X), _ptr(G), _DTYPES[dtype], M, K, N,
                         _ptr(rows), _ptr(cols), rows.size, _ptr(out))
    return out


def adamw(W, g, m, v, gtype: str, lr, b1, b2, eps, wd, step, inv_scale):
    """One AdamW step; returns new (W, m, v) float32 arrays, inputs untouched."""
    W = np.array(W, dtype=np.float32, copy=True)
    m = np.array(m, dtype=np.float32, copy=True)
    v = np.array(v, dtype=np.float32, copy=True)
    g = _as_input(g, gtype)
    if not (W.shape == m.shape == v.shape and g.size == W.size):
        raise ValueError("W, g, m, v must have the same number of elements")
    rc = _load().oracle_adamw(_ptr(W), _ptr(g), _DTYPES[gtype], _ptr(m), _ptr(v), W.size,
                              lr, b1, b2, eps, wd, int(step), inv_scale)
    if rc != 0:
        raise ValueError("adamw: invalid hyper-parameters (step=%r, b1=%r, b2=%r)"
                         % (step, b1, b2))
    return W, m, v


def round16(a, dtype: str) -> np.ndarray:
    """fp32 values rounded to nearest even as 'bf16' or 'f16' bit patterns (uint16)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    _load().oracle_round16(_ptr(a), a.size, _DTYPES[dtype], _ptr(out))
    return out


def adamw_ex(W, g, m, v, gtype: str, lr, b1, b2, eps, wd, step, inv_scale,
             clip=None, skip=False, w16=None):
    """The AdamW step with the loop's optional parts: clip (float or None) multiplies
    the unscaled gradient, skip leaves everything unchanged, w16 ('bf16' / 'f16' /
    None) also returns the updated W rounded to 16 bits.  Returns (W, m, v, W16)."""
    W = np.array(W, dtype=np.float32, copy=True)
    m = np.array(m, dtype=np.float32, copy=True)
    v = np.array(v, dtype=np.float32, copy=True)
    g = _as_input(g, gtype)
    if not (W.shape == m.shape == v.shape and g.size == W.size):
        raise ValueError("W, g, m, v must have the same number of elements")
    W16 = np.zeros(W.shape, dtype=np.uint16) if w16 is not None else None
    c = np.array([clip], dtype=np.float32) if clip is not None else None
    rc = _load().oracle_adamw_ex(_ptr(W), _ptr(g), _DTYPES[gtype], _ptr(m), _ptr(v), W.size,
                                 lr, b1, b2, eps, wd, int(step), inv_scale,
                                 _ptr(c) if c is not None else None, int(bool(skip)),
                                 _ptr(W16) if W16 is not None else None,
                                 _DTYPES[w16] if w16 is not None else 0)
    if rc != 0:
        raise ValueError("adamw_ex: invalid arguments (step=%r, b1=%r, b2=%r, w16=%r)"
                         % (step, b1, b2, w16))
    return W, m, v, W16


def grad_norm(g, gtype: str, inv_scale=1.0, max_norm=0.0):
    """(norm, clip factor, found_inf) of the unscaled gradient float(g)*inv_scale."""
    g = _as_input(g, gtype)
    out = np.zeros(2, dtype=np.float32)
    bad = np.zeros(1, dtype=np.int32)
    _load().oracle_grad_norm(_ptr(g), _DTYPES[gtype], g.size, inv_scale, max_norm, _ptr(out),
                             _ptr(bad))
    return float(out[0]), float(out[1]), bool(bad[0])
