"""Linear-layer backward (dX = dY·Wᵀ, dW = Xᵀ·dY) and fused unscale + AdamW on MI355X.

A thin binding over the C ABI of ``liblinbwd.so`` (declared in
``include/linbwd.h``): it checks and marshals torch tensors into device
pointers and sizes, selects torch's current HIP stream, and raises
``RuntimeError`` with the library's message when a call fails.  Every step of
the computation runs in the library's HIP kernels; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["lin_bwd", "lin_bwd_ex", "adamw_step", "adamw_step_f16", "adamw_step_bf16",
           "adamw_step_ex", "grad_norm", "softmax_bwd", "lb_set_stream", "lb_set_lin_bwd_path",
           "lin_bwd_path", "lb_last_error", "lb_version", "lb_shutdown", "library", "LIB_PATH",
           "LB_F32", "LB_BF16", "LB_F16", "LB_PATH_AUTO", "LB_PATH_TILE", "LB_PATH_SMALL_M",
           "LB_PATH_GENERAL", "LB_PATH_FUSED_SMALL_M"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblinbwd.so")
LB_F32, LB_BF16, LB_F16 = 0, 1, 2
LB_OK, LB_EINVAL, LB_EDTYPE, LB_EHIP = 0, -1, -2, -4
LB_PATH_AUTO, LB_PATH_TILE, LB_PATH_SMALL_M, LB_PATH_GENERAL, LB_PATH_FUSED_SMALL_M = 0, 1, 2, 3, 4

_lib = None


def library() -> ctypes.CDLL:
    """Load liblinbwd.so (built in-tree by ``python -m linear_layer_backward_bwd_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("%s is not built: run `python -m linear_layer_backward_bwd_amd.build` "
                           "(the HIP library is required; there is no fallback)" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
    lib.lin_bwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i32]
    lib.lin_bwd.restype = i32
    for name in ("lin_bwd_ex", "lin_bwd_ex_noalloc"):
        fn = getattr(lib, name)
        fn.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i32]
        fn.restype = i32
    lib.softmax_bwd.argtypes = [vp, vp, vp, i64, i64, i32]
    lib.softmax_bwd.restype = i32
    for name in ("adamw_step", "adamw_step_f16", "adamw_step_bf16"):
        fn = getattr(lib, name)
        fn.argtypes = [vp, vp, vp, vp, i64, f32, f32, f32, f32, f32, i32, f32]
        fn.restype = i32
    lib.adamw_step_ex.argtypes = [vp, vp, i32, vp, vp, i64, f32, f32, f32, f32, f32, i32, f32,
                                  vp, vp, vp, i32]
    lib.adamw_step_ex.restype = i32
    lib.grad_norm.argtypes = [vp, i32, i64, f32, f32, vp, vp]
    lib.grad_norm.restype = i32
    lib.lb_set_stream.argtypes = [vp]
    lib.lb_set_stream.restype = i32
    lib.lb_set_lin_bwd_path.argtypes = [i32]
    lib.lb_set_lin_bwd_path.restype = i32
    lib.lb_last_error.argtypes = []
    lib.lb_last_error.restype = ctypes.c_char_p
    lib.lb_version.argtypes = []
    lib.lb_version.restype = ctypes.c_char_p
    lib.lb_shutdown.argtypes = []
    lib.lb_shutdown.restype = i32
    _lib = lib
    return lib


def lb_last_error() -> str:
    return library().lb_last_error().decode()


def lb_version() -> str:
    return library().lb_version().decode()


def lb_shutdown() -> None:
    """Frees the library-owned per-device workspace; no call may be in flight."""
    _check(library().lb_shutdown(), "lb_shutdown")


def lb_set_stream(stream) -> None:
    """Select the HIP stream (a torch.cuda.Stream, a raw handle int, or None)."""
    handle = getattr(stream, "cuda_stream", stream)
    library().lb_set_stream(ctypes.c_void_p(handle or 0))


def lb_set_lin_bwd_path(path: int) -> None:
    """Force the kernels of this thread's later lin_bwd / lin_bwd_ex calls (LB_PATH_*)."""
    _check(library().lb_set_lin_bwd_path(int(path)), "lb_set_lin_bwd_path")


class lin_bwd_path:
    """Context manager: ``with lin_bwd_path(LB_PATH_TILE): ...`` forces a kernel path for
    the calls inside and restores automatic selection afterwards."""

    def __init__(self, path: int):
        self.path = path

    def __enter__(self):
        lb_set_lin_bwd_path(self.path)
        return self

    def __exit__(self, *exc):
        lb_set_lin_bwd_path(LB_PATH_AUTO)
        return False


def _check(rc: int, name: str) -> None:
    if rc != LB_OK:
        raise RuntimeError("%s failed (code %d): %s" % (name, rc, lb_last_error()))


def _ptr(t):
    return None if t is None else (t.data_ptr() or None)


def _device_of(tensors):
    import torch
    devs = {t.device for t in tensors if t is not None}
    if len(devs) != 1:
        raise ValueError("all tensors must be on one device, got %s" % devs)
    dev = devs.pop()
    if dev.type != "cuda":
        raise ValueError("tensors must be on the GPU (torch 'cuda' device), got %s" % dev)
    for t in tensors:
        if t is not None and not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    return dev


def _use_current_stream(dev) -> None:
    import torch
    library().lb_set_stream(ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream))


def lin_bwd(X, W, dY, dX=None, dW=None) -> None:
    """dX = dY·Wᵀ (into dX, dtype of the operands) and dW = Xᵀ·dY (into dW, float32).

    X [M,K], W [K,N], dY [M,N]: all bfloat16 or all float32, contiguous, on one GPU.
    Either output may be None to skip it; outputs are overwritten.
    """
    import torch
    ops = [t for t in (X, W, dY) if t is not None]
    if not ops:
        raise ValueError("lin_bwd needs operands")
    dtype = ops[0].dtype
    if dtype not in (torch.bfloat16, torch.float32) or any(t.dtype != dtype for t in ops):
        raise TypeError("X, W, dY must all be bfloat16 or all float32")
    if X is None or W is None or dY is None:
        raise ValueError("X, W and dY are required")
    if X.dim() != 2 or W.dim() != 2 or dY.dim() != 2:
        raise ValueError("X, W, dY must be 2-D (flatten batch and sequence into M)")
    M, K = X.shape
    N = W.shape[1]
    if W.shape[0] != K or tuple(dY.shape) != (M, N):
        raise ValueError("shape mismatch: X%s W%s dY%s" % (tuple(X.shape), tuple(W.shape),
                                                           tuple(dY.shape)))
    if dX is not None and (dX.dtype != dtype or tuple(dX.shape) != (M, K)):
        raise ValueError("dX must be %s of shape (%d, %d)" % (dtype, M, K))
    if dW is not None and (dW.dtype != torch.float32 or tuple(dW.shape) != (K, N)):
        raise ValueError("dW must be float32 of shape (%d, %d)" % (K, N))
    dev = _device_of([X, W, dY, dX, dW])
    _use_current_stream(dev)
    rc = library().lin_bwd(_ptr(X), _ptr(W), _ptr(dY), _ptr(dX), _ptr(dW), M, K, N,
                           LB_BF16 if dtype == torch.bfloat16 else LB_F32)
    _check(rc, "lin_bwd")


def lin_bwd_ex(X, W, dY, dX=None, dW=None, db=None, no_alloc=False) -> None:
    """lin_bwd plus the bias gradient db[n] = Σ_m dY[m,n] (into db, float32 [N]).

    X and W may be None when dX and dW are None (db only).  no_alloc=True calls
    lin_bwd_ex_noalloc: the same results, temporaries in the library's static array (no
    device allocation; calls that overlap on one device race).
    """
    import torch
    if dY is None or dY.dim() != 2:
        raise ValueError("dY must be a 2-D tensor")
    dtype = dY.dtype
    if dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("dY must be bfloat16 or float32")
    M, N = dY.shape
    if dX is not None or dW is not None or X is not None or W is not None:
        if X is None or W is None:
            raise ValueError("X and W are required with dX or dW")
        if X.dtype != dtype or W.dtype != dtype:
            raise TypeError("X, W, dY must all be bfloat16 or all float32")
        if X.dim() != 2 or W.dim() != 2 or X.shape[0] != M or W.shape[1] != N or W.shape[0] != X.shape[1]:
            raise ValueError("shape mismatch: X%s W%s dY%s" % (tuple(X.shape), tuple(W.shape),
                                                               tuple(dY.shape)))
        K = X.shape[1]
    else:
        K = 0
    if dX is not None and (dX.dtype != dtype or tuple(dX.shape) != (M, K)):
        raise ValueError("dX must be %s of shape (%d, %d)" % (dtype, M, K))
    if dW is not None and (dW.dtype != torch.float32 or tuple(dW.shape) != (K, N)):
        raise ValueError("dW must be float32 of shape (%d, %d)" % (K, N))
    if db is not None and (db.dtype != torch.float32 or db.numel() != N):
        raise ValueError("db must be float32 with %d elements" % N)
    dev = _device_of([X, W, dY, dX, dW, db])
    _use_current_stream(dev)
    name = "lin_bwd_ex_noalloc" if no_alloc else "lin_bwd_ex"
    rc = getattr(library(), name)(_ptr(X), _ptr(W), _ptr(dY), _ptr(dX), _ptr(dW), _ptr(db), M, K, N,
                                  LB_BF16 if dtype == torch.bfloat16 else LB_F32)
    _check(rc, name)


def _adamw(name, W, grad, m, v, lr, b1, b2, eps, wd, step, inv_scale):
    import torch
    for t, nm in ((W, "W"), (m, "m"), (v, "v")):
        if t.dtype != torch.float32:
            raise TypeError("%s must be float32" % nm)
    n = W.numel()
    if m.numel() != n or v.numel() != n or grad.numel() != n:
        raise ValueError("W, grad, m, v must have the same number of elements")
    dev = _device_of([W, grad, m, v])
    _use_current_stream(dev)
    rc = getattr(library(), name)(_ptr(W), _ptr(grad), _ptr(m), _ptr(v), n, lr, b1, b2, eps, wd,
                                  int(step), inv_scale)
    _check(rc, name)


def adamw_step(W, grad, m, v, lr, b1, b2, eps, wd, step, inv_scale=1.0) -> None:
    """One fused unscale + AdamW step in place on W, m, v (float32); grad is read only.

    The C entry point is chosen by grad's dtype: float32 -> adamw_step,
    float16 -> adamw_step_f16, bfloat16 -> adamw_step_bf16.
    """
    import torch
    name = {torch.float32: "adamw_step", torch.float16: "adamw_step_f16",
            torch.bfloat16: "adamw_step_bf16"}.get(grad.dtype)
    if name is None:
        raise TypeError("grad must be float32, float16 or bfloat16")
    _adamw(name, W, grad, m, v, lr, b1, b2, eps, wd, step, inv_scale)


def adamw_step_f16(W, grad, m, v, lr, b1, b2, eps, wd, step, inv_scale=1.0) -> None:
    import torch
    if grad.dtype != torch.float16:
        raise TypeError("grad must be float16")
    _adamw("adamw_step_f16", W, grad, m, v, lr, b1, b2, eps, wd, step, inv_scale)


def adamw_step_bf16(W, grad, m, v, lr, b1, b2, eps, wd, step, inv_scale=1.0) -> None:
    import torch
    if grad.dtype != torch.bfloat16:
        raise TypeError("grad must be bfloat16")
    _adamw("adamw_step_bf16", W, grad, m, v, lr, b1, b2, eps, wd, step, inv_scale)


def adamw_step_ex(W, grad, m, v, lr, b1, b2, eps, wd, step, inv_scale=1.0, clip=None, skip=None,
                  w16=None) -> None:
    """The AdamW step with the training loop's optional parts (C: adamw_step_ex).

    grad: float32, float16 or bfloat16.  clip: a one-element float32 GPU tensor whose
    value multiplies the unscaled gradient, or None.  skip: a one-element int32 GPU
    tensor; when nonzero the step writes nothing.  w16: a bfloat16 or float16 tensor
    receiving the updated W rounded to nearest even, or None.  The kernel reads clip and
    skip itself, so factors computed on the GPU need no synchronisation.
    """
    import torch
    gd = {torch.float32: LB_F32, torch.float16: LB_F16, torch.bfloat16: LB_BF16}.get(grad.dtype)
    if gd is None:
        raise TypeError("grad must be float32, float16 or bfloat16")
    for t, nm in ((W, "W"), (m, "m"), (v, "v")):
        if t.dtype != torch.float32:
            raise TypeError("%s must be float32" % nm)
    n = W.numel()
    if m.numel() != n or v.numel() != n or grad.numel() != n:
        raise ValueError("W, grad, m, v must have the same number of elements")
    if clip is not None and (clip.dtype != torch.float32 or clip.numel() != 1):
        raise TypeError("clip must be a one-element float32 tensor")
    if skip is not None and (skip.dtype != torch.int32 or skip.numel() != 1):
        raise TypeError("skip must be a one-element int32 tensor")
    wd16 = 0
    if w16 is not None:
        wd16 = {torch.bfloat16: LB_BF16, torch.float16: LB_F16}.get(w16.dtype)
        if wd16 is None:
            raise TypeError("w16 must be bfloat16 or float16")
        if w16.numel() != n:
            raise ValueError("w16 must have n elements")
    dev = _device_of([W, grad, m, v, clip, skip, w16])
    _use_current_stream(dev)
    rc = library().adamw_step_ex(_ptr(W), _ptr(grad), gd, _ptr(m), _ptr(v), n, lr, b1, b2, eps, wd,
                                 int(step), inv_scale, _ptr(clip), _ptr(skip), _ptr(w16), wd16)
    _check(rc, "adamw_step_ex")


def grad_norm(grad, inv_scale=1.0, max_norm=0.0, out=None, found_inf=None):
    """Norm of the unscaled gradient, clip factor and inf/NaN flag, on the GPU (C: grad_norm).

    Returns (out, found_inf): out a float32 tensor [norm, clip factor], found_inf an
    int32 tensor [flag]; both stay on the device (pass out[1:] as adamw_step_ex's clip and
    found_inf as its skip).  Tensors may be given to reuse them.
    """
    import torch
    gd = {torch.float32: LB_F32, torch.float16: LB_F16, torch.bfloat16: LB_BF16}.get(grad.dtype)
    if gd is None:
        raise TypeError("grad must be float32, float16 or bfloat16")
    if out is None:
        out = torch.empty(2, dtype=torch.float32, device=grad.device)
    if found_inf is None:
        found_inf = torch.empty(1, dtype=torch.int32, device=grad.device)
    if out.dtype != torch.float32 or out.numel() != 2:
        raise TypeError("out must be a two-element float32 tensor")
    if found_inf.dtype != torch.int32 or found_inf.numel() != 1:
        raise TypeError("found_inf must be a one-element int32 tensor")
    dev = _device_of([grad, out, found_inf])
    _use_current_stream(dev)
    rc = library().grad_norm(_ptr(grad), gd, grad.numel(), inv_scale, max_norm, _ptr(out),
                             _ptr(found_inf))
    _check(rc, "grad_norm")
    return out, found_inf


def softmax_bwd(P, dY, dX=None):
    """dX = P * (dY - rowsum(P * dY)) over the last dimension (C: softmax_bwd).

    P, dY: one shape, both bfloat16 or both float32, contiguous, on one GPU; rows are
    all leading dimensions flattened.  dX (same shape and dtype) may be given, also as
    P or dY itself (in place); returns dX.
    """
    import torch
    if P.dtype != dY.dtype or P.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("P and dY must both be bfloat16 or both float32")
    if P.shape != dY.shape or P.dim() < 1:
        raise ValueError("P and dY must have one shape")
    if dX is None:
        dX = torch.empty_like(P)
    if dX.dtype != P.dtype or dX.shape != P.shape:
        raise ValueError("dX must match P in shape and dtype")
    for t, nm in ((P, "P"), (dY, "dY"), (dX, "dX")):
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % nm)
    cols = P.shape[-1]
    rows = P.numel() // cols if cols else 0
    dev = _device_of([P, dY, dX])
    _use_current_stream(dev)
    rc = library().softmax_bwd(_ptr(P), _ptr(dY), _ptr(dX), rows, cols,
                               LB_BF16 if P.dtype == torch.bfloat16 else LB_F32)
    _check(rc, "softmax_bwd")
    return dX
