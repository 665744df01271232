"""The C-ABI library loads, exports every symbol include/linbwd.h declares, and
rejects bad arguments on the host before anything is launched (CPU only: no
call here reaches the GPU).
"""
import ctypes
import os
import re
import subprocess

import pytest

import linear_layer_backward_bwd_amd as lb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "linbwd.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for want in ("lin_bwd", "adamw_step", "adamw_step_f16", "adamw_step_bf16", "adamw_step_ex",
                 "grad_norm", "lin_bwd_ex", "softmax_bwd",
                 "lin_bwd_ex_noalloc", "lb_set_stream", "lb_set_lin_bwd_path", "lb_last_error",
                 "lb_version", "lb_shutdown"):
        assert want in names


def test_library_exports_every_declared_symbol():
    lib = lb.library()
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", lb.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in declared_functions():
        assert name in exported, name


def test_version_and_empty_error():
    assert "gfx950" in lb.lb_version()
    lib = lb.library()
    assert lib.lb_set_stream(None) == 0
    assert lb.lb_last_error() == ""


def test_header_compiles_as_c():
    src = '#include "linbwd.h"\nint main(void){return LB_OK + LB_BF16 - 1;}\n'
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                        "-x", "c", "-", "-o", "/dev/null", "-c"], input=src, text=True,
                       capture_output=True)
    assert r.returncode == 0, r.stderr


NULL = None


@pytest.mark.parametrize("args,code", [
    ((NULL, NULL, NULL, NULL, NULL, -1, 4, 4, 1), -1),         # negative M
    ((NULL, NULL, NULL, NULL, NULL, 4, -1, 4, 1), -1),         # negative K
    ((NULL, NULL, NULL, NULL, NULL, 4, 4, -5, 0), -1),         # negative N
    ((NULL, NULL, NULL, NULL, NULL, 4, 4, 4, 2), -2),          # unknown dtype
    ((NULL, NULL, NULL, NULL, NULL, 1 << 31, 4, 4, 1), -1),    # too large
    ((NULL, NULL, NULL, 16, NULL, 4, 4, 4, 1), -1),            # dX wanted, W/dY NULL
    ((NULL, NULL, NULL, NULL, 16, 4, 4, 4, 1), -1),            # dW wanted, X/dY NULL
])
def test_lin_bwd_rejects_on_host(args, code):
    lib = lb.library()
    assert lib.lin_bwd(*args) == code
    assert lb.lb_last_error() != ""


def test_lin_bwd_noop_cases_need_no_gpu():
    lib = lb.library()
    assert lib.lin_bwd(NULL, NULL, NULL, NULL, NULL, 8, 8, 8, 1) == 0      # nothing requested
    assert lib.lin_bwd(NULL, NULL, NULL, 16, 16, 8, 0, 8, 1) == 0          # K = 0: nothing to write
    assert lb.lb_last_error() == ""


@pytest.mark.parametrize("name", ["adamw_step", "adamw_step_f16", "adamw_step_bf16"])
@pytest.mark.parametrize("over,code", [
    (dict(n=-1), -1), (dict(step=0), -1), (dict(step=-3), -1), (dict(b1=1.0), -1),
    (dict(b2=1.0), -1), (dict(b1=-0.5), -1), (dict(b2=float("nan")), -1),
    (dict(n=10), -1),                                              # NULL buffers with n > 0
    (dict(n=0), 0),                                                # empty: no-op
])
def test_adamw_rejects_on_host(name, over, code):
    a = dict(n=0, lr=1e-3, b1=0.9, b2=0.999, eps=1e-8, wd=0.01, step=1, inv_scale=1.0)
    a.update(over)
    fn = getattr(lb.library(), name)
    rc = fn(NULL, NULL, NULL, NULL, a["n"], a["lr"], a["b1"], a["b2"], a["eps"], a["wd"],
            a["step"], a["inv_scale"])
    assert rc == code
    assert (lb.lb_last_error() != "") == (code != 0)


def test_python_binding_rejects_cpu_tensors():
    import torch
    x = torch.zeros(4, 4, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        lb.lin_bwd(x, x, x, torch.zeros_like(x), torch.zeros(4, 4))
    with pytest.raises(TypeError):
        lb.lin_bwd(x, x.float(), x)
    with pytest.raises(ValueError):
        lb.lin_bwd(x, torch.zeros(5, 4, dtype=torch.bfloat16), x)
    w = torch.zeros(8)
    with pytest.raises(TypeError):
        lb.adamw_step(w, w.to(torch.int32), w, w, 1e-3, 0.9, 0.99, 1e-8, 0.0, 1)


@pytest.mark.parametrize("over,code", [
    (dict(gd=3), -2), (dict(gd=-1), -2),                           # unknown gradient dtype
    (dict(w16=16, wd16=0), -2), (dict(w16=16, wd16=7), -2),        # 16-bit copy must be bf16/f16
    (dict(step=0), -1), (dict(b2=1.0), -1), (dict(n=-2), -1),
    (dict(n=10), -1),                                              # NULL buffers with n > 0
    (dict(n=0), 0), (dict(n=0, w16=16, wd16=1), 0),                # empty: no-op
])
def test_adamw_ex_rejects_on_host(over, code):
    a = dict(n=0, gd=1, step=1, b1=0.9, b2=0.999, w16=NULL, wd16=0)
    a.update(over)
    rc = lb.library().adamw_step_ex(NULL, NULL, a["gd"], NULL, NULL, a["n"], 1e-3, a["b1"], a["b2"],
                                    1e-8, 0.01, a["step"], 1.0, NULL, NULL, a["w16"], a["wd16"])
    assert rc == code
    assert (lb.lb_last_error() != "") == (code != 0)


def test_adamw_ex_binding_checks_types():
    import torch
    w = torch.zeros(8)
    with pytest.raises(TypeError):
        lb.adamw_step_ex(w, w.to(torch.int32), w, w, 1e-3, 0.9, 0.99, 1e-8, 0.0, 1)
    with pytest.raises(TypeError):
        lb.adamw_step_ex(w, w, w, w, 1e-3, 0.9, 0.99, 1e-8, 0.0, 1, w16=torch.zeros(8))
    with pytest.raises(TypeError):
        lb.adamw_step_ex(w, w, w, w, 1e-3, 0.9, 0.99, 1e-8, 0.0, 1, clip=torch.zeros(2))
    with pytest.raises(TypeError):
        lb.adamw_step_ex(w, w, w, w, 1e-3, 0.9, 0.99, 1e-8, 0.0, 1, skip=torch.zeros(1))


FAKE = ctypes.c_void_p(256)   # never dereferenced: every case below is rejected on the host


@pytest.mark.parametrize("gd,n,grad,out,code", [
    (3, 0, NULL, FAKE, -2), (-1, 4, FAKE, FAKE, -2),   # unknown gradient dtype
    (1, -1, FAKE, FAKE, -1),                           # negative size
    (0, 0, NULL, NULL, -1), (2, 8, FAKE, NULL, -1),    # NULL d_out
    (1, 8, NULL, FAKE, -1),                            # NULL grad with n > 0
])
def test_grad_norm_rejects_on_host(gd, n, grad, out, code):
    rc = lb.library().grad_norm(grad, gd, n, 1.0, 1.0, out, NULL)
    assert rc == code
    assert lb.lb_last_error() != ""


def test_grad_norm_binding_checks_types():
    import torch
    g = torch.zeros(8)
    with pytest.raises(TypeError):
        lb.grad_norm(g.to(torch.int32))
    with pytest.raises(TypeError):
        lb.grad_norm(g, out=torch.zeros(3))
    with pytest.raises(TypeError):
        lb.grad_norm(g, out=torch.zeros(2, dtype=torch.float64))
    with pytest.raises(TypeError):
        lb.grad_norm(g, found_inf=torch.zeros(1))


@pytest.mark.parametrize("args,code", [
    (dict(dtype=2), -2), (dict(dtype=-1), -2),                  # unknown dtype
    (dict(M=-1), -1), (dict(N=-5), -1), (dict(K=1 << 31), -1),  # bad sizes
    (dict(db=FAKE), -1),                                        # db requested, dY NULL
    (dict(db=FAKE, N=0), 0),                                    # N = 0: nothing to write
    (dict(), 0),                                                # nothing requested
])
@pytest.mark.parametrize("entry", ["lin_bwd_ex", "lin_bwd_ex_noalloc"])
def test_lin_bwd_ex_rejects_on_host(args, code, entry):
    a = dict(M=8, K=8, N=8, dtype=1, db=NULL)
    a.update(args)
    rc = getattr(lb.library(), entry)(NULL, NULL, NULL, NULL, NULL, a["db"], a["M"], a["K"], a["N"],
                                      a["dtype"])
    assert rc == code
    assert (lb.lb_last_error() != "") == (code != 0)
    if code and entry == "lin_bwd_ex_noalloc":
        assert lb.lb_last_error().startswith(entry)


def test_lin_bwd_ex_binding_checks():
    import torch
    g = torch.zeros(4, 6, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        lb.lin_bwd_ex(None, None, g, db=torch.zeros(5))
    with pytest.raises(ValueError):
        lb.lin_bwd_ex(None, None, g, db=torch.zeros(6, dtype=torch.float64))
    with pytest.raises(ValueError):
        lb.lin_bwd_ex(torch.zeros(4, 3, dtype=torch.bfloat16), None, g, db=torch.zeros(6))
    with pytest.raises(TypeError):
        lb.lin_bwd_ex(None, None, g.to(torch.float16), db=torch.zeros(6))


@pytest.mark.parametrize("args,code", [
    (dict(dtype=2), -2), (dict(dtype=9), -2),
    (dict(rows=-1), -1), (dict(cols=-3), -1), (dict(rows=1 << 40), -1),
    (dict(), -1),                                   # NULL buffers with rows, cols > 0
    (dict(rows=0), 0), (dict(cols=0), 0),           # nothing to write
])
def test_softmax_bwd_rejects_on_host(args, code):
    a = dict(rows=4, cols=8, dtype=1)
    a.update(args)
    rc = lb.library().softmax_bwd(NULL, NULL, NULL, a["rows"], a["cols"], a["dtype"])
    assert rc == code
    assert (lb.lb_last_error() != "") == (code != 0)


def test_softmax_bwd_binding_checks():
    import torch
    p = torch.zeros(4, 8)
    with pytest.raises(TypeError):
        lb.softmax_bwd(p, p.to(torch.bfloat16))
    with pytest.raises(TypeError):
        lb.softmax_bwd(p.double(), p.double())
    with pytest.raises(ValueError):
        lb.softmax_bwd(p, torch.zeros(4, 9))
    with pytest.raises(ValueError):
        lb.softmax_bwd(p, p, torch.zeros(4, 8, dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        lb.softmax_bwd(p.t(), p.t())


@pytest.mark.parametrize("path", [-1, 5, 99])
def test_set_lin_bwd_path_rejects_unknown_values(path):
    try:
        assert lb.library().lb_set_lin_bwd_path(path) == -1
        assert "LB_PATH" in lb.lb_last_error()
    finally:
        lb.library().lb_set_lin_bwd_path(lb.LB_PATH_AUTO)


# (path, M, K, N, dtype, X, W, dY, dX, dW): forced paths that cannot run the call are refused
# on the host, before any workspace or launch (the fake pointers are never dereferenced)
P16, P32, P48, P64 = (ctypes.c_void_p(v) for v in (4096, 8192, 12288, 16384))
ODD = ctypes.c_void_p(4098)


@pytest.mark.parametrize("path,M,K,N,dtype,ptrs", [
    (lb.LB_PATH_TILE, 64, 64, 64, 0, (P16, P32, P48, P64, NULL)),        # fp32 operands
    (lb.LB_PATH_SMALL_M, 64, 64, 64, 0, (P16, P32, P48, NULL, P64)),
    (lb.LB_PATH_TILE, 64, 64, 1 << 22, 1, (P16, P32, P48, P64, NULL)),   # dX: 256 rows of 2N bytes >= 2 GiB
    (lb.LB_PATH_TILE, 64, 1 << 25, 64, 1, (P16, P32, P48, NULL, P64)),   # dW: a 32-row slab of X >= 2 GiB
    (lb.LB_PATH_SMALL_M, 1025, 64, 64, 1, (P16, P32, P48, P64, NULL)),   # dX: M <= 1024 only
    (lb.LB_PATH_SMALL_M, 257, 64, 64, 1, (P16, P32, P48, NULL, P64)),    # dW: M <= 256 only
    (lb.LB_PATH_FUSED_SMALL_M, 65, 64, 64, 1, (P16, P32, P48, P64, P16)),  # M <= 64 only
    (lb.LB_PATH_FUSED_SMALL_M, 32, 64, 64, 1, (P16, P32, P48, P64, NULL)),  # needs dX and dW
    (lb.LB_PATH_FUSED_SMALL_M, 32, 64, 1 << 25, 1, (P16, P32, P48, P64, P16)),  # 64 N < 2^31
])
def test_forced_path_refused_on_host(path, M, K, N, dtype, ptrs):
    lib = lb.library()
    X, W, dY, dX, dW = ptrs
    assert lib.lb_set_lin_bwd_path(path) == 0
    try:
        assert lib.lin_bwd(X, W, dY, dX, dW, M, K, N, dtype) == -1
        assert "forced kernel path" in lb.lb_last_error()
        assert lib.lin_bwd_ex(X, W, dY, dX, dW, NULL, M, K, N, dtype) == -1
    finally:
        assert lib.lb_set_lin_bwd_path(lb.LB_PATH_AUTO) == 0


# bf16 calls with K or N not a multiple of 8, or with unaligned pointers, run on padded
# copies that the call allocates on its stream: a forced MFMA path takes them (here the
# call passes the host checks and then fails for want of a GPU), while the no-allocation
# entry point, which cannot copy, refuses them
STAGED = [
    (lb.LB_PATH_TILE, 64, 60, 64, (P16, P32, P48, P64, NULL)),        # K not a multiple of 8
    (lb.LB_PATH_TILE, 64, 64, 68, (P16, P32, P48, NULL, P64)),        # N not a multiple of 8
    (lb.LB_PATH_TILE, 64, 64, 64, (P16, P32, ODD, P64, NULL)),        # misaligned dY
    (lb.LB_PATH_SMALL_M, 32, 4100, 4096, (P16, P32, P48, P64, P16)),  # ragged K, both products
    (lb.LB_PATH_FUSED_SMALL_M, 32, 4096, 4100, (P16, P32, P48, P64, P16)),
]


@pytest.mark.parametrize("path,M,K,N,ptrs", STAGED)
def test_forced_path_takes_ragged_calls_through_padded_copies(path, M, K, N, ptrs):
    lib = lb.library()
    X, W, dY, dX, dW = ptrs
    assert lib.lb_set_lin_bwd_path(path) == 0
    try:
        lib.lin_bwd(X, W, dY, dX, dW, M, K, N, 1)
        assert "forced kernel path" not in lb.lb_last_error()
        assert lib.lin_bwd_ex_noalloc(X, W, dY, dX, dW, NULL, M, K, N, 1) == -1
        assert "forced kernel path" in lb.lb_last_error()
    finally:
        assert lib.lb_set_lin_bwd_path(lb.LB_PATH_AUTO) == 0


def test_staged_call_still_refuses_what_the_padded_call_cannot_run():
    """K = 2^25 - 4 pads to 2^25: a 32-row slab of the padded X is 2 GiB."""
    lib = lb.library()
    assert lib.lb_set_lin_bwd_path(lb.LB_PATH_TILE) == 0
    try:
        assert lib.lin_bwd(P16, P32, P48, NULL, P64, 64, (1 << 25) - 4, 64, 1) == -1
        assert "forced kernel path" in lb.lb_last_error()
    finally:
        assert lib.lb_set_lin_bwd_path(lb.LB_PATH_AUTO) == 0


def test_forced_path_is_per_thread_and_restored():
    import threading
    lib = lb.library()
    seen = []
    with lb.lin_bwd_path(lb.LB_PATH_TILE):
        # another thread still runs with automatic selection: fp32 is accepted there
        # (K = 0 writes nothing, so no GPU is touched)
        t = threading.Thread(target=lambda: seen.append(
            lib.lin_bwd(P16, P32, P48, P64, NULL, 64, 0, 64, 0)))
        t.start()
        t.join()
        assert lib.lin_bwd(P16, P32, P48, P64, NULL, 64, 64, 64, 0) == -1
    assert seen == [0]


def test_c_consumer_compiles_against_the_header():
    """The native consumer (tests/native/c_abi_consumer.c) builds with gcc against
    include/linbwd.h and the HIP runtime header alone."""
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-fsyntax-only", "-D__HIP_PLATFORM_AMD__",
                        "-I", os.path.join(rocm, "include"), "-I", os.path.join(ROOT, "include"),
                        os.path.join(ROOT, "tests", "native", "c_abi_consumer.c")],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
