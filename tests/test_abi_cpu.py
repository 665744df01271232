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
                 "lb_set_stream", "lb_last_error", "lb_version", "lb_shutdown"):
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
def test_lin_bwd_ex_rejects_on_host(args, code):
    a = dict(M=8, K=8, N=8, dtype=1, db=NULL)
    a.update(args)
    rc = lb.library().lin_bwd_ex(NULL, NULL, NULL, NULL, NULL, a["db"], a["M"], a["K"], a["N"],
                                 a["dtype"])
    assert rc == code
    assert (lb.lb_last_error() != "") == (code != 0)


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
