"""Build liblinbwd.so (HIP, gfx950) in-tree with hipcc.

Usage: ``python -m linear_layer_backward_bwd_amd.build`` or ``build()``.
"""
from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB_PATH = os.path.join(HERE, "liblinbwd.so")
SOURCES = ["api.hip", "lin_bwd.hip", "adamw.hip", "grad_norm.hip", "bias_grad.hip", "softmax_bwd.hip"]
# measurement only (bench.py): copy / read / AdamW-mix stream and MFMA peak kernels
CALIB_PATH = os.path.join(HERE, "libcalib.so")
CALIB_SOURCES = ["calib.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # keep the compiler from forming packed fp32 (v_pk_*_f32) instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the HIP library cannot be built")
    return path


def build(extra_flags=(), out=LIB_PATH, verbose=False, sources=None) -> str:
    """Compile liblinbwd.so (or, with `sources`, another library from csrc/)."""
    srcs = [os.path.join(CSRC, s) for s in (sources or SOURCES)]
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), *extra_flags, *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build_calib(verbose=False) -> str:
    return build(out=CALIB_PATH, verbose=verbose, sources=CALIB_SOURCES)


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_calib(verbose=True))
