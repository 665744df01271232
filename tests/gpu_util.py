"""Helpers for the GPU parity tests: guarded output buffers, metrics, sampling.

Outputs are carved out of a larger buffer whose guard bands hold a canary
pattern and whose interior is poisoned with NaN, so a kernel that writes out
of bounds, or leaves an entry unwritten, fails the comparison.
"""
import numpy as np
import torch

GUARD = 64  # elements on each side (128 or 256 bytes: keeps 16-byte alignment)

#: tolerances (written here, used by every parity test)
DX_RELF = 4e-3        # bf16 dX vs fp64: relative Frobenius error
DW_RELF = 1e-5        # fp32 dW vs fp64
F32_OUT_RELF = 1e-5   # fp32 dX (fp32 operands) vs fp64
ADAMW_ABS = 2e-6      # |gpu - oracle| <= ADAMW_ABS * max(1, |oracle|) for W, m, v
NORM_ULP = 1          # gradient norm: fp32 ulps from the oracle (same exact squares, fp64 sums)
CLIP_ULP = 2          # clip factor: fp32 ulps from the oracle's
DB_RELF = 1e-5        # fp32 bias gradient vs fp64: relative Frobenius error
DB_ABS = 1e-5         # ... and per column |error| <= DB_ABS * sum_m |dY[m,n]|
SM_RELF = {"f32": 1e-5, "bf16": 4e-3}   # softmax backward vs fp64: relative Frobenius error


def softmax_bound(P, dY, cols, dtype):
    """Per-element error bound of an fp32 softmax backward: the row's dot product summed
    in chains of at most cols/64 + 64 terms (relative error of the dot at most
    2^-24 * that length * sum_j |P_j dY_j|), one rounding each for the difference and the
    product, and the final rounding to bf16 (half an ulp, 2^-9) when dtype is bf16."""
    u = 2.0 ** -24
    P = np.abs(np.asarray(P, np.float64))
    g = np.abs(np.asarray(dY, np.float64))
    S = np.sum(P * g, axis=1, keepdims=True)
    gamma = u * (cols / 64.0 + 64.0)
    ref_mag = P * (g + S)
    b = P * (gamma * S + 2 * u * (g + S)) + 2 * u * ref_mag
    if dtype == "bf16":
        b = b + 2.0 ** -8 * ref_mag
    return b


class Guarded:
    """A (rows, cols) tensor inside a canary-banded 1-D buffer."""

    def __init__(self, rows, cols, dtype, device="cuda", offset=0):
        n = rows * cols
        self.dtype = dtype
        self.n = n
        self.lo = GUARD + offset
        self.buf = torch.empty(n + 2 * GUARD + offset, dtype=dtype, device=device)
        self.buf.fill_(-12345.0 if dtype == torch.float32 else -123.0)
        self.canary = self.buf[0].item()
        self.t = self.buf[self.lo:self.lo + n].view(rows, cols)
        self.t.fill_(float("nan"))

    def check_guards(self):
        before = self.buf[:self.lo].cpu()
        after = self.buf[self.lo + self.n:].cpu()
        assert bool((before == self.canary).all()), "write before the output buffer"
        assert bool((after == self.canary).all()), "write past the output buffer"


def relf(a, ref):
    a = np.asarray(a, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = float(np.linalg.norm(ref))
    num = float(np.linalg.norm(a - ref))
    if den == 0.0:
        return num if num > 1e-30 else 0.0
    return num / den


def host_f64(t):
    return t.detach().to("cpu", torch.float64).numpy() if t.dtype != torch.bfloat16 \
        else t.detach().to("cpu").float().double().numpy()


def bits(t):
    """Raw host element view (float32, or 16-bit patterns as uint16) of any tensor."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.float32:
        return t.numpy()
    return t.view(torch.int16).numpy().view(np.uint16)


def ulp_distance_f32(a, b):
    """Elementwise distance in units in the last place between two float32 arrays."""
    ai = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    bi = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    ai = np.where(ai < 0, np.int64(-2 ** 31) - ai, ai)
    bi = np.where(bi < 0, np.int64(-2 ** 31) - bi, bi)
    return np.abs(ai - bi)


def adamw_ok(gpu, ref):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    same = (np.isnan(gpu) & np.isnan(ref)) | (gpu == ref)   # NaN vs NaN, inf vs inf
    with np.errstate(invalid="ignore"):
        err = np.where(same, 0.0, np.abs(gpu - ref))
    ok = same | (err <= ADAMW_ABS * np.maximum(1.0, np.abs(ref)))
    worst = float(np.nanmax(err / np.maximum(1.0, np.abs(ref)))) if err.size else 0.0
    return bool(ok.all()), worst


# ---- per-element error bounds of the GEMM outputs -------------------------------------
#
# A kernel adds the R products of an entry in fp32: 32 at a time inside one MFMA, then into
# the accumulator (and, split across blocks, partial sums added in a fixed order).  With
# exact bf16 products and unit roundoff u = 2^-24 each entry's error is at most
#     gamma(R) * S,   gamma(R) = u * (R / 32 + 64),   S = Σ |a·b|
# (R / 32 accumulator additions, up to 32 inside an MFMA, and the split partials).  A bf16
# output adds one rounding to nearest, at most 2^-8 of the value.

U32 = 2.0 ** -24
U_BF16 = 2.0 ** -8


def gamma(R, sequential=False):
    """Error factor for R products summed by an MFMA kernel, or one by one in fp32
    (sequential: the element-wise kernel's chain of R roundings)."""
    return U32 * (R if sequential else R / 32.0 + 64.0)


def abs_bits(b, dtype):
    """The stored elements with their sign cleared (|x| exactly)."""
    if dtype == "f32":
        return np.abs(b)
    return b & np.uint16(0x7FFF)


def assert_within_bound(got, ref, S, R, bf16_out, what, sequential=False):
    got = np.asarray(got, np.float64)
    bound = 1.01 * gamma(R, sequential) * S
    if bf16_out:
        bound = bound + U_BF16 * (np.abs(ref) + bound)
    bad = np.abs(got - ref) > bound
    assert not bad.any(), "%s: %d entries beyond the per-element bound, e.g. got %r ref %r bound %r" % (
        what, int(bad.sum()), got[bad][:3], ref[bad][:3], bound[bad][:3])
