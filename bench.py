"""Benchmark: Linear backward (dX + dW, bf16 MFMA) + fused unscale/AdamW on one MI355X.

Default workload (one "step" = the whole hot path once): one Transformer
block's four projections at M = 16384 tokens (QKV 4096->12288, out 4096->4096,
up 4096->16384, down 16384->4096), lin_bwd on each, then one fused
unscale + AdamW pass (bf16 gradients x1024, step 100) over all 201,326,592
parameters.  Inputs are seeded synthetic draws made on the GPU before the
timed region.

Prints one JSON line.  ``value`` is the whole step's throughput: the step's
GEMM FLOPs (4·M·K·N per projection) divided by the wall time of the whole
step including the AdamW pass.  The per-kernel figures come from HIP events
recorded on the launch stream around every launch of the timed steps.

Roofline model ("GPU 如何训练模型：从算子到 Kernel", section "Roofline：先判断
“算不动”还是“搬不动”"): an op of F FLOP moving Q bytes cannot finish before
max(F/P, Q/B); the ideal GEMM traffic is Q = b·(MK + KN + MN).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "lin-bwd TFLOP/s (dX+dW, bf16) + fused AdamW GB/s; % of roofline, 1 GPU"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0        # MI355X HBM3E
ADAMW_BYTES_16BIT_GRAD = 26   # read g(2) W m v (12), write W m v (12)
ADAMW_BYTES_F32_GRAD = 28
ADAMW_EX_BYTES_16BIT_GRAD_BF16_COPY = 28   # the 26 above + the bf16 copy of W (2)
GRAD_NORM_BYTES_16BIT = 2                  # reads the gradient once


def ideal_intensity(M, K, N, bytes_per_elem=2):
    """FLOP per byte of one GEMM of 2MKN FLOP moving b·(MK+KN+MN) bytes."""
    return 2.0 * M * K * N / (bytes_per_elem * (M * K + K * N + M * N))


def lin_bwd_flops(M, K, N):
    """dX = G·Wᵀ and dW = Xᵀ·G: 2MKN each."""
    return 4.0 * M * K * N


def lin_bwd_min_bytes(M, K, N):
    """Algorithmic HBM bytes of lin_bwd: read X, W, G (bf16), write dX (bf16) and dW (fp32)."""
    return 2 * (M * K + K * N + M * N) + 2 * M * K + 4 * K * N


def lin_bwd_tiled_bytes(M, K, N, tile=256, cus_per_xcd=32, xcds=8):
    """HBM bytes the MFMA tile kernel must move for lin_bwd at large M, as a model.

    Operands: the kernel's tile order (tiles of each XCD gathered into one range and
    rastered in groups of 4 tile rows, 2 for a job with rotated starts or a dW job of
    at most 16 x 16 tiles over a reduction of at most 2048; dX tiles start
    their reduction at one of four rotated slabs when rows are a multiple of 32 KiB
    apart) with each XCD running 32
    tiles at a time.  A panel (the 256 operand rows or columns that one tile row or
    column reads over the whole reduction) is counted once per group of 32 concurrent
    tiles that reads it from the same starting slab, i.e. the tiles share lines in the
    XCD's L2 while they run and keep nothing for the next group.  Outputs: dX bf16 and
    dW fp32 written once.  Measured FETCH_SIZE + WRITE_SIZE of the kernel is this
    figure within 0.3-0.8% on the block's QKV, out and down projections.
    """
    def job(I, J, R, rot, offset, dw=False):
        ti_n, tj_n = -(-I // tile), -(-J // tile)
        n = ti_n * tj_n
        nslab = -(-R // 32)
        total = 0
        for x in range(xcds):
            seq = [t for t in range(n) if (offset + t) % xcds == x]
            for c in range(0, len(seq), cus_per_xcd):
                a, b = set(), set()
                for t in seq[c:c + cus_per_xcd]:
                    u = (t & 7) * (n >> 3) + (t >> 3) if n % 8 == 0 else t
                    gi = 2 if rot or (dw and ti_n <= 16 and tj_n <= 16 and R <= 2048) else 4
                    per_group = gi * tj_n
                    first_i = (u // per_group) * gi
                    rows = min(ti_n - first_i, gi)
                    in_group = u % per_group
                    ti, tj = first_i + in_group % rows, in_group // rows
                    start = (rot * ((tj >> 1) & 3)) % nslab if nslab else 0
                    a.add((ti, start))
                    b.add((tj, start))
                total += sum(min(tile, I - tile * ti) for ti, _ in a) * R * 2
                total += sum(min(tile, J - tile * tj) for tj, _ in b) * R * 2
        return total

    rot = 32 if (2 * N) % 32768 == 0 else 0
    n_dx = -(-M // tile) * -(-K // tile)
    n_dw = -(-K // tile) * -(-N // tile)
    dx_first = N >= M      # the job with the longer reduction takes the first blocks
    dx = job(M, K, N, rot, 0 if dx_first else n_dw)
    dw = job(K, N, M, 0, n_dx if dx_first else 0, dw=True)
    return dx + dw + 2 * M * K + 4 * K * N


def _sync():
    import torch
    torch.cuda.synchronize()


def lin_bwd_roofs(M, K, N):
    """Roofline limits of lin_bwd at one shape (TFLOP/s): min(P, I·B) with the pages' ideal
    traffic b(MK+KN+MN) per product ("GPU 如何训练模型：从算子到 Kernel", section "Roofline"),
    and with the traffic the call must move at least (bf16 X, W, dY, dX and the fp32 dW)."""
    flops = lin_bwd_flops(M, K, N)
    i_pages = ideal_intensity(M, K, N)
    i_actual = flops / lin_bwd_min_bytes(M, K, N)
    return {"pages": min(PEAK_BF16_TFLOPS, i_pages * PEAK_HBM_GBPS / 1000.0),
            "fp32_dw_aware": min(PEAK_BF16_TFLOPS, i_actual * PEAK_HBM_GBPS / 1000.0),
            "intensity_pages": i_pages, "intensity_actual": i_actual}


def cpu_description():
    """CPU model, logical CPUs this process may use, and physical cores among them."""
    model, phys = None, set()
    cur = {}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if not line.strip():
                    if "processor" in cur:
                        phys.add((cur.get("processor"), cur.get("physical id"), cur.get("core id")))
                    cur = {}
                    continue
                k, _, v = line.partition(":")
                cur[k.strip()] = v.strip()
                if k.strip() == "model name" and model is None:
                    model = v.strip()
    except OSError:
        pass
    allowed = os.sched_getaffinity(0) if hasattr(os, "sched_getaffinity") else set(range(os.cpu_count() or 1))
    cores = {(p, c) for proc, p, c in phys if proc is not None and int(proc) in allowed and c is not None}
    return {"cpu_model": model, "logical_cpus_allowed": len(allowed),
            "physical_cores_allowed": len(cores) or None}


CALIB_PATH = os.path.join(ROOT, "linear_layer_backward_bwd_amd", "libcalib.so")


def calibrate(reps=10):
    """What this part sustains: a plain copy, a read-only pass, the AdamW traffic mix without
    arithmetic (26 B per element, as the AdamW kernel issues it) and back-to-back bf16 MFMAs
    on random values; HIP events around `reps` launches of each, best of two sizes where the
    launch shape matters."""
    import ctypes

    import torch
    if not os.path.exists(CALIB_PATH):
        raise RuntimeError("%s is not built (python -m linear_layer_backward_bwd_amd.build)" % CALIB_PATH)
    lib = ctypes.CDLL(CALIB_PATH)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.calib_copy.argtypes = [vp, vp, i64, vp]
    lib.calib_read.argtypes = [vp, i64, vp, vp]
    lib.calib_stream.argtypes = [vp, vp, vp, vp, i64, vp]
    lib.calib_mfma.argtypes = [i32, i32, vp, vp]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def timed(fn):
        for _ in range(3):
            assert fn() == 0
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            assert fn() == 0
        b.record()
        _sync()
        return a.elapsed_time(b) / reps * 1e-3

    out = {}
    nbytes = 1 << 30
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    word = torch.zeros(1, dtype=torch.int32, device="cuda")
    t = timed(lambda: lib.calib_copy(dst.data_ptr(), src.data_ptr(), nbytes, stream))
    out["copy_gbps"] = round(2 * nbytes / t / 1e9, 1)
    big = torch.ones(2 * nbytes // 4, dtype=torch.float32, device="cuda")
    t = timed(lambda: lib.calib_read(big.data_ptr(), 2 * nbytes, word.data_ptr(), stream))
    out["read_gbps"] = round(2 * nbytes / t / 1e9, 1)
    del src, dst, big
    n = 1 << 28
    W = torch.zeros(n, dtype=torch.float32, device="cuda")
    m = torch.zeros_like(W)
    v = torch.zeros_like(W)
    g = torch.zeros(n, dtype=torch.int16, device="cuda")
    t = timed(lambda: lib.calib_stream(W.data_ptr(), g.data_ptr(), m.data_ptr(), v.data_ptr(), n, stream))
    out["adamw_mix_stream_gbps"] = round(ADAMW_BYTES_16BIT_GRAD * n / t / 1e9, 1)
    del W, m, v, g
    torch.cuda.empty_cache()
    best = 0.0
    iters = 4000
    for blocks in (256, 512, 1024):
        t = timed(lambda: lib.calib_mfma(blocks, iters, word.data_ptr(), stream))
        best = max(best, blocks * 4 * iters * 16 * 16384.0 / t / 1e12)
    out["mfma_bf16_tflops"] = round(best, 1)
    out["note"] = ("copy: one 16-byte vector per thread; read: 2 GiB once; adamw_mix_stream: reads "
                   "a 16-bit g and fp32 W, m, v and writes W, m, v per element (26 B) with no "
                   "arithmetic, 2^28 elements; mfma: v_mfma_f32_16x16x32_bf16 back to back on "
                   "random bf16 values in registers, best of 1, 2 and 4 waves per SIMD")
    return out


KERNEL_SOURCES = {"k_lin_bwd_mfma": "linear_layer_backward_bwd_amd/csrc/lin_bwd.hip",
                  "k_lin_bwd_mfma_split": "linear_layer_backward_bwd_amd/csrc/lin_bwd.hip",
                  "k_dw_smallm": "linear_layer_backward_bwd_amd/csrc/lin_bwd.hip",
                  "k_smallm_pair": "linear_layer_backward_bwd_amd/csrc/lin_bwd.hip",
                  "k_adamw": "linear_layer_backward_bwd_amd/csrc/adamw.hip",
                  "k_norm_partial": "linear_layer_backward_bwd_amd/csrc/grad_norm.hip",
                  "k_bias_partial": "linear_layer_backward_bwd_amd/csrc/bias_grad.hip",
                  "k_softmax_bwd_wave": "linear_layer_backward_bwd_amd/csrc/softmax_bwd.hip"}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def code_hash(text):
    """sha256 (16 hex digits) of C/HIP source with its comments and whitespace removed, so
    that a record stays valid across edits of comments only (the kernels' source has no
    string literal holding a comment marker)."""
    import hashlib
    import re
    code = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    code = re.sub(r"//[^\n]*", " ", code)
    code = re.sub(r"\s+", " ", code).strip()
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def source_hash(kernel):
    with open(os.path.join(ROOT, KERNEL_SOURCES[kernel]), encoding="utf-8") as f:
        return code_hash(f.read())


def recorded_traffic(kernel, workload):
    """HBM bytes per launch measured by rocprofv3 FETCH_SIZE / WRITE_SIZE (scaled by a copy
    kernel of known size), as recorded in profiles/traffic.json -- or None when there is no
    record for this kernel and workload or the kernel's code (comments aside) changed since
    it was taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)[kernel][workload]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("source_sha256_16") != source_hash(kernel):
        return None
    return rec["hbm_bytes_per_launch"]


def copy_calibration(steps):
    """A plain copy of exactly 1 GiB, `steps` times: the reference for scaling counter bytes."""
    import torch
    src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(steps):
        dst.copy_(src)
    _sync()
    return {"copy_bytes_per_launch": 1 << 30, "launches": steps}


class Timer:
    """HIP events on the current (launch) stream around each launch of the timed steps."""

    def __init__(self, names):
        self.names = names
        self.ms = {n: 0.0 for n in names}
        self.count = {n: 0 for n in names}
        self.samples = {n: [] for n in names}
        self.pending = []

    def run(self, name, fn):
        import torch
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        self.pending.append((name, a, b))

    def collect(self):
        _sync()
        for name, a, b in self.pending:
            t = a.elapsed_time(b)
            self.ms[name] += t
            self.count[name] += 1
            self.samples[name].append(t)
        self.pending = []


def bench_block(steps, warmup, seed):
    import torch

    import linear_layer_backward_bwd_amd as lb
    import synth
    dev = "cuda"
    cases, opt = synth.block_case(seed=seed, device=dev)
    outs = []
    for c in cases:
        c.W_master = None
        outs.append((torch.empty(c.M, c.K, dtype=torch.bfloat16, device=dev),
                     torch.empty(c.K, c.N, dtype=torch.float32, device=dev)))
    torch.cuda.empty_cache()
    names = [c.name for c in cases] + ["adamw"]
    flops = {c.name: lin_bwd_flops(c.M, c.K, c.N) for c in cases}
    n_params = opt.W.numel()

    def step(timer=None):
        for c, (dX, dW) in zip(cases, outs):
            f = lambda c=c, dX=dX, dW=dW: lb.lin_bwd(c.X, c.W, c.G, dX, dW)
            timer.run(c.name, f) if timer else f()
        f = lambda: lb.adamw_step(opt.W, opt.g, opt.m, opt.v, opt.lr, opt.b1, opt.b2, opt.eps,
                                  opt.wd, opt.steps[0], opt.inv_scale)
        timer.run("adamw", f) if timer else f()

    for _ in range(warmup):
        step()
    # exactly `steps` steps, bracketed by device synchronisation; HIP events on the
    # launch stream around every launch give the per-kernel durations
    timer = Timer(names)
    _sync()
    t0 = time.perf_counter()
    for _ in range(steps):
        step(timer)
    _sync()
    wall = time.perf_counter() - t0
    timer.collect()

    gemm_flops = sum(flops.values())
    gemm_ms = sum(timer.ms[c.name] for c in cases) / steps
    adamw_ms = timer.ms["adamw"] / steps
    adamw_gbps = ADAMW_BYTES_16BIT_GRAD * n_params / (adamw_ms * 1e-3) / 1e9
    per_proj = []
    for c in cases:
        ms = timer.ms[c.name] / steps
        t = sorted(timer.samples[c.name])
        per_proj.append({"name": c.name, "M": c.M, "K": c.K, "N": c.N, "ms": round(ms, 4),
                         "ms_median": round(t[len(t) // 2], 4), "ms_min": round(t[0], 4),
                         "tflops": round(flops[c.name] / (ms * 1e-3) / 1e12, 1)})
    ms_step = wall / steps * 1e3
    result = {
        "value": gemm_flops / (wall / steps) / 1e12,
        "ms_per_step": ms_step,
        "config": {"workload": "block_bwd_update_M16384_D4096",
                   "tokens": synth.BLOCK_TOKENS,
                   "projections": [[c.name, c.K, c.N] for c in cases],
                   "params": n_params, "adamw_grad": "bf16 x1024", "adamw_step": opt.steps[0]},
        "parts": {
            "lin_bwd": {"ms": round(gemm_ms, 4), "tflops": round(gemm_flops / (gemm_ms * 1e-3) / 1e12, 1),
                        "frac_of_peak": round(gemm_flops / (gemm_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                        "per_projection": per_proj},
            "adamw": {"ms": round(adamw_ms, 4), "gbps": round(adamw_gbps, 1),
                      "frac_of_peak": round(adamw_gbps / PEAK_HBM_GBPS, 4),
                      "traffic": recorded_traffic("k_adamw", "block_bwd_update_M16384_D4096"),
                      "gparams_per_s": round(n_params / (adamw_ms * 1e-3) / 1e9, 2),
                      "bytes_per_param": ADAMW_BYTES_16BIT_GRAD},
        },
        "roofline": {"bound": "mfma", "kernel": "k_lin_bwd_mfma",
                     "achieved": round(gemm_flops / (gemm_ms * 1e-3) / 1e12, 1),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(gemm_flops / (gemm_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                     "traffic": recorded_traffic("k_lin_bwd_mfma", "block_bwd_update_M16384_D4096"),
                     "algorithmic_bytes_per_launch": sum(lin_bwd_min_bytes(c.M, c.K, c.N)
                                                         for c in cases) / len(cases),
                     "tiled_model_bytes_per_launch": sum(lin_bwd_tiled_bytes(c.M, c.K, c.N)
                                                         for c in cases) / len(cases),
                     "per_launch_flops": gemm_flops / len(cases),
                     "launch_ms": round(gemm_ms / len(cases), 4)},
    }
    return result, (cases, opt)


_SLEEP_CYCLES_PER_MS = None


def hold_queue(ms):
    """Enqueue a sleep kernel of about `ms` milliseconds on the current stream, so that
    the launches queued behind it while it runs start back to back on the GPU: HIP events
    around them then bracket GPU time, not the host's per-call launch latency (a few tens
    of microseconds through Python and ctypes, longer than an M = 32 call on the GPU)."""
    import torch
    global _SLEEP_CYCLES_PER_MS
    if _SLEEP_CYCLES_PER_MS is None:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        torch.cuda._sleep(1 << 20)
        b.record()
        _sync()
        _SLEEP_CYCLES_PER_MS = (1 << 20) / max(a.elapsed_time(b), 1e-3)
    torch.cuda._sleep(int(ms * _SLEEP_CYCLES_PER_MS))


def plain_stream_floor(read_bytes, write_bytes, calls=40, rotate_bytes=768 << 20):
    """GPU time per launch of the calibration read kernel over `read_bytes` and of the
    write kernel over `write_bytes` (16-byte vectors, one per thread), cold: each call on
    the next of enough buffers to exceed the 256 MB last-level cache, queued behind a
    sleep kernel, an event pair around each call; medians.  Their sum is what two plain
    streaming kernels need to move the bytes of a memory-bound call on this part."""
    import ctypes

    import torch
    if not os.path.exists(CALIB_PATH):
        raise RuntimeError("%s is not built (python -m linear_layer_backward_bwd_amd.build)" % CALIB_PATH)
    lib = ctypes.CDLL(CALIB_PATH)
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    lib.calib_read.argtypes = [vp, i64, vp, vp]
    lib.calib_write.argtypes = [vp, i64, ctypes.c_uint32, vp]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    word = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = {}
    for name, nbytes in (("read", read_bytes), ("write", write_bytes)):
        nbytes = (nbytes + 15) // 16 * 16
        nb = max(4, -(-rotate_bytes // nbytes))
        bufs = [torch.ones(nbytes // 4, dtype=torch.float32, device="cuda") for _ in range(nb)]
        if name == "read":
            fn = lambda i: lib.calib_read(bufs[i % nb].data_ptr(), nbytes, word.data_ptr(), stream)
        else:
            fn = lambda i: lib.calib_write(bufs[i % nb].data_ptr(), nbytes, 0x3f800000, stream)
        for i in range(4):
            assert fn(i) == 0
        _sync()
        hold_queue(calls * 0.05 + 2.0)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * calls)]
        for i in range(calls):
            ev[2 * i].record()
            assert fn(i) == 0
            ev[2 * i + 1].record()
        _sync()
        t = sorted(ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(calls))
        out[name + "_ms"] = round(t[len(t) // 2], 5)
        del bufs
        torch.cuda.empty_cache()
    out["sum_ms"] = round(out["read_ms"] + out["write_ms"], 5)
    return out


def bench_linear(M, K, N, steps, warmup, seed, rotate_bytes=768 << 20):
    """lin_bwd alone at one shape; rotates over buffer sets larger than the 256 MB MALL.
    The timed calls are queued behind a sleep kernel (hold_queue), so that the events
    around them measure the GPU's time, not the host's launch latency."""
    import torch

    import linear_layer_backward_bwd_amd as lb
    import synth
    dev = "cuda"
    one = 2 * (M * K + K * N + M * N) + 2 * M * K + 4 * K * N
    nsets = max(1, min(16, -(-rotate_bytes // one)))     # one set when it exceeds the MALL anyway
    sets = []
    for i in range(nsets):
        c = synth.linear_case(M, K, N, "bf16", seed=seed + i, device=dev)
        sets.append((c, torch.empty(M, K, dtype=torch.bfloat16, device=dev),
                     torch.empty(K, N, dtype=torch.float32, device=dev)))
    for i in range(warmup):
        c, dX, dW = sets[i % nsets]
        lb.lin_bwd(c.X, c.W, c.G, dX, dW)
    # back to back: one event pair around `steps` calls queued behind a sleep kernel
    timer = Timer(["batch"])
    _sync()
    hold_queue(steps * 0.1 + 2.0)

    def calls():
        for i in range(steps):
            c, dX, dW = sets[i % nsets]
            lb.lin_bwd(c.X, c.W, c.G, dX, dW)
    timer.run("batch", calls)
    timer.collect()
    ms_b2b = timer.ms["batch"] / steps
    # the same calls with an event pair around each: the per-call figure
    per = Timer(["lin_bwd"])
    _sync()
    hold_queue(steps * 0.1 + 2.0)
    for i in range(steps):
        c, dX, dW = sets[i % nsets]
        per.run("lin_bwd", lambda: lb.lin_bwd(c.X, c.W, c.G, dX, dW))
    per.collect()
    ms = per.ms["lin_bwd"] / steps
    cold = sorted(per.samples["lin_bwd"])
    # warm: the same calls on one buffer set, whose inputs the last-level cache then holds
    warm_median = None
    if nsets > 1:
        warm = Timer(["lin_bwd"])
        c0, dX0, dW0 = sets[0]
        lb.lin_bwd(c0.X, c0.W, c0.G, dX0, dW0)
        _sync()
        hold_queue(steps * 0.1 + 2.0)
        for i in range(steps):
            warm.run("lin_bwd", lambda: lb.lin_bwd(c0.X, c0.W, c0.G, dX0, dW0))
        warm.collect()
        ws = sorted(warm.samples["lin_bwd"])
        warm_median = ws[len(ws) // 2]
    fl = lin_bwd_flops(M, K, N)
    tf = fl / (ms * 1e-3) / 1e12
    q = lin_bwd_min_bytes(M, K, N)
    roofs = lin_bwd_roofs(M, K, N)
    floor = None
    if roofs["pages"] < PEAK_BF16_TFLOPS:   # memory-bound: what plain streaming kernels need
        floor = plain_stream_floor(2 * (M * K + K * N + M * N), 2 * M * K + 4 * K * N)
        floor["floor_over_ms"] = round(floor["sum_ms"] / ms, 4)
        floor["what"] = ("the calibration read kernel over the bytes the call reads (bf16 X, W, dY) "
                         "plus the write kernel over the bytes it writes (bf16 dX, fp32 dW), cold, "
                         "an event pair around each launch, medians")
    pair = M <= 64 and N <= 8192 and K * N <= (1 << 25 if N <= 4096 else 5 << 22)
    kernel = ("k_smallm_pair" if pair else "k_dw_smallm" if M <= 64
              else "k_lin_bwd_mfma_split" if 256 < M <= 1024 and N > 0 else "k_lin_bwd_mfma")
    return {"M": M, "K": K, "N": N, "ms": round(ms, 5), "tflops": round(tf, 1),
            "frac_of_mfma_peak": round(tf / PEAK_BF16_TFLOPS, 4),
            "bound": "hbm" if roofs["pages"] < PEAK_BF16_TFLOPS else "mfma",
            "roof_pages_tflops": round(roofs["pages"], 1),
            "frac_of_roof_pages": round(tf / roofs["pages"], 4),
            "roof_fp32_dw_aware_tflops": round(roofs["fp32_dw_aware"], 1),
            "frac_of_roof_fp32_dw_aware": round(tf / roofs["fp32_dw_aware"], 4),
            "gbps_alg": round(q / (ms * 1e-3) / 1e9, 1),
            "frac_of_hbm_peak_alg": round(q / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
            "bytes_alg": q,
            "intensity_pages": round(roofs["intensity_pages"], 2),
            "intensity_actual": round(roofs["intensity_actual"], 2),
            "ms_median": round(cold[len(cold) // 2], 5), "ms_min": round(cold[0], 5),
            "warm_ms_median": None if warm_median is None else round(warm_median, 5),
            "ms_back_to_back": round(ms_b2b, 5),
            "rotating_sets": nsets,
            "timing": "GPU time per call, cold (inputs rotate over buffer sets larger than the "
                      "last-level cache): calls queued behind a sleep kernel, an event pair around "
                      "each (ms = mean, ms_median, ms_min); the same calls with one event pair "
                      "around them all (ms_back_to_back); warm_ms_median: the same per-call "
                      "timing on one buffer set",
            "traffic": recorded_traffic(kernel, "lin_bwd_M%d_K%d_N%d" % (M, K, N)),
            **({"plain_stream_floor": floor} if floor else {})}


def bench_adamw(n, steps, warmup, seed):
    import torch

    import linear_layer_backward_bwd_amd as lb
    import synth
    case = synth.adamw_2p28(seed=seed, n=n, device="cuda")
    for i in range(warmup):
        lb.adamw_step(case.W, case.g, case.m, case.v, case.lr, case.b1, case.b2, case.eps, case.wd,
                      1 + i % 10, case.inv_scale)
    timer = Timer(["adamw"])
    for i in range(steps):
        timer.run("adamw", lambda: lb.adamw_step(case.W, case.g, case.m, case.v, case.lr, case.b1,
                                                 case.b2, case.eps, case.wd, 1 + i % 10, case.inv_scale))
    timer.collect()
    ms = timer.ms["adamw"] / steps
    t = sorted(timer.samples["adamw"])
    gbps = ADAMW_BYTES_16BIT_GRAD * n / (ms * 1e-3) / 1e9
    return {"n": n, "grad": "f16", "ms": round(ms, 4), "ms_median": round(t[len(t) // 2], 4),
            "ms_min": round(t[0], 4), "steps": steps, "warmup": warmup, "gbps": round(gbps, 1),
            "frac_of_hbm_peak": round(gbps / PEAK_HBM_GBPS, 4),
            "gparams_per_s": round(n / (ms * 1e-3) / 1e9, 2),
            "traffic": recorded_traffic("k_adamw", "adamw_2p28_f16")}


def bench_clipped_step(n, steps, warmup, seed):
    """grad_norm then adamw_step_ex (clip factor and skip flag from the norm, bf16 copy of W)."""
    import torch

    import linear_layer_backward_bwd_amd as lb
    import synth
    case = synth.adamw_2p28(seed=seed, n=n, device="cuda")
    w16 = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    out = torch.empty(2, dtype=torch.float32, device="cuda")
    found = torch.empty(1, dtype=torch.int32, device="cuda")
    norm = lambda: lb.grad_norm(case.g, case.inv_scale, 1.0, out=out, found_inf=found)
    upd = lambda t: lb.adamw_step_ex(case.W, case.g, case.m, case.v, case.lr, case.b1, case.b2,
                                     case.eps, case.wd, t, case.inv_scale, clip=out[1:2],
                                     skip=found, w16=w16)
    for i in range(warmup):
        norm()
        upd(1 + i % 10)
    # each kernel back to back (its own rate), then the pair as one step; the
    # norm's launches are shorter than the binding's host time, so they are
    # timed as one batch between two events (the queue never drains)
    timer = Timer(["norm", "adamw_ex", "step"])
    timer.run("norm", lambda: [norm() for _ in range(steps)])
    for i in range(steps):
        timer.run("adamw_ex", lambda: upd(1 + i % 10))
    for i in range(steps):
        timer.run("step", lambda: (norm(), upd(1 + i % 10)))
    timer.collect()
    norm_ms = timer.ms["norm"] / steps
    upd_ms = timer.ms["adamw_ex"] / steps
    step_ms = timer.ms["step"] / steps
    norm_gbps = GRAD_NORM_BYTES_16BIT * n / (norm_ms * 1e-3) / 1e9
    upd_gbps = ADAMW_EX_BYTES_16BIT_GRAD_BF16_COPY * n / (upd_ms * 1e-3) / 1e9
    return {"n": n, "grad": "f16", "copy": "bf16",
            "grad_norm": {"ms": round(norm_ms, 4), "gbps": round(norm_gbps, 1),
                          "frac_of_hbm_peak": round(norm_gbps / PEAK_HBM_GBPS, 4),
                          "bytes_per_param": GRAD_NORM_BYTES_16BIT,
                          "traffic": recorded_traffic("k_norm_partial", "grad_norm_2p28_f16")},
            "adamw_step_ex": {"ms": round(upd_ms, 4), "gbps": round(upd_gbps, 1),
                              "frac_of_hbm_peak": round(upd_gbps / PEAK_HBM_GBPS, 4),
                              "bytes_per_param": ADAMW_EX_BYTES_16BIT_GRAD_BF16_COPY,
                              "traffic": recorded_traffic("k_adamw", "adamw_ex_2p28_f16_bf16_copy")},
            "step_ms": round(step_ms, 4),
            "gparams_per_s": round(n / (step_ms * 1e-3) / 1e9, 2)}


def bench_bias(steps, warmup, seed):
    """db = column sums of dY for the block's four projections (lin_bwd_ex with db only)."""
    import torch

    import linear_layer_backward_bwd_amd as lb
    import synth
    gens = [synth._gen(seed + 1 + i, "cuda") for i in range(len(synth.BLOCK_PROJECTIONS))]
    Gs = [synth.to_storage(synth.normal((synth.BLOCK_TOKENS, n), 1e-4, g), "bf16")
          for g, (_, _, n) in zip(gens, synth.BLOCK_PROJECTIONS)]
    dbs = [torch.empty(G.shape[1], device="cuda") for G in Gs]
    run = lambda: [lb.lin_bwd_ex(None, None, G, db=db) for G, db in zip(Gs, dbs)]
    for _ in range(warmup):
        run()
    timer = Timer(["bias"])
    timer.run("bias", lambda: [run() for _ in range(steps)])
    timer.collect()
    ms = timer.ms["bias"] / steps
    nbytes = sum(G.numel() * 2 + G.shape[1] * 4 for G in Gs)
    gbps = nbytes / (ms * 1e-3) / 1e9
    return {"workload": "block dY, M=16384, N=12288/4096/16384/4096, bf16", "ms": round(ms, 4),
            "gbps": round(gbps, 1), "frac_of_hbm_peak": round(gbps / PEAK_HBM_GBPS, 4),
            "bytes": nbytes,
            "traffic_per_launch": recorded_traffic("k_bias_partial", "bias_grad_block_M16384")}


def bench_softmax(steps, warmup, seed):
    """softmax_bwd over the attention probabilities of one block (bf16, rows of 2048)."""
    import torch

    import linear_layer_backward_bwd_amd as lb
    import synth
    rows, cols = synth.SOFTMAX_ROWS, synth.SOFTMAX_COLS
    P, dY = synth.softmax_case(rows, cols, "bf16", seed=seed, device="cuda")
    dX = torch.empty_like(P)
    for _ in range(warmup):
        lb.softmax_bwd(P, dY, dX)
    timer = Timer(["softmax"])
    for _ in range(steps):
        timer.run("softmax", lambda: lb.softmax_bwd(P, dY, dX))
    timer.collect()
    ms = timer.ms["softmax"] / steps
    nbytes = 3 * 2 * rows * cols
    gbps = nbytes / (ms * 1e-3) / 1e9
    return {"workload": "softmax_bwd rows=%d (8x32x2048) cols=%d bf16" % (rows, cols),
            "ms": round(ms, 4), "gbps": round(gbps, 1),
            "frac_of_hbm_peak": round(gbps / PEAK_HBM_GBPS, 4), "bytes_per_elem": 6,
            "traffic": recorded_traffic("k_softmax_bwd_wave", "softmax_bwd_524288x2048_bf16")}


def cpu_baseline(cases, opt, target_s=12.0):
    """The CPU oracle on a bounded sample of the block workload, extrapolated to one step."""
    import numpy as np

    import oracle
    import synth
    rng = np.random.default_rng(0)
    host = [(c, synth.bits(c.X.cpu()), synth.bits(c.W.cpu()), synth.bits(c.G.cpu())) for c in cases]

    # calibrate on a small sample, then size the sample to about target_s of work
    def gemm_sample(count):
        macs = 0
        t0 = time.perf_counter()
        for c, Xb, Wb, Gb in host:
            r, k = rng.integers(0, c.M, count), rng.integers(0, c.K, count)
            oracle.dx_at(Gb, Wb, "bf16", r, k)
            k2, n2 = rng.integers(0, c.K, count), rng.integers(0, c.N, count)
            oracle.dw_at(Xb, Gb, "bf16", k2, n2)
            macs += count * c.N + count * c.M
        return macs, time.perf_counter() - t0
    macs, dt = gemm_sample(256)
    count = int(256 * max(1.0, (0.8 * target_s) / max(dt, 1e-3)))
    macs, dt = gemm_sample(count)
    gemm_rate = 2.0 * macs / dt                        # FLOP/s on the host
    n = 1 << 23
    sl = slice(0, n)
    W = opt.W[sl].cpu().numpy()
    m = opt.m[sl].cpu().numpy()
    v = opt.v[sl].cpu().numpy()
    g = synth.bits(opt.g[sl].cpu())
    t0 = time.perf_counter()
    oracle.adamw(W, g, m, v, "bf16", opt.lr, opt.b1, opt.b2, opt.eps, opt.wd, opt.steps[0],
                 opt.inv_scale)
    adamw_rate = n / (time.perf_counter() - t0)        # params/s on the host
    step_flops = sum(lin_bwd_flops(c.M, c.K, c.N) for c in cases)
    step_s = step_flops / gemm_rate + opt.W.numel() / adamw_rate
    return {"value": step_flops / step_s / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle", **cpu_description(),
            "sample": ("%d dX + %d dW entries per projection (fp64 dot products on the bf16 inputs) "
                       "and one AdamW step over 2^23 params (scalar fp32), extrapolated to the "
                       "whole step; host GEMM %.2f GFLOP/s, host AdamW %.1f Mparam/s"
                       % (count, count, gemm_rate / 1e9, adamw_rate / 1e6)),
            "oracle_step_s_extrapolated": round(step_s, 1)}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the M=32 / M=2048 / 2^28-param AdamW figures")
    ap.add_argument("--only", choices=["block", "m32", "m1024", "m2048", "adamw", "clipped", "bias", "softmax",
                                       "copycal", "calib"],
                    default=None,
                    help="time one workload only (for profiling); copycal = 1 GiB copies for "
                         "scaling HBM byte counters; calib = the calibration kernels")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print("bench.py: one GPU only; --gpus %d is not supported "
              "(the multi-GPU sharding is a design note, not code)" % args.gpus, file=sys.stderr)
        return 2
    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    import linear_layer_backward_bwd_amd as lb
    lb.library()

    if args.only in ("m32", "m1024", "m2048"):
        M = int(args.only[1:])
        print(json.dumps(bench_linear(M, 4096, 4096, args.steps, args.warmup, args.seed)), flush=True)
        return 0
    if args.only == "adamw":
        print(json.dumps(bench_adamw(1 << 28, args.steps, args.warmup, args.seed)), flush=True)
        return 0
    if args.only == "clipped":
        print(json.dumps(bench_clipped_step(1 << 28, args.steps, args.warmup, args.seed)), flush=True)
        return 0
    if args.only == "bias":
        print(json.dumps(bench_bias(args.steps, args.warmup, args.seed)), flush=True)
        return 0
    if args.only == "softmax":
        print(json.dumps(bench_softmax(args.steps, args.warmup, args.seed)), flush=True)
        return 0
    if args.only == "copycal":
        print(json.dumps(copy_calibration(args.steps)), flush=True)
        return 0
    if args.only == "calib":
        print(json.dumps(calibrate(args.steps)), flush=True)
        return 0

    print("bench: block workload, warmup %d, steps %d" % (args.warmup, args.steps),
          file=sys.stderr, flush=True)
    res, (cases, opt) = bench_block(args.steps, args.warmup, args.seed)
    out = {"metric": METRIC, "value": round(res["value"], 2), "unit": "TFLOP/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(res["ms_per_step"], 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic (seeded normal draws on the GPU; random-init weights)",
           "config": res["config"], "parts": res["parts"], "roofline": res["roofline"]}
    if args.only == "block":
        print(json.dumps(out), flush=True)
        return 0
    if not args.no_cpu_baseline:
        print("bench: cpu baseline (oracle on a bounded sample)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(cases, opt)
    del cases, opt
    torch.cuda.empty_cache()
    if not args.no_extra:
        print("bench: calibration kernels", file=sys.stderr, flush=True)
        cal = calibrate()
        out["calibration"] = cal
        lin = out["parts"]["lin_bwd"]
        lin["frac_of_measured_mfma_peak"] = round(lin["tflops"] / cal["mfma_bf16_tflops"], 4)
        out["roofline"]["measured_peak"] = cal["mfma_bf16_tflops"]
        out["roofline"]["frac_of_measured_peak"] = round(out["roofline"]["achieved"] / cal["mfma_bf16_tflops"], 4)
        ad = out["parts"]["adamw"]
        ad["frac_of_measured_copy"] = round(ad["gbps"] / cal["copy_gbps"], 4)
        ad["frac_of_measured_adamw_mix_stream"] = round(ad["gbps"] / cal["adamw_mix_stream_gbps"], 4)
        print("bench: extra shapes", file=sys.stderr, flush=True)
        out["also"] = {
            "lin_bwd_M32_K4096_N4096": bench_linear(32, 4096, 4096, 50, 5, args.seed),
            "lin_bwd_M2048_K4096_N4096": bench_linear(2048, 4096, 4096, 50, 5, args.seed),
            # the block's shard on 16 data-parallel ranks: dX with its reduction split over tiles
            "lin_bwd_M1024_K4096_N4096": bench_linear(1024, 4096, 4096, 50, 5, args.seed),
            # the down projection at 65536 tokens: X and dX of 2 GiB each
            "lin_bwd_M65536_K16384_N4096": bench_linear(65536, 16384, 4096, 3, 1, args.seed,
                                                        rotate_bytes=0),
            # N not a multiple of 8: the call runs on zero-padded copies of dY, W and dW
            "lin_bwd_M16384_K4096_N4100": bench_linear(16384, 4096, 4100, 5, 2, args.seed,
                                                       rotate_bytes=0),
            # 10 warm-up steps: the first ten or so launches of a long series of these passes
            # run up to 10% slower than the ones after them, arithmetic or not
            "adamw_2p28_f16": bench_adamw(1 << 28, 20, 10, args.seed),
            "grad_norm_adamw_ex_2p28_f16": bench_clipped_step(1 << 28, 20, 10, args.seed),
            "bias_grad_block": bench_bias(20, 3, args.seed),
            "softmax_bwd_attention": bench_softmax(10, 2, args.seed),
        }
        for key in ("lin_bwd_M32_K4096_N4096", "lin_bwd_M1024_K4096_N4096", "lin_bwd_M2048_K4096_N4096"):
            out["also"][key]["frac_of_measured_mfma_peak"] = round(
                out["also"][key]["tflops"] / cal["mfma_bf16_tflops"], 4)
        m32 = out["also"]["lin_bwd_M32_K4096_N4096"]
        m32["frac_of_measured_copy_alg"] = round(m32["gbps_alg"] / cal["copy_gbps"], 4)
        a2 = out["also"]["adamw_2p28_f16"]
        a2["frac_of_measured_copy"] = round(a2["gbps"] / cal["copy_gbps"], 4)
        a2["frac_of_measured_adamw_mix_stream"] = round(a2["gbps"] / cal["adamw_mix_stream_gbps"], 4)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
