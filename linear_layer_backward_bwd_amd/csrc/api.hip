// C ABI of liblinbwd: argument validation, stream selection, error strings.
// The declarations and their contracts are in include/linbwd.h.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <map>
#include <mutex>
#include <string>
#include <utility>

#include "../../include/linbwd.h"
#include "kernels.h"

namespace {

thread_local hipStream_t tl_stream = nullptr;
thread_local int tl_path = lb::PATH_AUTO;
thread_local std::string tl_error;

int fail(int code, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    tl_error = buf;
    return code;
}

int hip_fail(const char *what, hipError_t e) {
    return fail(LB_EHIP, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
}

bool beta_ok(float b) { return b >= 0.0f && b < 1.0f; } // false for NaN

// Library-owned workspace, allocated on first use for each (device, stream)
// pair and kept until the process ends or lb_shutdown(): grad_norm's
// per-block partial sums and flags, lin_bwd_ex's per-split bias partials and
// the fp32 dX partials of lin_bwd's split dX (bf16, M <= 2048), in separate
// regions.
// Calls on one stream run in order, so they can share one workspace; calls on
// two streams of a device get two workspaces and may overlap.
struct Workspace {
    double *norm_partial = nullptr;
    int *norm_flag = nullptr;
    float *bias_partial = nullptr;
    float *dx_partial = nullptr;
};
std::mutex ws_mutex;
std::map<std::pair<int, hipStream_t>, Workspace> ws_by_stream;

constexpr size_t kNormBytes = lb::kNormMaxBlocks * (sizeof(double) + sizeof(int));
constexpr size_t kBiasBytes = lb::kBiasWorkspaceFloats * sizeof(float);
constexpr size_t kDxBytes = lb::kDxPartialFloats * sizeof(float);

hipError_t workspace(Workspace &out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    std::lock_guard<std::mutex> lock(ws_mutex);
    const auto key = std::make_pair(dev, tl_stream);
    auto it = ws_by_stream.find(key);
    if (it == ws_by_stream.end()) {
        void *p = nullptr;
        e = hipMalloc(&p, kNormBytes + kBiasBytes + kDxBytes);
        if (e != hipSuccess)
            return e;
        Workspace w;
        w.norm_partial = static_cast<double *>(p);
        w.norm_flag = reinterpret_cast<int *>(w.norm_partial + lb::kNormMaxBlocks);
        w.bias_partial = reinterpret_cast<float *>(static_cast<char *>(p) + kNormBytes);
        w.dx_partial = reinterpret_cast<float *>(static_cast<char *>(p) + kNormBytes + kBiasBytes);
        it = ws_by_stream.emplace(key, w).first;
    }
    out = it->second;
    return hipSuccess;
}

// ---- memory pool for the padded copies of ragged or unaligned calls --------
// One stream-ordered pool per device, created on first use, that keeps what
// it holds across synchronisations (release threshold: never).  The device's
// default pool gives its memory back at every synchronisation, and the next
// allocation then maps it again: a ragged call with a synchronisation after
// it took 335 us instead of 89 (M = 32) and 339 instead of 215 (M = 2048).
// lb_shutdown() destroys the pools.
std::mutex pool_mutex;
std::map<int, hipMemPool_t> pool_by_device;

// ---- static scratch for lin_bwd_ex_noalloc ----------------------------------
// The temporaries of lin_bwd_ex (small-M dX split partials, then the bias row
// partials) for callers that cannot allocate, in a file-scope device array of
// the same capacity as a stream's workspace, so that both entry points choose
// the same splits (the launchers fit them to the capacity; no size needs
// more) and produce the same bits.  Each device holds its own copy for the
// life of the process.  Its host-side name is not a device address: the
// address comes from hipGetSymbolAddress, once per device with that device
// current, and only that address is ever passed to a kernel.
constexpr int64_t kScratchFloats = lb::kDxPartialFloats + lb::kBiasWorkspaceFloats;
static __device__ __align__(256) float scratch[kScratchFloats];
std::mutex scratch_mutex;
std::map<int, float *> scratch_by_device;

hipError_t scratch_address(float **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    std::lock_guard<std::mutex> lock(scratch_mutex);
    auto it = scratch_by_device.find(dev);
    if (it == scratch_by_device.end()) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        it = scratch_by_device.emplace(dev, static_cast<float *>(p)).first;
    }
    *out = it->second;
    return hipSuccess;
}

// lin_bwd, lin_bwd_ex and lin_bwd_ex_noalloc: the temporaries go to the
// stream's workspace, or with `no_alloc` to the static scratch array.
int lin_bwd_impl(const char *name, const void *X, const void *W, const void *dY, void *dX, float *dW, float *db,
                 int64_t M, int64_t K, int64_t N, int dtype, bool no_alloc) {
    tl_error.clear();
    if (dtype != LB_F32 && dtype != LB_BF16)
        return fail(LB_EDTYPE, "%s: dtype %d is not LB_F32 (0) or LB_BF16 (1)", name, dtype);
    if (M < 0 || K < 0 || N < 0)
        return fail(LB_EINVAL, "%s: negative size M=%lld K=%lld N=%lld", name, (long long)M, (long long)K,
                    (long long)N);
    const int64_t lim = (int64_t)1 << 31;
    if (M >= lim || K >= lim || N >= lim)
        return fail(LB_EINVAL, "%s: sizes must be below 2^31 (M=%lld K=%lld N=%lld)", name, (long long)M,
                    (long long)K, (long long)N);
    // dX has M*K entries and sums over N; dW has K*N entries and sums over M;
    // db has N entries and sums over M.
    if (dX && M > 0 && K > 0 && N > 0 && (!dY || !W))
        return fail(LB_EINVAL, "%s: dX requested but dY or W is NULL", name);
    if (dW && K > 0 && N > 0 && M > 0 && (!X || !dY))
        return fail(LB_EINVAL, "%s: dW requested but X or dY is NULL", name);
    if (db && N > 0 && M > 0 && !dY)
        return fail(LB_EINVAL, "%s: db requested but dY is NULL", name);
    lb::LinBwdArgs a;
    a.X = X;
    a.W = W;
    a.dY = dY;
    a.dX = dX;
    a.dW = dW;
    a.M = M;
    a.K = K;
    a.N = N;
    a.bf16 = dtype == LB_BF16;
    a.path = tl_path;
    // ragged or unaligned bf16 calls run on padded copies allocated on the
    // stream, which the no-allocation entry point cannot do: there they take
    // the element-wise kernel
    a.may_stage = !no_alloc;
    if (const char *why = lb::lin_bwd_path_refusal(a))
        return fail(LB_EINVAL, "%s: the forced kernel path (%d) cannot run this call: %s", name, tl_path, why);
    float *dx_partial = nullptr, *bias_partial = nullptr;
    const bool dx_split = dX && dtype == LB_BF16 && M > 0 && M <= lb::kDxSplitMaxM && K > 0 && N > 0;
    if ((db && N > 0) || dx_split) {
        if (no_alloc) {
            float *p = nullptr;
            hipError_t e = scratch_address(&p);
            if (e != hipSuccess)
                return hip_fail("lin_bwd_ex_noalloc (address of the scratch array)", e);
            dx_partial = p;
            bias_partial = p + lb::kDxPartialFloats;
        } else {
            Workspace ws;
            hipError_t e = workspace(ws);
            if (e != hipSuccess)
                return hip_fail("lin_bwd_ex (workspace)", e);
            dx_partial = ws.dx_partial;
            bias_partial = ws.bias_partial;
        }
    }
    // the dX partials only where every entry point passes them (bf16,
    // 1 <= M <= kDxSplitMaxM), so that lin_bwd and lin_bwd_ex with or without
    // db choose the same splits and give the same bits
    a.dx_partial = dx_split ? dx_partial : nullptr;
    a.dx_partial_floats = a.dx_partial ? lb::kDxPartialFloats : 0;
    hipError_t e = lb::launch_lin_bwd(a, tl_stream);
    if (e != hipSuccess)
        return hip_fail(name, e);
    if (db) {
        lb::BiasArgs b;
        b.dY = dY;
        b.db = db;
        b.M = M;
        b.N = N;
        b.bf16 = dtype == LB_BF16;
        b.partial = bias_partial;
        e = lb::launch_bias_grad(b, tl_stream);
        if (e != hipSuccess)
            return hip_fail(name, e);
    }
    return LB_OK;
}


int adamw_impl(const char *name, lb::GradType gt, float *W, const void *g, float *m, float *v, int64_t n,
               float lr, float b1, float b2, float eps, float wd, int step, float inv_scale,
               const float *clip = nullptr, const int32_t *skip = nullptr, void *W16 = nullptr,
               lb::ShadowType shadow = lb::SHADOW_NONE) {
    tl_error.clear();
    if (n < 0)
        return fail(LB_EINVAL, "%s: n = %lld is negative", name, (long long)n);
    if (step < 1)
        return fail(LB_EINVAL, "%s: step = %d; steps are numbered from 1", name, step);
    if (!beta_ok(b1) || !beta_ok(b2))
        return fail(LB_EINVAL, "%s: b1 = %g, b2 = %g must lie in [0, 1)", name, (double)b1, (double)b2);
    if (n == 0)
        return LB_OK;
    if (!W || !g || !m || !v)
        return fail(LB_EINVAL, "%s: NULL buffer with n = %lld", name, (long long)n);
    if (W16 && (W16 == (void *)W || W16 == g || W16 == (void *)m || W16 == (void *)v))
        return fail(LB_EINVAL, "%s: the 16-bit copy must not alias W, grad, m or v", name);
    lb::AdamWArgs a;
    a.W = W;
    a.g = g;
    a.m = m;
    a.v = v;
    a.n = n;
    a.lr = lr;
    a.b1 = b1;
    a.b2 = b2;
    a.eps = eps;
    a.wd = wd;
    a.one_minus_b1 = 1.0f - b1;
    a.one_minus_b2 = 1.0f - b2;
    a.bc1 = (float)(1.0 - std::pow((double)b1, (double)step));
    a.bc2 = (float)(1.0 - std::pow((double)b2, (double)step));
    a.inv_scale = inv_scale;
    a.clip = clip;
    a.skip = skip;
    a.W16 = static_cast<uint16_t *>(W16);
    hipError_t e = lb::launch_adamw(a, gt, W16 ? shadow : lb::SHADOW_NONE, tl_stream);
    if (e != hipSuccess)
        return hip_fail(name, e);
    return LB_OK;
}

} // namespace

namespace lb {
hipError_t staging_pool(hipMemPool_t *out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    std::lock_guard<std::mutex> lock(pool_mutex);
    auto it = pool_by_device.find(dev);
    if (it == pool_by_device.end()) {
        hipMemPoolProps props = {};
        props.allocType = hipMemAllocationTypePinned;
        props.handleTypes = hipMemHandleTypeNone;
        props.location.type = hipMemLocationTypeDevice;
        props.location.id = dev;
        hipMemPool_t pool = nullptr;
        e = hipMemPoolCreate(&pool, &props);
        if (e != hipSuccess)
            return e;
        uint64_t keep = UINT64_MAX;
        e = hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &keep);
        if (e != hipSuccess) {
            (void)hipMemPoolDestroy(pool);
            return e;
        }
        it = pool_by_device.emplace(dev, pool).first;
    }
    *out = it->second;
    return hipSuccess;
}
} // namespace lb

extern "C" {

int lin_bwd_ex(const void *X, const void *W, const void *dY, void *dX, float *dW, float *db, int64_t M,
               int64_t K, int64_t N, int dtype) {
    return lin_bwd_impl(db ? "lin_bwd_ex" : "lin_bwd", X, W, dY, dX, dW, db, M, K, N, dtype, false);
}

int lin_bwd_ex_noalloc(const void *X, const void *W, const void *dY, void *dX, float *dW, float *db,
                       int64_t M, int64_t K, int64_t N, int dtype) {
    return lin_bwd_impl("lin_bwd_ex_noalloc", X, W, dY, dX, dW, db, M, K, N, dtype, true);
}

int lin_bwd(const void *X, const void *W, const void *dY, void *dX, float *dW, int64_t M, int64_t K,
            int64_t N, int dtype) {
    return lin_bwd_ex(X, W, dY, dX, dW, nullptr, M, K, N, dtype);
}

int adamw_step(float *W, const float *grad, float *m, float *v, int64_t n, float lr, float b1, float b2,
               float eps, float wd, int step, float inv_scale) {
    return adamw_impl("adamw_step", lb::GRAD_F32, W, grad, m, v, n, lr, b1, b2, eps, wd, step, inv_scale);
}

int adamw_step_f16(float *W, const uint16_t *grad, float *m, float *v, int64_t n, float lr, float b1,
                   float b2, float eps, float wd, int step, float inv_scale) {
    return adamw_impl("adamw_step_f16", lb::GRAD_F16, W, grad, m, v, n, lr, b1, b2, eps, wd, step,
                      inv_scale);
}

int adamw_step_bf16(float *W, const uint16_t *grad, float *m, float *v, int64_t n, float lr, float b1,
                    float b2, float eps, float wd, int step, float inv_scale) {
    return adamw_impl("adamw_step_bf16", lb::GRAD_BF16, W, grad, m, v, n, lr, b1, b2, eps, wd, step,
                      inv_scale);
}

int adamw_step_ex(float *W, const void *grad, int grad_dtype, float *m, float *v, int64_t n, float lr,
                  float b1, float b2, float eps, float wd, int step, float inv_scale, const float *d_clip,
                  const int32_t *d_skip, void *W16, int w16_dtype) {
    tl_error.clear();
    lb::GradType gt;
    switch (grad_dtype) {
    case LB_F32: gt = lb::GRAD_F32; break;
    case LB_F16: gt = lb::GRAD_F16; break;
    case LB_BF16: gt = lb::GRAD_BF16; break;
    default:
        return fail(LB_EDTYPE, "adamw_step_ex: grad_dtype %d is not LB_F32, LB_F16 or LB_BF16", grad_dtype);
    }
    lb::ShadowType sh = lb::SHADOW_NONE;
    if (W16) {
        if (w16_dtype == LB_BF16)
            sh = lb::SHADOW_BF16;
        else if (w16_dtype == LB_F16)
            sh = lb::SHADOW_F16;
        else
            return fail(LB_EDTYPE, "adamw_step_ex: w16_dtype %d is not LB_BF16 or LB_F16", w16_dtype);
    }
    return adamw_impl("adamw_step_ex", gt, W, grad, m, v, n, lr, b1, b2, eps, wd, step, inv_scale, d_clip,
                      d_skip, W16, sh);
}

int grad_norm(const void *grad, int grad_dtype, int64_t n, float inv_scale, float max_norm, float *d_out,
              int32_t *d_found_inf) {
    tl_error.clear();
    lb::GradType gt;
    switch (grad_dtype) {
    case LB_F32: gt = lb::GRAD_F32; break;
    case LB_F16: gt = lb::GRAD_F16; break;
    case LB_BF16: gt = lb::GRAD_BF16; break;
    default: return fail(LB_EDTYPE, "grad_norm: grad_dtype %d is not LB_F32, LB_F16 or LB_BF16", grad_dtype);
    }
    if (n < 0)
        return fail(LB_EINVAL, "grad_norm: n = %lld is negative", (long long)n);
    if (!d_out)
        return fail(LB_EINVAL, "grad_norm: d_out is NULL");
    if (n > 0 && !grad)
        return fail(LB_EINVAL, "grad_norm: grad is NULL with n = %lld", (long long)n);
    Workspace ws;
    hipError_t e = workspace(ws);
    if (e != hipSuccess)
        return hip_fail("grad_norm (workspace)", e);
    lb::NormArgs a;
    a.g = grad;
    a.n = n;
    a.inv_scale = inv_scale;
    a.max_norm = max_norm;
    a.partial = ws.norm_partial;
    a.flag = ws.norm_flag;
    a.out = d_out;
    a.found_inf = d_found_inf;
    e = lb::launch_grad_norm(a, gt, tl_stream);
    if (e != hipSuccess)
        return hip_fail("grad_norm", e);
    return LB_OK;
}

int softmax_bwd(const void *P, const void *dY, void *dX, int64_t rows, int64_t cols, int dtype) {
    tl_error.clear();
    if (dtype != LB_F32 && dtype != LB_BF16)
        return fail(LB_EDTYPE, "softmax_bwd: dtype %d is not LB_F32 (0) or LB_BF16 (1)", dtype);
    if (rows < 0 || cols < 0)
        return fail(LB_EINVAL, "softmax_bwd: negative size rows=%lld cols=%lld", (long long)rows,
                    (long long)cols);
    if (rows >= ((int64_t)1 << 40) || cols >= ((int64_t)1 << 40))
        return fail(LB_EINVAL, "softmax_bwd: sizes must be below 2^40 (rows=%lld cols=%lld)", (long long)rows,
                    (long long)cols);
    if (rows > 0 && cols > 0 && (!P || !dY || !dX))
        return fail(LB_EINVAL, "softmax_bwd: NULL P, dY or dX with rows=%lld cols=%lld", (long long)rows,
                    (long long)cols);
    lb::SoftmaxArgs a;
    a.P = P;
    a.dY = dY;
    a.dX = dX;
    a.rows = rows;
    a.cols = cols;
    a.bf16 = dtype == LB_BF16;
    hipError_t e = lb::launch_softmax_bwd(a, tl_stream);
    if (e != hipSuccess)
        return hip_fail("softmax_bwd", e);
    return LB_OK;
}

int lb_set_stream(void *hip_stream) {
    tl_stream = static_cast<hipStream_t>(hip_stream);
    return LB_OK;
}

int lb_set_lin_bwd_path(int path) {
    tl_error.clear();
    if (path < LB_PATH_AUTO || path > LB_PATH_FUSED_SMALL_M)
        return fail(LB_EINVAL, "lb_set_lin_bwd_path: %d is not an LB_PATH_* value", path);
    tl_path = path;
    return LB_OK;
}

const char *lb_last_error(void) { return tl_error.c_str(); }

const char *lb_version(void) { return "linbwd 0.1.0 gfx950"; }

int lb_shutdown(void) {
    tl_error.clear();
    int cur = 0;
    hipError_t first = hipGetDevice(&cur);
    if (first != hipSuccess)
        return hip_fail("lb_shutdown", first);
    std::lock_guard<std::mutex> lock(ws_mutex);
    for (const auto &kv : ws_by_stream) {
        // one allocation per (device, stream); norm_partial is its start
        hipError_t e = hipSetDevice(kv.first.first);
        if (e == hipSuccess)
            e = hipFree(kv.second.norm_partial);
        if (e != hipSuccess && first == hipSuccess)
            first = e;
    }
    ws_by_stream.clear();
    {
        std::lock_guard<std::mutex> plock(pool_mutex);
        for (const auto &kv : pool_by_device) {
            hipError_t e = hipSetDevice(kv.first);
            if (e == hipSuccess)
                e = hipMemPoolDestroy(kv.second);
            if (e != hipSuccess && first == hipSuccess)
                first = e;
        }
        pool_by_device.clear();
    }
    const hipError_t e = hipSetDevice(cur);
    if (first == hipSuccess)
        first = e;
    return first == hipSuccess ? LB_OK : hip_fail("lb_shutdown", first);
}

} // extern "C"
