// Fused unscale + AdamW over fp32 master weights: one HBM streaming pass.
//
// Per parameter (pages: "GPU 优化实战 Part 2", sections "AdamW 优化器——融合内核"
// and "混合精度训练（FP16 / BF16）"; "Mastering LLM Training with CUDA and
// ROCm", section "AdamW Algorithm"):
//     g = float(grad)·inv_scale;  m = b1·m + (1-b1)·g;  v = b2·v + (1-b2)·g·g
//     W = W - lr·( (m/bc1) / (sqrt(v/bc2) + eps) + wd·W )
//
// The kernel is memory bound: it reads grad, W, m, v once and writes W, m, v
// once (26 B per parameter with a 16-bit gradient, 28 B with fp32), never
// writes the gradient, and takes the bias corrections bc1 = 1-b1^t,
// bc2 = 1-b2^t from the host instead of evaluating pow per thread.  Each
// thread moves 8 parameters per trip with 16-byte non-temporal accesses, in
// a grid-stride loop sized to keep every CU's memory pipeline full.
//
// The float arithmetic is evaluated in the order above with contraction off
// and IEEE division / square root, so each parameter's result does not
// depend on how the work is split.
#include "device.h"
#include "kernels.h"

namespace lb {
namespace {

constexpr int kThreads = 256;
constexpr int kVec = 8; // parameters per thread per trip

template <int GT> struct Grad;
template <> struct Grad<GRAD_F32> {
    static __device__ __forceinline__ void load8(const void *g, int64_t i, float (&out)[8]) {
        const f32x4_t *p = reinterpret_cast<const f32x4_t *>(static_cast<const float *>(g) + i);
        f32x4_t a = __builtin_nontemporal_load(p);
        f32x4_t b = __builtin_nontemporal_load(p + 1);
        for (int e = 0; e < 4; ++e) {
            out[e] = a[e];
            out[4 + e] = b[e];
        }
    }
    static __device__ __forceinline__ float load1(const void *g, int64_t i) {
        return static_cast<const float *>(g)[i];
    }
};
template <> struct Grad<GRAD_F16> {
    static __device__ __forceinline__ void load8(const void *g, int64_t i, float (&out)[8]) {
        const u32x4_t *p = reinterpret_cast<const u32x4_t *>(static_cast<const uint16_t *>(g) + i);
        u32x4_t w = __builtin_nontemporal_load(p);
        for (int e = 0; e < 4; ++e) {
            out[2 * e] = f16_bits_to_f32((uint16_t)(w[e] & 0xffffu));
            out[2 * e + 1] = f16_bits_to_f32((uint16_t)(w[e] >> 16));
        }
    }
    static __device__ __forceinline__ float load1(const void *g, int64_t i) {
        return f16_bits_to_f32(static_cast<const uint16_t *>(g)[i]);
    }
};
template <> struct Grad<GRAD_BF16> {
    static __device__ __forceinline__ void load8(const void *g, int64_t i, float (&out)[8]) {
        const u32x4_t *p = reinterpret_cast<const u32x4_t *>(static_cast<const uint16_t *>(g) + i);
        u32x4_t w = __builtin_nontemporal_load(p);
        for (int e = 0; e < 4; ++e) {
            out[2 * e] = bf16_bits_to_f32(w[e] & 0xffffu);
            out[2 * e + 1] = bf16_bits_to_f32(w[e] >> 16);
        }
    }
    static __device__ __forceinline__ float load1(const void *g, int64_t i) {
        return bf16_bits_to_f32(static_cast<const uint16_t *>(g)[i]);
    }
};

__device__ __forceinline__ void update(float &w, float &m, float &v, float graw, const AdamWArgs &a) {
#pragma clang fp contract(off)
    const float g = graw * a.inv_scale;
    m = a.b1 * m + a.one_minus_b1 * g;
    v = a.b2 * v + a.one_minus_b2 * g * g;
    const float mh = m / a.bc1;
    const float vh = v / a.bc2;
    w = w - a.lr * (mh / (sqrtf(vh) + a.eps) + a.wd * w);
}

__device__ __forceinline__ void load8f(const float *p, float (&out)[8]) {
    const f32x4_t *q = reinterpret_cast<const f32x4_t *>(p);
    f32x4_t x = __builtin_nontemporal_load(q);
    f32x4_t y = __builtin_nontemporal_load(q + 1);
    for (int e = 0; e < 4; ++e) {
        out[e] = x[e];
        out[4 + e] = y[e];
    }
}

__device__ __forceinline__ void store8f(float *p, const float (&in)[8]) {
    f32x4_t *q = reinterpret_cast<f32x4_t *>(p);
    f32x4_t x = {in[0], in[1], in[2], in[3]};
    f32x4_t y = {in[4], in[5], in[6], in[7]};
    __builtin_nontemporal_store(x, q);
    __builtin_nontemporal_store(y, q + 1);
}

// VEC: all four buffers 16-byte aligned; groups of 8 parameters, scalar tail.
template <int GT, bool VEC>
__global__ __launch_bounds__(kThreads) void k_adamw(AdamWArgs a) {
    const int64_t tid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int64_t nthreads = (int64_t)gridDim.x * kThreads;
    int64_t done = 0;
    if (VEC) {
        const int64_t groups = a.n / kVec;
        for (int64_t gi = tid; gi < groups; gi += nthreads) {
            const int64_t i = gi * kVec;
            float g[8], w[8], m[8], v[8];
            Grad<GT>::load8(a.g, i, g);
            load8f(a.W + i, w);
            load8f(a.m + i, m);
            load8f(a.v + i, v);
#pragma unroll
            for (int e = 0; e < 8; ++e)
                update(w[e], m[e], v[e], g[e], a);
            store8f(a.W + i, w);
            store8f(a.m + i, m);
            store8f(a.v + i, v);
        }
        done = groups * kVec;
    }
    for (int64_t i = done + tid; i < a.n; i += nthreads) {
        float w = a.W[i], m = a.m[i], v = a.v[i];
        update(w, m, v, Grad<GT>::load1(a.g, i), a);
        a.W[i] = w;
        a.m[i] = m;
        a.v[i] = v;
    }
}

template <int GT>
hipError_t launch_t(const AdamWArgs &a, hipStream_t s) {
    const bool vec = ((reinterpret_cast<uintptr_t>(a.W) | reinterpret_cast<uintptr_t>(a.m) |
                       reinterpret_cast<uintptr_t>(a.v) | reinterpret_cast<uintptr_t>(a.g)) & 15u) == 0;
    // enough resident waves to cover HBM latency: 256 CUs x 8 blocks of 4 waves
    const int64_t work = vec ? (a.n + kVec - 1) / kVec : a.n;
    int64_t blocks = (work + kThreads - 1) / kThreads;
    if (blocks > 2048) blocks = 2048;
    if (blocks < 1) blocks = 1;
    if (vec)
        hipLaunchKernelGGL((k_adamw<GT, true>), dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL((k_adamw<GT, false>), dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

} // namespace

hipError_t launch_adamw(const AdamWArgs &a, GradType gt, hipStream_t s) {
    switch (gt) {
    case GRAD_F32: return launch_t<GRAD_F32>(a, s);
    case GRAD_F16: return launch_t<GRAD_F16>(a, s);
    default: return launch_t<GRAD_BF16>(a, s);
    }
}

} // namespace lb
