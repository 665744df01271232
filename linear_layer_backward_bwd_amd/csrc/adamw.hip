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
// bc2 = 1-b2^t from the host instead of evaluating pow per thread.
//
// The float arithmetic is evaluated in the order above with contraction off
// and IEEE division / square root, so each parameter's result does not
// depend on how the work is split.
//
// Optional parts of the training step around the update (pages: "GPU 优化实战
// Part 2", section "完整训练循环（整合一切）"): a clip factor read from device
// memory multiplies the unscaled gradient (g = (grad·inv_scale)·clip, two
// roundings; a factor of exactly 1 changes nothing), a device flag skips the
// whole step, and the updated W is also stored rounded to bf16 or fp16 for
// the next forward pass (2 more bytes per parameter in the same pass).
#include "device.h"
#include "kernels.h"

namespace lb {
namespace {

constexpr int kThreads = 256;
constexpr int kVec = 4; // parameters per thread

template <int GT> struct Grad;
template <> struct Grad<GRAD_F32> {
    static __device__ __forceinline__ void load4(const void *g, int64_t i, float (&out)[4]) {
        const f32x4_t a = *reinterpret_cast<const f32x4_t *>(static_cast<const float *>(g) + i);
        for (int e = 0; e < 4; ++e)
            out[e] = a[e];
    }
    static __device__ __forceinline__ float load1(const void *g, int64_t i) {
        return static_cast<const float *>(g)[i];
    }
};
template <> struct Grad<GRAD_F16> {
    static __device__ __forceinline__ void load4(const void *g, int64_t i, float (&out)[4]) {
        const u32x2_t w = *reinterpret_cast<const u32x2_t *>(static_cast<const uint16_t *>(g) + i);
        for (int e = 0; e < 2; ++e) {
            out[2 * e] = f16_bits_to_f32((uint16_t)(w[e] & 0xffffu));
            out[2 * e + 1] = f16_bits_to_f32((uint16_t)(w[e] >> 16));
        }
    }
    static __device__ __forceinline__ float load1(const void *g, int64_t i) {
        return f16_bits_to_f32(static_cast<const uint16_t *>(g)[i]);
    }
};
template <> struct Grad<GRAD_BF16> {
    static __device__ __forceinline__ void load4(const void *g, int64_t i, float (&out)[4]) {
        const u32x2_t w = *reinterpret_cast<const u32x2_t *>(static_cast<const uint16_t *>(g) + i);
        for (int e = 0; e < 2; ++e) {
            out[2 * e] = bf16_bits_to_f32(w[e] & 0xffffu);
            out[2 * e + 1] = bf16_bits_to_f32(w[e] >> 16);
        }
    }
    static __device__ __forceinline__ float load1(const void *g, int64_t i) {
        return bf16_bits_to_f32(static_cast<const uint16_t *>(g)[i]);
    }
};

__device__ __forceinline__ void update(float &w, float &m, float &v, float graw, float clip,
                                       const AdamWArgs &a) {
#pragma clang fp contract(off)
    const float g = (graw * a.inv_scale) * clip;
    m = a.b1 * m + a.one_minus_b1 * g;
    v = a.b2 * v + a.one_minus_b2 * g * g;
    const float mh = m / a.bc1;
    const float vh = v / a.bc2;
    w = w - a.lr * (mh / (sqrtf(vh) + a.eps) + a.wd * w);
}

// W rounded to nearest even as bf16 / fp16 bits (the hardware conversions
// round to nearest even; NaN stays NaN)
template <int SH> __device__ __forceinline__ uint16_t round16(float w) {
    if constexpr (SH == SHADOW_BF16)
        return f32_to_bf16_bits(w);
    else
        return __builtin_bit_cast(uint16_t, (_Float16)w);
}

// One thread per group of 4 parameters (the grid covers n exactly): on this
// part a single 16-byte access per stream per thread, with plain (temporal)
// loads and stores and no grid-stride loop, streams fastest.  VEC: W, m, v
// 16-byte aligned, the gradient and the 16-bit copy 8-byte aligned (16 for
// an fp32 gradient); the last partial group and misaligned buffers take the
// scalar loop.
template <int GT, int SH, bool VEC>
__global__ __launch_bounds__(kThreads) void k_adamw(AdamWArgs a) {
    const int64_t i = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * kVec;
    if (i >= a.n)
        return;
    if (a.skip && *a.skip != 0)
        return;
    const float clip = a.clip ? *a.clip : 1.0f;
    if (VEC && i + kVec <= a.n) {
        float g[4], w[4], m[4], v[4];
        Grad<GT>::load4(a.g, i, g);
        const f32x4_t W4 = *reinterpret_cast<const f32x4_t *>(a.W + i);
        const f32x4_t M4 = *reinterpret_cast<const f32x4_t *>(a.m + i);
        const f32x4_t V4 = *reinterpret_cast<const f32x4_t *>(a.v + i);
        for (int e = 0; e < 4; ++e) {
            w[e] = W4[e];
            m[e] = M4[e];
            v[e] = V4[e];
        }
#pragma unroll
        for (int e = 0; e < 4; ++e)
            update(w[e], m[e], v[e], g[e], clip, a);
        *reinterpret_cast<f32x4_t *>(a.W + i) = f32x4_t{w[0], w[1], w[2], w[3]};
        *reinterpret_cast<f32x4_t *>(a.m + i) = f32x4_t{m[0], m[1], m[2], m[3]};
        *reinterpret_cast<f32x4_t *>(a.v + i) = f32x4_t{v[0], v[1], v[2], v[3]};
        if constexpr (SH != SHADOW_NONE) {
            const u32x2_t h = {(uint32_t)round16<SH>(w[0]) | ((uint32_t)round16<SH>(w[1]) << 16),
                               (uint32_t)round16<SH>(w[2]) | ((uint32_t)round16<SH>(w[3]) << 16)};
            *reinterpret_cast<u32x2_t *>(a.W16 + i) = h;
        }
        return;
    }
    const int64_t end = i + kVec < a.n ? i + kVec : a.n;
    for (int64_t j = i; j < end; ++j) {
        float w = a.W[j], m = a.m[j], v = a.v[j];
        update(w, m, v, Grad<GT>::load1(a.g, j), clip, a);
        a.W[j] = w;
        a.m[j] = m;
        a.v[j] = v;
        if constexpr (SH != SHADOW_NONE)
            a.W16[j] = round16<SH>(w);
    }
}

template <int GT, int SH>
hipError_t launch_t(const AdamWArgs &a, hipStream_t s) {
    const uintptr_t galign = GT == GRAD_F32 ? 15u : 7u;
    const bool vec = ((reinterpret_cast<uintptr_t>(a.W) | reinterpret_cast<uintptr_t>(a.m) |
                       reinterpret_cast<uintptr_t>(a.v)) & 15u) == 0 &&
                     (reinterpret_cast<uintptr_t>(a.g) & galign) == 0 &&
                     (SH == SHADOW_NONE || (reinterpret_cast<uintptr_t>(a.W16) & 7u) == 0);
    const int64_t groups = (a.n + kVec - 1) / kVec;
    const int64_t blocks = (groups + kThreads - 1) / kThreads;
    if (blocks > 0x7fffffff)
        return hipErrorInvalidConfiguration;
    if (vec)
        hipLaunchKernelGGL((k_adamw<GT, SH, true>), dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL((k_adamw<GT, SH, false>), dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

template <int GT>
hipError_t launch_g(const AdamWArgs &a, ShadowType sh, hipStream_t s) {
    switch (sh) {
    case SHADOW_BF16: return launch_t<GT, SHADOW_BF16>(a, s);
    case SHADOW_F16: return launch_t<GT, SHADOW_F16>(a, s);
    default: return launch_t<GT, SHADOW_NONE>(a, s);
    }
}

} // namespace

hipError_t launch_adamw(const AdamWArgs &a, GradType gt, ShadowType shadow, hipStream_t s) {
    switch (gt) {
    case GRAD_F32: return launch_g<GRAD_F32>(a, shadow, s);
    case GRAD_F16: return launch_g<GRAD_F16>(a, shadow, s);
    default: return launch_g<GRAD_BF16>(a, shadow, s);
    }
}

} // namespace lb
