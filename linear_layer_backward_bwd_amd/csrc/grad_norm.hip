// Global L2 norm of the unscaled gradient, the clip factor and an inf/NaN
// flag, all left in device memory (pages: "GPU 优化实战 Part 2", section
// "完整训练循环（整合一切）", the clipping step of the loop: the norm of the
// fp32 gradient, and a scale of max_norm / norm when it exceeds max_norm).
//
//   g32  = float(grad) * inv_scale                      fp32, as in the AdamW pass
//   norm = sqrt(sum g32^2)                              exact squares, fp64 sums
//   clip = norm > max_norm ? max_norm / norm : 1        fp32; max_norm <= 0: 1
//
// Read-only and HBM-bound (2 or 4 bytes per parameter).  Two launches:
// k_norm_partial reduces a contiguous chunk per block, per thread in a fixed
// order and then across the block in a fixed tree order; k_norm_final
// combines the per-block partials in a fixed order and writes the results.
// The grid depends only on n and the gradient type, so the result does not
// depend on timing.
#include "device.h"
#include "kernels.h"

namespace lb {
namespace {

constexpr int kThreads = 256;
constexpr int kVec = 8; // gradient elements per thread per iteration

// The gradient is read once: non-temporal 16-byte loads.
template <int GT> struct Load8;
template <> struct Load8<GRAD_F32> {
    static __device__ __forceinline__ void load(const void *g, int64_t i, float (&x)[8]) {
        const f32x4_t a = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t *>(static_cast<const float *>(g) + i));
        const f32x4_t b = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t *>(static_cast<const float *>(g) + i + 4));
        for (int e = 0; e < 4; ++e) {
            x[e] = a[e];
            x[4 + e] = b[e];
        }
    }
    static __device__ __forceinline__ float one(const void *g, int64_t i) { return static_cast<const float *>(g)[i]; }
};
template <> struct Load8<GRAD_F16> {
    static __device__ __forceinline__ void load(const void *g, int64_t i, float (&x)[8]) {
        const u32x4_t w = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(static_cast<const uint16_t *>(g) + i));
        for (int e = 0; e < 4; ++e) {
            x[2 * e] = f16_bits_to_f32((uint16_t)(w[e] & 0xffffu));
            x[2 * e + 1] = f16_bits_to_f32((uint16_t)(w[e] >> 16));
        }
    }
    static __device__ __forceinline__ float one(const void *g, int64_t i) {
        return f16_bits_to_f32(static_cast<const uint16_t *>(g)[i]);
    }
};
template <> struct Load8<GRAD_BF16> {
    static __device__ __forceinline__ void load(const void *g, int64_t i, float (&x)[8]) {
        const u32x4_t w = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(static_cast<const uint16_t *>(g) + i));
        for (int e = 0; e < 4; ++e) {
            x[2 * e] = bf16_bits_to_f32(w[e] & 0xffffu);
            x[2 * e + 1] = bf16_bits_to_f32(w[e] >> 16);
        }
    }
    static __device__ __forceinline__ float one(const void *g, int64_t i) {
        return bf16_bits_to_f32(static_cast<const uint16_t *>(g)[i]);
    }
};

__device__ __forceinline__ void accumulate(float raw, float inv_scale, double &s, int &bad) {
#pragma clang fp contract(off)
    const float x = raw * inv_scale;
    bad |= !__builtin_isfinite(x);
    s += (double)x * (double)x; // the product is exact in fp64
}

// Fixed-order tree over a block of T threads: pairs (t, t + h) for
// h = T/2, T/4, ...
template <int T> __device__ __forceinline__ void block_reduce(double &s, int &bad, double *sh, int *shb) {
    const int t = threadIdx.x;
    sh[t] = s;
    shb[t] = bad;
    __syncthreads();
    for (int h = T / 2; h > 0; h >>= 1) {
        if (t < h) {
            sh[t] = sh[t] + sh[t + h];
            shb[t] |= shb[t + h];
        }
        __syncthreads();
    }
    s = sh[0];
    bad = shb[0];
}

// Loads in flight per thread: 8 x 16 B for a 16-bit gradient, 4 x 32 B for
// fp32, so one unrolled round of a block reads 32 KiB.
template <int GT> constexpr int kUnroll = GT == GRAD_F32 ? 4 : 8;

// Block b reduces the contiguous elements [b*chunk, min((b+1)*chunk, n)),
// chunk a whole number of rounds of kThreads * kUnroll 8-element groups, in
// rounds of kUnroll coalesced loads per thread (at the sizes of a model's
// gradient most blocks run exactly one round).  VEC: grad 16-byte aligned;
// the last n % 8 elements, and all of them when misaligned, are read one by
// one.
template <int GT, bool VEC>
__global__ __launch_bounds__(kThreads) void k_norm_partial(const void *g, int64_t n, int64_t chunk,
                                                          float inv_scale, double *partial, int *flag) {
    __shared__ double sh[kThreads];
    __shared__ int shb[kThreads];
    constexpr int U = kUnroll<GT>;
    double s = 0.0;
    int bad = 0;
    const int64_t lo = (int64_t)blockIdx.x * chunk;
    const int64_t hi = lo + chunk < n ? lo + chunk : n;
    int64_t i = lo + (int64_t)threadIdx.x * kVec; // first element of this thread's group
    if (VEC) {
        const int64_t hi8 = hi - hi % kVec; // lo is a multiple of 8
        for (; i + (int64_t)(U - 1) * kThreads * kVec + kVec <= hi8; i += (int64_t)U * kThreads * kVec) {
            float x[U][8];
#pragma unroll
            for (int u = 0; u < U; ++u)
                Load8<GT>::load(g, i + (int64_t)u * kThreads * kVec, x[u]);
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    accumulate(x[u][e], inv_scale, s, bad);
        }
        for (; i + kVec <= hi8; i += kThreads * kVec) {
            float x[8];
            Load8<GT>::load(g, i, x);
#pragma unroll
            for (int e = 0; e < 8; ++e)
                accumulate(x[e], inv_scale, s, bad);
        }
        for (int64_t j = hi8 + threadIdx.x; j < hi; j += kThreads)
            accumulate(Load8<GT>::one(g, j), inv_scale, s, bad);
    } else {
        for (int64_t j = lo + threadIdx.x; j < hi; j += kThreads)
            accumulate(Load8<GT>::one(g, j), inv_scale, s, bad);
    }
    block_reduce<kThreads>(s, bad, sh, shb);
    if (threadIdx.x == 0) {
        partial[blockIdx.x] = s;
        flag[blockIdx.x] = bad;
    }
}

// One block of kFinalThreads combines the partials: thread t takes entries
// t, t + kFinalThreads, ... (all loads issued before the in-order sum, so the
// pass is not a chain of dependent memory latencies), then the tree.
constexpr int kFinalThreads = 1024;
constexpr int kFinalPerThread = kNormMaxBlocks / kFinalThreads;
static_assert(kNormMaxBlocks % kFinalThreads == 0, "partials split evenly over the final block");

__global__ __launch_bounds__(kFinalThreads) void k_norm_final(const double *partial, const int *flag, int nblocks,
                                                             float max_norm, float *out, int32_t *found_inf) {
    __shared__ double sh[kFinalThreads];
    __shared__ int shb[kFinalThreads];
    double p[kFinalPerThread];
    int f[kFinalPerThread];
#pragma unroll
    for (int k = 0; k < kFinalPerThread; ++k) {
        const int b = threadIdx.x + k * kFinalThreads;
        p[k] = b < nblocks ? partial[b] : 0.0;
        f[k] = b < nblocks ? flag[b] : 0;
    }
    double s = 0.0;
    int bad = 0;
#pragma unroll
    for (int k = 0; k < kFinalPerThread; ++k) {
        s += p[k];
        bad |= f[k];
    }
    block_reduce<kFinalThreads>(s, bad, sh, shb);
    if (threadIdx.x == 0) {
#pragma clang fp contract(off)
        const float norm = (float)__builtin_sqrt(s);
        out[0] = norm;
        out[1] = (max_norm > 0.0f && norm > max_norm) ? max_norm / norm : 1.0f;
        if (found_inf)
            *found_inf = bad;
    }
}

template <int GT>
hipError_t launch_t(const NormArgs &a, hipStream_t s) {
    // chunk: whole rounds, enough of them that at most kNormMaxBlocks blocks
    // cover n; the grid depends only on n and the gradient type
    const int64_t round = (int64_t)kThreads * kUnroll<GT> * kVec;
    const int64_t rounds = (a.n + round - 1) / round;
    const int64_t per_block = rounds <= kNormMaxBlocks ? 1 : (rounds + kNormMaxBlocks - 1) / kNormMaxBlocks;
    const int64_t chunk = per_block * round;
    const int nblocks = a.n == 0 ? 1 : (int)((a.n + chunk - 1) / chunk);
    const bool vec = (reinterpret_cast<uintptr_t>(a.g) & 15u) == 0;
    if (vec)
        hipLaunchKernelGGL((k_norm_partial<GT, true>), dim3(nblocks), dim3(kThreads), 0, s, a.g, a.n, chunk,
                           a.inv_scale, a.partial, a.flag);
    else
        hipLaunchKernelGGL((k_norm_partial<GT, false>), dim3(nblocks), dim3(kThreads), 0, s, a.g, a.n, chunk,
                           a.inv_scale, a.partial, a.flag);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(k_norm_final, dim3(1), dim3(kFinalThreads), 0, s, a.partial, a.flag, nblocks, a.max_norm,
                       a.out, a.found_inf);
    return hipGetLastError();
}

} // namespace

hipError_t launch_grad_norm(const NormArgs &a, GradType gt, hipStream_t s) {
    switch (gt) {
    case GRAD_F32: return launch_t<GRAD_F32>(a, s);
    case GRAD_F16: return launch_t<GRAD_F16>(a, s);
    default: return launch_t<GRAD_BF16>(a, s);
    }
}

} // namespace lb
