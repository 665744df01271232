// Softmax backward over the rows of a row-major [rows, cols] matrix:
//     dX[r,i] = P[r,i] * (dY[r,i] - sum_j P[r,j] * dY[r,j])
// with P the forward softmax output (pages: "GPU 优化实战 Part 2", section
// "Softmax 和 LayerNorm 的梯度（自定义内核）", softmax backward).
//
// HBM-bound: P and dY are read once and dX written once (3 elements of
// traffic per element).  The pages' kernel gives each row to one thread and
// walks the row twice; here one 64-lane wave owns a row of up to 4096
// columns and holds it in registers (16-byte loads, each lane's vectors 1 KiB
// apart so every load instruction of the wave covers 1 KiB of contiguous
// memory), reduces the dot product with a butterfly (every lane ends with the
// same value, as a + b == b + a), then writes dX from the registers.  Longer
// rows go to a block-per-row kernel that reads the row twice.
//
// The row is read completely before any of it is written, so dX may be the
// same buffer as dY or P.
#include "device.h"
#include "kernels.h"

namespace lb {
namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerBlock = kThreads / 64;

// dX is written once: non-temporal 16-byte stores (A/B, 524288 x 2048 bf16: 5.62 -> 6.00 TB/s).
template <typename T> struct V;
template <> struct V<float> {
    static constexpr int kN = 4;
    template <bool NT = false>
    static __device__ __forceinline__ void load(const void *p, int64_t i, float (&x)[4]) {
        const f32x4_t *q = reinterpret_cast<const f32x4_t *>(static_cast<const float *>(p) + i);
        const f32x4_t a = NT ? __builtin_nontemporal_load(q) : *q;
        for (int e = 0; e < 4; ++e)
            x[e] = a[e];
    }
    static __device__ __forceinline__ void store(void *p, int64_t i, const float (&x)[4]) {
        __builtin_nontemporal_store(f32x4_t{x[0], x[1], x[2], x[3]}, reinterpret_cast<f32x4_t *>(static_cast<float *>(p) + i));
    }
    static __device__ __forceinline__ float one(const void *p, int64_t i) { return static_cast<const float *>(p)[i]; }
    static __device__ __forceinline__ void put(void *p, int64_t i, float x) { static_cast<float *>(p)[i] = x; }
};
template <> struct V<uint16_t> { // bf16 bits
    static constexpr int kN = 8;
    template <bool NT = false>
    static __device__ __forceinline__ void load(const void *p, int64_t i, float (&x)[8]) {
        const u32x4_t *q = reinterpret_cast<const u32x4_t *>(static_cast<const uint16_t *>(p) + i);
        const u32x4_t w = NT ? __builtin_nontemporal_load(q) : *q;
        for (int e = 0; e < 4; ++e) {
            x[2 * e] = bf16_bits_to_f32(w[e] & 0xffffu);
            x[2 * e + 1] = bf16_bits_to_f32(w[e] >> 16);
        }
    }
    static __device__ __forceinline__ void store(void *p, int64_t i, const float (&x)[8]) {
        u32x4_t w;
        for (int e = 0; e < 4; ++e)
            w[e] = (uint32_t)f32_to_bf16_bits(x[2 * e]) | ((uint32_t)f32_to_bf16_bits(x[2 * e + 1]) << 16);
        __builtin_nontemporal_store(w, reinterpret_cast<u32x4_t *>(static_cast<uint16_t *>(p) + i));
    }
    static __device__ __forceinline__ float one(const void *p, int64_t i) {
        return bf16_bits_to_f32(static_cast<const uint16_t *>(p)[i]);
    }
    static __device__ __forceinline__ void put(void *p, int64_t i, float x) {
        static_cast<uint16_t *>(p)[i] = f32_to_bf16_bits(x);
    }
};

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int k = 32; k > 0; k >>= 1)
        x += __shfl_xor(x, k, 64);
    return x;
}

// One wave per row; lane l holds vectors v = 0..NV-1 covering columns
// (v*64 + l)*kN ... +kN-1.  VEC: cols a multiple of kN and all three buffers
// 16-byte aligned (so every row starts aligned); otherwise element accesses
// with a column check.
template <typename T, int NV, bool VEC>
__global__ __launch_bounds__(kThreads) void k_softmax_bwd_wave(const void *P, const void *dY, void *dX, int64_t rows,
                                                               int64_t cols) {
    constexpr int kN = V<T>::kN;
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
    if (row >= rows) // uniform over the wave
        return;
    const int64_t base = row * cols;
    float p[NV][kN], g[NV][kN];
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const int64_t c0 = (int64_t)(v * 64 + lane) * kN;
        if (VEC) {
            // Unconditional loads (a lane past the row end reads the row's first
            // vector and zeroes it): a load under a branch must land before the
            // branch rejoins, which had serialized the NV loads of a wave.
            const bool in = c0 < cols;
            V<T>::template load<true>(P, base + (in ? c0 : 0), p[v]); // read once: non-temporal
            V<T>::template load<true>(dY, base + (in ? c0 : 0), g[v]);
#pragma unroll
            for (int e = 0; e < kN; ++e) {
                p[v][e] = in ? p[v][e] : 0.0f;
                g[v][e] = in ? g[v][e] : 0.0f;
            }
        } else {
#pragma unroll
            for (int e = 0; e < kN; ++e) {
                const bool in = c0 + e < cols;
                p[v][e] = in ? V<T>::one(P, base + c0 + e) : 0.0f;
                g[v][e] = in ? V<T>::one(dY, base + c0 + e) : 0.0f;
            }
        }
    }
    float dot = 0.0f;
#pragma unroll
    for (int v = 0; v < NV; ++v)
#pragma unroll
        for (int e = 0; e < kN; ++e)
            dot += p[v][e] * g[v][e];
    dot = wave_sum(dot);
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const int64_t c0 = (int64_t)(v * 64 + lane) * kN;
        float x[kN];
#pragma unroll
        for (int e = 0; e < kN; ++e)
            x[e] = p[v][e] * (g[v][e] - dot);
        if (VEC) {
            if (c0 < cols)
                V<T>::store(dX, base + c0, x);
        } else {
#pragma unroll
            for (int e = 0; e < kN; ++e)
                if (c0 + e < cols)
                    V<T>::put(dX, base + c0 + e, x[e]);
        }
    }
}

// Rows longer than a wave holds: one block per row, the dot product in a
// first pass (per thread in column order, then a fixed tree over the block),
// dX in a second pass that reads P and dY again.
template <typename T, bool VEC>
__global__ __launch_bounds__(kThreads) void k_softmax_bwd_row(const void *P, const void *dY, void *dX, int64_t cols) {
    constexpr int kN = V<T>::kN;
    __shared__ float sh[kThreads];
    const int64_t base = (int64_t)blockIdx.x * cols;
    const int t = threadIdx.x;
    float dot = 0.0f;
    if (VEC) {
        for (int64_t c0 = (int64_t)t * kN; c0 < cols; c0 += (int64_t)kThreads * kN) {
            float p[kN], g[kN];
            V<T>::load(P, base + c0, p);
            V<T>::load(dY, base + c0, g);
#pragma unroll
            for (int e = 0; e < kN; ++e)
                dot += p[e] * g[e];
        }
    } else {
        for (int64_t c = t; c < cols; c += kThreads)
            dot += V<T>::one(P, base + c) * V<T>::one(dY, base + c);
    }
    sh[t] = dot;
    __syncthreads();
    for (int h = kThreads / 2; h > 0; h >>= 1) {
        if (t < h)
            sh[t] = sh[t] + sh[t + h];
        __syncthreads();
    }
    dot = sh[0];
    if (VEC) {
        for (int64_t c0 = (int64_t)t * kN; c0 < cols; c0 += (int64_t)kThreads * kN) {
            float p[kN], g[kN], x[kN];
            V<T>::load(P, base + c0, p);
            V<T>::load(dY, base + c0, g);
#pragma unroll
            for (int e = 0; e < kN; ++e)
                x[e] = p[e] * (g[e] - dot);
            V<T>::store(dX, base + c0, x);
        }
    } else {
        for (int64_t c = t; c < cols; c += kThreads)
            V<T>::put(dX, base + c, V<T>::one(P, base + c) * (V<T>::one(dY, base + c) - dot));
    }
}

template <typename T, int NV, bool VEC>
void launch_wave(const SoftmaxArgs &a, hipStream_t s) {
    const int64_t blocks = (a.rows + kRowsPerBlock - 1) / kRowsPerBlock;
    hipLaunchKernelGGL((k_softmax_bwd_wave<T, NV, VEC>), dim3((unsigned)blocks), dim3(kThreads), 0, s, a.P, a.dY,
                       a.dX, a.rows, a.cols);
}

template <typename T, bool VEC>
hipError_t launch_v(const SoftmaxArgs &a, hipStream_t s) {
    constexpr int64_t kWaveCols = 64 * V<T>::kN; // columns per vector slot of a wave
    const int64_t nv = (a.cols + kWaveCols - 1) / kWaveCols;
    if (nv <= 1)
        launch_wave<T, 1, VEC>(a, s);
    else if (nv <= 2)
        launch_wave<T, 2, VEC>(a, s);
    else if (nv <= 4)
        launch_wave<T, 4, VEC>(a, s);
    else if (nv <= 8)
        launch_wave<T, 8, VEC>(a, s);
    else if (nv * kWaveCols <= kSoftmaxWaveMaxCols)
        launch_wave<T, kSoftmaxWaveMaxCols / kWaveCols, VEC>(a, s);
    else if (a.rows > 0x7fffffff)
        return hipErrorInvalidConfiguration;
    else
        hipLaunchKernelGGL((k_softmax_bwd_row<T, VEC>), dim3((unsigned)a.rows), dim3(kThreads), 0, s, a.P, a.dY,
                           a.dX, a.cols);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const SoftmaxArgs &a, hipStream_t s) {
    const bool vec = a.cols % V<T>::kN == 0 &&
                     ((reinterpret_cast<uintptr_t>(a.P) | reinterpret_cast<uintptr_t>(a.dY) |
                       reinterpret_cast<uintptr_t>(a.dX)) & 15u) == 0;
    return vec ? launch_v<T, true>(a, s) : launch_v<T, false>(a, s);
}

} // namespace

hipError_t launch_softmax_bwd(const SoftmaxArgs &a, hipStream_t s) {
    if (a.rows == 0 || a.cols == 0)
        return hipSuccess;
    if ((a.rows + kRowsPerBlock - 1) / kRowsPerBlock > 0x7fffffff)
        return hipErrorInvalidConfiguration;
    return a.bf16 ? launch_t<uint16_t>(a, s) : launch_t<float>(a, s);
}

} // namespace lb
