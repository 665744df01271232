// Bias gradient of a Linear layer: db[n] = sum over rows m of dY[m, n].
//
// The forward with a bias is Y = X·W + b with b added to every one of the M
// rows (pages: "GPU 优化实战 Part 2", section "反向传播——Linear 层的梯度",
// which writes the forward with a bias and then speaks of dW and db), so the
// gradient of b is the column sum of dY.  fp32 out, like dW.
//
// HBM-bound: dY is read once (2 or 4 bytes per element), db written once.
// Split over rows so that a launch has enough blocks to fill the chip:
//   k_bias_partial  block (strip, split) sums a row range of one column strip;
//                   each thread owns 16 bytes of columns and keeps up to two
//                   batches of kUnroll rows of loads in flight, the 4 waves take
//                   interleaved rows and are combined through LDS in wave order.
//   k_bias_final    per column, the split partials in a fixed order, summed
//                   in fp64 and rounded once.  With one split the partial kernel
//                   writes db itself.
// The grid depends only on M, N and the element type, so results repeat bit
// for bit.
#include "device.h"
#include "kernels.h"

namespace lb {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kUnroll = 4;          // rows of 16-byte loads per batch (two batches in flight)
constexpr int kFinalBatch = 16;     // independent partial loads per final-pass round
constexpr int kTargetBlocks = 1024; // enough waves to keep HBM busy; 2048 was 5% slower (more partials)

// dY is read once: non-temporal 16-byte loads.
template <typename T> struct Elt;
template <> struct Elt<uint16_t> { // bf16 bits
    static constexpr int kCols = 8;
    static __device__ __forceinline__ void load(const void *p, int64_t i, float (&x)[8]) {
        const u32x4_t w = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(static_cast<const uint16_t *>(p) + i));
        for (int e = 0; e < 4; ++e) {
            x[2 * e] = bf16_bits_to_f32(w[e] & 0xffffu);
            x[2 * e + 1] = bf16_bits_to_f32(w[e] >> 16);
        }
    }
    static __device__ __forceinline__ float one(const void *p, int64_t i) {
        return bf16_bits_to_f32(static_cast<const uint16_t *>(p)[i]);
    }
};
template <> struct Elt<float> {
    static constexpr int kCols = 4;
    static __device__ __forceinline__ void load(const void *p, int64_t i, float (&x)[4]) {
        const f32x4_t a = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t *>(static_cast<const float *>(p) + i));
        for (int e = 0; e < 4; ++e)
            x[e] = a[e];
    }
    static __device__ __forceinline__ float one(const void *p, int64_t i) { return static_cast<const float *>(p)[i]; }
};

// VEC: dY 16-byte aligned and N a multiple of kCols (every thread's columns
// are one aligned 16-byte access per row); otherwise element loads with a
// column check.
template <typename T, bool VEC>
__global__ __launch_bounds__(kThreads) void k_bias_partial(const void *dY, int64_t M, int64_t N, int64_t rows_per,
                                                           float *out, int64_t out_stride) {
    constexpr int C = Elt<T>::kCols;
    constexpr int kStrip = 64 * C;
    __shared__ float sh[kWaves][kStrip];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t col0 = (int64_t)blockIdx.x * kStrip + lane * C;
    const int64_t lo = (int64_t)blockIdx.y * rows_per;
    const int64_t hi = lo + rows_per < M ? lo + rows_per : M;
    float acc[C];
#pragma unroll
    for (int c = 0; c < C; ++c)
        acc[c] = 0.0f;
    if (VEC) {
        if (col0 < N) {
            int64_t r = lo + wave;
            // Two batches: the next batch's loads go out before this one is
            // added, so a thread never waits with nothing in flight (A/B on the
            // block's four dY: batches of 8 loaded and then added, 5.40 TB/s;
            // batches of 16, 5.47; two batches of 8, 5.58; two of 4, 5.69).
            // The rows are added in the same order either way.
            constexpr int64_t B = (int64_t)kWaves * kUnroll; // rows per batch
            constexpr int64_t L = (int64_t)kWaves * (kUnroll - 1);
            if (r + B + L < hi) {
                float xa[kUnroll][C], xb[kUnroll][C];
#pragma unroll
                for (int u = 0; u < kUnroll; ++u)
                    Elt<T>::load(dY, (r + (int64_t)u * kWaves) * N + col0, xa[u]);
                // xa holds the batch at r; batches r + B and r + 2B are in range
                for (; r + 2 * B + L < hi; r += 2 * B) {
#pragma unroll
                    for (int u = 0; u < kUnroll; ++u)
                        Elt<T>::load(dY, (r + B + (int64_t)u * kWaves) * N + col0, xb[u]);
#pragma unroll
                    for (int u = 0; u < kUnroll; ++u)
#pragma unroll
                        for (int c = 0; c < C; ++c)
                            acc[c] += xa[u][c];
#pragma unroll
                    for (int u = 0; u < kUnroll; ++u)
                        Elt<T>::load(dY, (r + 2 * B + (int64_t)u * kWaves) * N + col0, xa[u]);
#pragma unroll
                    for (int u = 0; u < kUnroll; ++u)
#pragma unroll
                        for (int c = 0; c < C; ++c)
                            acc[c] += xb[u][c];
                }
#pragma unroll
                for (int u = 0; u < kUnroll; ++u)
#pragma unroll
                    for (int c = 0; c < C; ++c)
                        acc[c] += xa[u][c];
                r += B;
            }
            for (; r + L < hi; r += B) {
                float x[kUnroll][C];
#pragma unroll
                for (int u = 0; u < kUnroll; ++u)
                    Elt<T>::load(dY, (r + (int64_t)u * kWaves) * N + col0, x[u]);
#pragma unroll
                for (int u = 0; u < kUnroll; ++u)
#pragma unroll
                    for (int c = 0; c < C; ++c)
                        acc[c] += x[u][c];
            }
            for (; r < hi; r += kWaves) {
                float x[C];
                Elt<T>::load(dY, r * N + col0, x);
#pragma unroll
                for (int c = 0; c < C; ++c)
                    acc[c] += x[c];
            }
        }
    } else {
        for (int64_t r = lo + wave; r < hi; r += kWaves)
#pragma unroll
            for (int c = 0; c < C; ++c)
                if (col0 + c < N)
                    acc[c] += Elt<T>::one(dY, r * N + col0 + c);
    }
#pragma unroll
    for (int c = 0; c < C; ++c)
        sh[wave][lane * C + c] = acc[c];
    __syncthreads();
    for (int j = threadIdx.x; j < kStrip; j += kThreads) {
        const int64_t col = (int64_t)blockIdx.x * kStrip + j;
        if (col < N) {
            float s = sh[0][j];
#pragma unroll
            for (int w = 1; w < kWaves; ++w)
                s += sh[w][j];
            out[(int64_t)blockIdx.y * out_stride + col] = s;
        }
    }
}

// Block = kFinalCols columns x kFinalGroups split groups: thread (g, c) sums
// splits g, g + kFinalGroups, ... of its column in increasing order (loads
// issued kFinalBatch at a time), then the groups are added in group order.
constexpr int kFinalCols = 32;
constexpr int kFinalGroups = kThreads / kFinalCols;

__global__ __launch_bounds__(kThreads) void k_bias_final(const float *partial, int splits, int64_t N, float *db) {
    __shared__ double sh[kFinalGroups][kFinalCols];
    const int c = threadIdx.x % kFinalCols, g = threadIdx.x / kFinalCols;
    const int64_t n = (int64_t)blockIdx.x * kFinalCols + c;
    double s = 0.0;
    if (n < N) {
        for (int s0 = g; s0 < splits; s0 += kFinalGroups * kFinalBatch) {
            // unconditional loads (a split past the end reads split 0 and is
            // dropped): a load under a branch must land before the branch
            // rejoins, which had made the batch's loads go out one at a time
            float p[kFinalBatch];
#pragma unroll
            for (int k = 0; k < kFinalBatch; ++k) {
                const int sp = s0 + k * kFinalGroups;
                p[k] = partial[(int64_t)(sp < splits ? sp : 0) * N + n];
            }
#pragma unroll
            for (int k = 0; k < kFinalBatch; ++k)
                p[k] = s0 + k * kFinalGroups < splits ? p[k] : 0.0f;
#pragma unroll
            for (int k = 0; k < kFinalBatch; ++k)
                s += (double)p[k];
        }
    }
    sh[g][c] = s;
    __syncthreads();
    if (g == 0 && n < N) {
        double t = sh[0][c];
#pragma unroll
        for (int k = 1; k < kFinalGroups; ++k)
            t += sh[k][c];
        db[n] = (float)t;
    }
}

template <typename T>
hipError_t launch_t(const BiasArgs &a, hipStream_t s) {
    constexpr int C = Elt<T>::kCols;
    constexpr int64_t kStrip = 64 * C;
    const int64_t strips = (a.N + kStrip - 1) / kStrip;
    if (strips > 0x7fffffff)
        return hipErrorInvalidConfiguration;
    // splits: toward kTargetBlocks blocks, at least 64 rows each, and within
    // the workspace (splits * N partials)
    int64_t splits = (kTargetBlocks + strips - 1) / strips;
    const int64_t by_rows = (a.M + 63) / 64;
    if (splits > by_rows)
        splits = by_rows;
    if (splits > kBiasMaxSplits)
        splits = kBiasMaxSplits;
    if (splits * a.N > kBiasWorkspaceFloats)
        splits = kBiasWorkspaceFloats / a.N;
    if (splits < 1)
        splits = 1;
    const int64_t rows_per = (a.M + splits - 1) / splits;
    const bool vec = (reinterpret_cast<uintptr_t>(a.dY) & 15u) == 0 && a.N % C == 0;
    float *out = splits == 1 ? a.db : a.partial;
    const dim3 grid((unsigned)strips, (unsigned)splits);
    if (vec)
        hipLaunchKernelGGL((k_bias_partial<T, true>), grid, dim3(kThreads), 0, s, a.dY, a.M, a.N, rows_per, out,
                           a.N);
    else
        hipLaunchKernelGGL((k_bias_partial<T, false>), grid, dim3(kThreads), 0, s, a.dY, a.M, a.N, rows_per, out,
                           a.N);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || splits == 1)
        return e;
    hipLaunchKernelGGL(k_bias_final, dim3((unsigned)((a.N + kFinalCols - 1) / kFinalCols)), dim3(kThreads), 0, s,
                       a.partial, (int)splits, a.N, a.db);
    return hipGetLastError();
}

} // namespace

hipError_t launch_bias_grad(const BiasArgs &a, hipStream_t s) {
    if (a.N == 0)
        return hipSuccess;
    return a.bf16 ? launch_t<uint16_t>(a, s) : launch_t<float>(a, s);
}

} // namespace lb
