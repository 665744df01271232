// Linear-layer backward on gfx950: dX = dY·Wᵀ and dW = Xᵀ·dY.
//
// Pages: "GPU 优化实战 Part 2", section "反向传播——Linear 层的梯度" (a forward
// product becomes two backward products); "GPU 如何训练模型：从算子到 Kernel",
// section "一个线性层，前向和反向到底在算什么" (X[M,K], W[K,N], G = dL/dY [M,N];
// 4MKN FLOP for the pair; transposes expressed through strides, not copies).
//
// Both products are written as one tile problem  C[i,j] = Σ_r A(i,r)·B(j,r):
//
//   dX[m,k] = Σ_n dY[m,n]·W[k,n]   i=m, j=k, r=n   A, B "r-contiguous"  (rows of dY, W)
//   dW[k,n] = Σ_m X[m,k]·dY[m,n]   i=k, j=n, r=m   A, B "outer-contiguous" (columns of X, dY)
//
// Kernels:
//   k_lin_bwd_mfma   bf16 MFMA (v_mfma_f32_32x32x16_bf16, fp32 accumulate), 256x256
//                    output tile per 4-wave workgroup, reduction in slabs of 64 staged
//                    through a double-buffered, XOR-swizzled LDS tile.  One launch runs
//                    the tiles of both products; blocks are ordered longest reduction
//                    first and mapped so that each XCD works on a compact group of tiles.
//                    For dW the reduction index is the slow index of both operands; each
//                    thread loads an 8x8 block (8 rows of 16 bytes) and transposes it in
//                    registers before the LDS store, so LDS always holds tiles with the
//                    reduction index contiguous and every MFMA operand is one 16-byte
//                    LDS read.
//   k_dx_smallm      dX for M <= 64 (decode-like): bound by streaming W once, so the
//                    reduction over n is split across the waves of a block and
//                    operands go straight from global memory into MFMA registers.
//   k_lin_bwd_simt   any dtype / alignment / shape: fp32 path and ragged bf16 shapes.
#include "device.h"
#include "kernels.h"

#include <algorithm>

namespace lb {
namespace {

// ------------------------------------------------------------------------
// MFMA tile kernel
// ------------------------------------------------------------------------
constexpr int kTile = 256;                        // output tile edge (i and j)
constexpr int kBK = 64;                           // reduction slab per stage
constexpr int kThreads = 256;                     // 4 waves, 2x2, 128x128 each
constexpr int kRowBytes = kBK * 2;                // one LDS row: 64 bf16
constexpr int kOperandBytes = kTile * kRowBytes;  // 32 KiB
constexpr int kStageBytes = 2 * kOperandBytes;    // A and B
constexpr int kLdsBytes = 2 * kStageBytes;        // double buffered: 128 KiB
constexpr int kGroupI = 4;                        // tile rows per raster group

// 16-byte chunk c (0..7) of LDS row `row`: XOR swizzle so that the MFMA reads
// (8 consecutive rows, same chunk) and both store patterns hit distinct banks.
__device__ __forceinline__ int lds_off(int row, int chunk) {
    const int swz = (row & 7) ^ ((row >> 3) & 7);
    return row * kRowBytes + ((chunk ^ swz) << 4);
}

enum JobKind { JOB_DX = 0, JOB_DW = 1 };

struct TileJob {
    const uint16_t *a; // operand giving output rows i
    const uint16_t *b; // operand giving output cols j
    void *c;           // output, row-major [I, J], leading dim J
    int64_t I, J, R;   // output rows, cols, reduction length
    int64_t lda, ldb;  // leading dims of a and b in elements
    int tiles_i, tiles_j, ntiles;
    int kind;          // JOB_DX: r-contiguous operands, bf16 out; JOB_DW: outer-contiguous, fp32 out
};

struct MfmaParams {
    TileJob job[2];
    int njobs;
};

// r-contiguous operand: element (o, r) at base[o*ld + r].  Thread t loads
// rows (t>>3) + 32p, chunk t&7 of the slab: each wave instruction reads
// eight 128-byte row segments.
__device__ __forceinline__ void load_rc(u32x4_t (&reg)[8], const uint16_t *base, int64_t ld,
                                        int64_t O, int64_t R, int64_t o0, int64_t r0, int t) {
    const int c = t & 7;
    const int orow = t >> 3;
    const int64_t r = r0 + 8 * c;
    const bool rok = r < R; // R % 8 == 0: a chunk is entirely in or out
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        const int64_t o = o0 + orow + 32 * p;
        if (rok && o < O)
            reg[p] = *reinterpret_cast<const u32x4_t *>(base + o * ld + r);
        else
            reg[p] = u32x4_t{0, 0, 0, 0};
    }
}

__device__ __forceinline__ void store_rc(char *lds, const u32x4_t (&reg)[8], int t) {
    const int c = t & 7;
    const int orow = t >> 3;
#pragma unroll
    for (int p = 0; p < 8; ++p)
        *reinterpret_cast<u32x4_t *>(lds + lds_off(orow + 32 * p, c)) = reg[p];
}

// outer-contiguous operand: element (o, r) at base[r*ld + o].  Thread t
// loads the 8x8 block r in [8(t>>5), +8), o in [8(t&31), +8): eight 16-byte
// loads, one per r; a wave instruction reads two 512-byte row segments.
__device__ __forceinline__ void load_oc(u32x4_t (&reg)[8], const uint16_t *base, int64_t ld,
                                        int64_t O, int64_t R, int64_t o0, int64_t r0, int t) {
    const int oc = t & 31;
    const int rb = t >> 5;
    const int64_t o = o0 + 8 * oc;
    const bool ook = o < O; // O % 8 == 0
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        const int64_t r = r0 + 8 * rb + p;
        if (ook && r < R)
            reg[p] = *reinterpret_cast<const u32x4_t *>(base + r * ld + o);
        else
            reg[p] = u32x4_t{0, 0, 0, 0};
    }
}

// Transpose the 8x8 block in registers (reg[p] holds r = p, o = 0..7) and
// store row o = 8(t&31)+e of the LDS tile with its 8 r values (chunk t>>5).
__device__ __forceinline__ void store_oc(char *lds, const u32x4_t (&reg)[8], int t) {
    const int oc = t & 31;
    const int rb = t >> 5;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int q = e >> 1;
        u32x4_t out;
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            const uint32_t lo = reg[2 * h][q];     // r = 2h
            const uint32_t hi = reg[2 * h + 1][q]; // r = 2h + 1
            out[h] = (e & 1) ? ((lo >> 16) | (hi & 0xffff0000u))
                             : ((lo & 0xffffu) | (hi << 16));
        }
        *reinterpret_cast<u32x4_t *>(lds + lds_off(8 * oc + e, rb)) = out;
    }
}

// One 64-deep slab: 4 MFMA k-steps of 16 over the wave's 4x4 grid of 32x32 blocks.
// MFMA operand roles are swapped (src A = the j-side tile) so that each lane's
// accumulators hold 4 consecutive output columns of one output row.
__device__ __forceinline__ void mma_slab(const char *la, const char *lb, f32x16_t (&acc)[4][4],
                                         int wm, int wn, int lane) {
    const int rl = lane & 31;
    const int half = lane >> 5;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        bf16x8_t af[4], bf[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            af[x] = *reinterpret_cast<const bf16x8_t *>(la + lds_off(wm * 128 + x * 32 + rl, 2 * s + half));
            bf[x] = *reinterpret_cast<const bf16x8_t *>(lb + lds_off(wn * 128 + x * 32 + rl, 2 * s + half));
        }
#pragma unroll
        for (int x = 0; x < 4; ++x)
#pragma unroll
            for (int y = 0; y < 4; ++y)
                acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[y], af[x], acc[x][y], 0, 0, 0);
    }
}

// Tile index within a job -> (ti, tj).  Consecutive block ids land on
// different XCDs (round-robin dispatch), so first gather each XCD's blocks
// into one contiguous range of tiles, then raster that range in groups of
// kGroupI tile rows so concurrently running tiles share operand panels in L2.
__device__ __forceinline__ void tile_coords(const TileJob &jb, int t, int &ti, int &tj) {
    int u = t;
    if ((jb.ntiles & 7) == 0)
        u = (t & 7) * (jb.ntiles >> 3) + (t >> 3);
    const int per_group = kGroupI * jb.tiles_j;
    const int group = u / per_group;
    const int first_i = group * kGroupI;
    const int rows = min(jb.tiles_i - first_i, kGroupI);
    const int in_group = u - group * per_group;
    ti = first_i + in_group % rows;
    tj = in_group / rows;
}

template <int KIND>
__device__ __forceinline__ void run_tile(const TileJob &jb, int t_index, char *smem) {
    int ti, tj;
    tile_coords(jb, t_index, ti, tj);
    const int64_t i0 = (int64_t)ti * kTile;
    const int64_t j0 = (int64_t)tj * kTile;
    const int t = threadIdx.x;
    const int lane = t & 63;
    const int w = t >> 6;
    const int wm = w >> 1, wn = w & 1;

    f32x16_t acc[4][4];
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y)
            acc[x][y] = f32x16_t{};

    const int nslab = (int)((jb.R + kBK - 1) / kBK);
    u32x4_t ra[8], rb[8];
    auto load = [&](int64_t r0) {
        if (KIND == JOB_DX) {
            load_rc(ra, jb.a, jb.lda, jb.I, jb.R, i0, r0, t);
            load_rc(rb, jb.b, jb.ldb, jb.J, jb.R, j0, r0, t);
        } else {
            load_oc(ra, jb.a, jb.lda, jb.I, jb.R, i0, r0, t);
            load_oc(rb, jb.b, jb.ldb, jb.J, jb.R, j0, r0, t);
        }
    };
    auto store = [&](char *stage) {
        if (KIND == JOB_DX) {
            store_rc(stage, ra, t);
            store_rc(stage + kOperandBytes, rb, t);
        } else {
            store_oc(stage, ra, t);
            store_oc(stage + kOperandBytes, rb, t);
        }
    };

    if (nslab > 0) {
        load(0);
        store(smem);
        __syncthreads();
    }
    for (int s = 0; s < nslab; ++s) {
        char *cur = smem + (s & 1) * kStageBytes;
        char *nxt = smem + ((s + 1) & 1) * kStageBytes;
        const bool more = s + 1 < nslab;
        if (more)
            load((int64_t)(s + 1) * kBK); // global loads in flight during the MFMAs
        mma_slab(cur, cur + kOperandBytes, acc, wm, wn, lane);
        if (more)
            store(nxt);
        __syncthreads();
    }

    // Epilogue: lane holds C[i][j..j+3] for i = .. + (lane&31), j = .. + 8g + 4(lane>>5).
    const int64_t ib = i0 + wm * 128 + (lane & 31);
    const int64_t jb0 = j0 + wn * 128 + 4 * (lane >> 5);
#pragma unroll
    for (int x = 0; x < 4; ++x) {
        const int64_t i = ib + x * 32;
        if (i >= jb.I)
            continue;
#pragma unroll
        for (int y = 0; y < 4; ++y)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int64_t j = jb0 + y * 32 + 8 * g;
                if (j >= jb.J)
                    continue; // J % 8 == 0: j..j+3 all in range
                const f32x16_t &a = acc[x][y];
                if (KIND == JOB_DX) {
                    u32x2_t pk = {pack_bf16x2(a[4 * g], a[4 * g + 1]),
                                  pack_bf16x2(a[4 * g + 2], a[4 * g + 3])};
                    *reinterpret_cast<u32x2_t *>(static_cast<uint16_t *>(jb.c) + i * jb.J + j) = pk;
                } else {
                    f32x4_t v = {a[4 * g], a[4 * g + 1], a[4 * g + 2], a[4 * g + 3]};
                    *reinterpret_cast<f32x4_t *>(static_cast<float *>(jb.c) + i * jb.J + j) = v;
                }
            }
    }
}

__global__ __launch_bounds__(kThreads, 1) void k_lin_bwd_mfma(MfmaParams p) {
    __shared__ __attribute__((aligned(16))) char smem[kLdsBytes];
    int b = blockIdx.x;
    const TileJob *jb = &p.job[0];
    if (b >= p.job[0].ntiles) {
        b -= p.job[0].ntiles;
        jb = &p.job[1];
    }
    if (jb->kind == JOB_DX)
        run_tile<JOB_DX>(*jb, b, smem);
    else
        run_tile<JOB_DW>(*jb, b, smem);
}

// ------------------------------------------------------------------------
// small-M dX: dX[m,k] = Σ_n dY[m,n]·W[k,n] for M <= 64
// ------------------------------------------------------------------------
constexpr int kSmallWaves = 8;
constexpr int kSmallUnroll = 8;
constexpr int kSmallMaxM = 64;

// Block: 16 output columns k (one 16x16x32 MFMA column block), all M rows
// (up to 4 blocks of 16).  Wave w reduces n over its own contiguous range;
// the per-wave partials are summed in LDS in a fixed order.
__global__ __launch_bounds__(kSmallWaves * 64) void k_dx_smallm(const uint16_t *__restrict__ G,
                                                                 const uint16_t *__restrict__ W,
                                                                 uint16_t *__restrict__ dX,
                                                                 int64_t M, int64_t K, int64_t N) {
    __shared__ f32x4_t red[kSmallWaves][4][64];
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int64_t k0 = (int64_t)blockIdx.x * 16;
    const int mb_count = (int)((M + 15) / 16);

    // wave's reduction range, in units of 32
    const int64_t steps = (N + 31) / 32;
    const int64_t per_wave = (steps + kSmallWaves - 1) / kSmallWaves;
    const int64_t s_beg = w * per_wave;
    const int64_t s_end = min(steps, s_beg + per_wave);

    const int64_t krow = k0 + (lane & 15);
    const bool kok = krow < K;
    const int sub = 8 * (lane >> 4); // this lane's 8 reduction elements within a step of 32
    const uint16_t *wrow = W + krow * N + sub;

    f32x4_t acc[4] = {f32x4_t{}, f32x4_t{}, f32x4_t{}, f32x4_t{}};
    for (int64_t s = s_beg; s < s_end; s += kSmallUnroll) {
        bf16x8_t wf[kSmallUnroll];
        bf16x8_t gf[kSmallUnroll][4];
#pragma unroll
        for (int u = 0; u < kSmallUnroll; ++u) {
            const int64_t n = (s + u) * 32 + sub;
            const bool nok = (s + u) < s_end && n < N; // N % 8 == 0
            wf[u] = (nok && kok) ? *reinterpret_cast<const bf16x8_t *>(wrow + (s + u) * 32)
                                 : bf16x8_t{};
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) {
                const int64_t m = mb * 16 + (lane & 15);
                gf[u][mb] = (mb < mb_count && nok && m < M)
                                ? *reinterpret_cast<const bf16x8_t *>(G + m * N + n)
                                : bf16x8_t{};
            }
        }
#pragma unroll
        for (int u = 0; u < kSmallUnroll; ++u)
#pragma unroll
            for (int mb = 0; mb < 4; ++mb)
                if (mb < mb_count)
                    acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[u], gf[u][mb], acc[mb], 0, 0, 0);
    }
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
        red[w][mb][lane] = acc[mb];
    __syncthreads();
    // wave mb sums the partials of m-block mb; lane holds dX[m][k..k+3]
    if (w < mb_count) {
        f32x4_t s = red[0][w][lane];
        for (int ww = 1; ww < kSmallWaves; ++ww)
            s += red[ww][w][lane];
        const int64_t m = w * 16 + (lane & 15);
        const int64_t k = k0 + 4 * (lane >> 4);
        if (m < M && k < K) { // K % 8 == 0: k..k+3 in range
            u32x2_t pk = {pack_bf16x2(s[0], s[1]), pack_bf16x2(s[2], s[3])};
            *reinterpret_cast<u32x2_t *>(dX + m * K + k) = pk;
        }
    }
}

// ------------------------------------------------------------------------
// SIMT fallback: any alignment, any sizes; fp32 or bf16 operands.
// ------------------------------------------------------------------------
struct SimtJob {
    const void *a;
    const void *b;
    void *c;
    int64_t I, J, R;
    int64_t sai, sar, sbj, sbr; // A(i,r) = a[i*sai + r*sar], B(j,r) = b[j*sbj + r*sbr]
    bool c_bf16;
};
struct SimtParams {
    SimtJob job[2];
    int njobs;
};

template <bool BF16>
__device__ __forceinline__ float ld_elem(const void *p, int64_t idx) {
    if (BF16)
        return bf16_bits_to_f32(static_cast<const uint16_t *>(p)[idx]);
    return static_cast<const float *>(p)[idx];
}

constexpr int kSimtTile = 64;
constexpr int kSimtBK = 16;

template <bool BF16>
__global__ __launch_bounds__(256) void k_lin_bwd_simt(SimtParams p) {
    const SimtJob &jb = p.job[blockIdx.z];
    const int64_t i0 = (int64_t)blockIdx.y * kSimtTile;
    const int64_t j0 = (int64_t)blockIdx.x * kSimtTile;
    if (i0 >= jb.I || j0 >= jb.J)
        return;
    __shared__ float As[kSimtBK][kSimtTile + 1];
    __shared__ float Bs[kSimtBK][kSimtTile + 1];
    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
    float acc[4][4] = {};
    for (int64_t r0 = 0; r0 < jb.R; r0 += kSimtBK) {
        for (int e = threadIdx.x; e < kSimtBK * kSimtTile; e += 256) {
            const int rr = e / kSimtTile, oo = e % kSimtTile;
            const int64_t r = r0 + rr;
            const int64_t i = i0 + oo, j = j0 + oo;
            As[rr][oo] = (r < jb.R && i < jb.I) ? ld_elem<BF16>(jb.a, i * jb.sai + r * jb.sar) : 0.0f;
            Bs[rr][oo] = (r < jb.R && j < jb.J) ? ld_elem<BF16>(jb.b, j * jb.sbj + r * jb.sbr) : 0.0f;
        }
        __syncthreads();
        for (int rr = 0; rr < kSimtBK; ++rr)
            for (int x = 0; x < 4; ++x)
                for (int y = 0; y < 4; ++y)
                    acc[x][y] += As[rr][ty + 16 * x] * Bs[rr][tx + 16 * y];
        __syncthreads();
    }
    for (int x = 0; x < 4; ++x)
        for (int y = 0; y < 4; ++y) {
            const int64_t i = i0 + ty + 16 * x, j = j0 + tx + 16 * y;
            if (i < jb.I && j < jb.J) {
                if (jb.c_bf16)
                    static_cast<uint16_t *>(jb.c)[i * jb.J + j] = f32_to_bf16_bits(acc[x][y]);
                else
                    static_cast<float *>(jb.c)[i * jb.J + j] = acc[x][y];
            }
        }
}

// ------------------------------------------------------------------------
// host-side dispatch
// ------------------------------------------------------------------------
inline bool is_aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int ceil_div(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

TileJob make_tile_job(int kind, const void *a, const void *b, void *c, int64_t I, int64_t J,
                      int64_t R, int64_t lda, int64_t ldb) {
    TileJob j;
    j.a = static_cast<const uint16_t *>(a);
    j.b = static_cast<const uint16_t *>(b);
    j.c = c;
    j.I = I;
    j.J = J;
    j.R = R;
    j.lda = lda;
    j.ldb = ldb;
    j.tiles_i = ceil_div(I, kTile);
    j.tiles_j = ceil_div(J, kTile);
    j.ntiles = j.tiles_i * j.tiles_j;
    j.kind = kind;
    return j;
}

hipError_t launch_simt(const LinBwdArgs &a, bool need_dx, bool need_dw, hipStream_t s) {
    SimtParams p{};
    int nj = 0;
    int64_t maxI = 0, maxJ = 0;
    if (need_dx) { // dX[m,k] = Σ_n dY[m,n] W[k,n]
        SimtJob &j = p.job[nj++];
        j = SimtJob{a.dY, a.W, a.dX, a.M, a.K, a.N, a.N, 1, a.N, 1, a.bf16};
        maxI = std::max(maxI, a.M);
        maxJ = std::max(maxJ, a.K);
    }
    if (need_dw) { // dW[k,n] = Σ_m X[m,k] dY[m,n]
        SimtJob &j = p.job[nj++];
        j = SimtJob{a.X, a.dY, a.dW, a.K, a.N, a.M, 1, a.K, 1, a.N, false};
        maxI = std::max(maxI, a.K);
        maxJ = std::max(maxJ, a.N);
    }
    p.njobs = nj;
    dim3 grid((unsigned)ceil_div(maxJ, kSimtTile), (unsigned)ceil_div(maxI, kSimtTile), (unsigned)nj);
    if (grid.y > 65535u)
        return hipErrorInvalidConfiguration;
    if (a.bf16)
        hipLaunchKernelGGL(k_lin_bwd_simt<true>, grid, dim3(256), 0, s, p);
    else
        hipLaunchKernelGGL(k_lin_bwd_simt<false>, grid, dim3(256), 0, s, p);
    return hipGetLastError();
}

} // namespace

hipError_t launch_lin_bwd(const LinBwdArgs &a, hipStream_t s) {
    const bool need_dx = a.dX != nullptr && a.M > 0 && a.K > 0;
    const bool need_dw = a.dW != nullptr && a.K > 0 && a.N > 0;
    if (!need_dx && !need_dw)
        return hipSuccess;

    bool vec = a.bf16 && (a.K % 8 == 0) && (a.N % 8 == 0);
    if (need_dx)
        vec = vec && is_aligned16(a.dX) && (a.N == 0 || (is_aligned16(a.dY) && is_aligned16(a.W)));
    if (need_dw)
        vec = vec && is_aligned16(a.dW) && (a.M == 0 || (is_aligned16(a.X) && is_aligned16(a.dY)));
    if (!vec)
        return launch_simt(a, need_dx, need_dw, s);

    const bool small_dx = need_dx && a.M <= kSmallMaxM && a.N > 0;
    MfmaParams p{};
    int nj = 0;
    TileJob jx{}, jw{};
    bool have_x = false, have_w = false;
    if (need_dx && !small_dx) {
        jx = make_tile_job(JOB_DX, a.dY, a.W, a.dX, a.M, a.K, a.N, a.N, a.N);
        have_x = true;
    }
    if (need_dw) {
        jw = make_tile_job(JOB_DW, a.X, a.dY, a.dW, a.K, a.N, a.M, a.K, a.N);
        have_w = true;
    }
    // longest reduction first: those tiles start on the first wave of CUs
    if (have_x && have_w) {
        if (jw.R > jx.R) {
            p.job[nj++] = jw;
            p.job[nj++] = jx;
        } else {
            p.job[nj++] = jx;
            p.job[nj++] = jw;
        }
    } else if (have_x) {
        p.job[nj++] = jx;
    } else if (have_w) {
        p.job[nj++] = jw;
    }
    p.njobs = nj;
    if (nj > 0) {
        const int64_t blocks = (int64_t)p.job[0].ntiles + (nj > 1 ? p.job[1].ntiles : 0);
        if (blocks > 0x7fffffff)
            return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL(k_lin_bwd_mfma, dim3((unsigned)blocks), dim3(kThreads), 0, s, p);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    if (small_dx) {
        hipLaunchKernelGGL(k_dx_smallm, dim3((unsigned)ceil_div(a.K, 16)), dim3(kSmallWaves * 64), 0, s,
                           static_cast<const uint16_t *>(a.dY), static_cast<const uint16_t *>(a.W),
                           static_cast<uint16_t *>(a.dX), a.M, a.K, a.N);
        return hipGetLastError();
    }
    return hipSuccess;
}

} // namespace lb
