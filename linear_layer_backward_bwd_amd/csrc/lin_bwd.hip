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
#include <type_traits>

namespace lb {
namespace {

// ------------------------------------------------------------------------
// MFMA tile kernel
// ------------------------------------------------------------------------
constexpr int kTile = 256;                        // output tile edge (i and j)
constexpr int kBK = 64;                           // reduction slab per stage
constexpr int kThreads = 256;                     // 4 waves, 2x2, 128x128 each
constexpr int kOperandBytes = kTile * kBK * 2;    // one operand slab in LDS: 32 KiB
constexpr int kStageBytes = 2 * kOperandBytes;    // A and B
constexpr int kLdsBytes = 2 * kStageBytes;        // double buffered: 128 KiB
constexpr int kGroupI = 4;                        // tile rows per raster group
constexpr uint32_t kOOB = 0x80000000u;            // buffer offset past num_records: reads 0

#define LDS __attribute__((address_space(3)))
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));

// Operand slabs live in LDS in one of two layouts, both written by
// global->LDS DMA (buffer_load_dwordx4 ... lds: lane l of a wave
// instruction writes 16 bytes at M0 + 16*l, so one instruction fills 1 KiB).
// The XOR swizzles are applied by choosing which global chunk each lane
// fetches; the LDS side is always contiguous.
//
//  RC ("reduction contiguous", dX operands dY and W): 256 rows (output index)
//     x 64 r, 128 B per row; 16-byte chunk c of row `row` is stored at
//     chunk c ^ swz_rc(row).  MFMA fragment = one ds_read_b128 (8 r values).
//  OC ("outer contiguous", dW operands X and dY): 64 rows (r) x 256 outer
//     indices, 512 B per row; chunk c of row r is stored at chunk
//     c ^ swz_oc(r).  MFMA fragment = two ds_read_b64_tr_b16: within each
//     16-lane group the instruction reads a 4-row x 16-column block (each
//     lane addresses 4 columns of one row) and hands lane i column i, so a
//     lane receives 4 consecutive r of its own outer index.
__device__ __forceinline__ int swz_rc(int row) { return (row & 7) ^ ((row >> 3) & 7); }
__device__ __forceinline__ int swz_oc(int row) { return 2 * (row & 3); }
__device__ __forceinline__ int rc_off(int row, int chunk) { return row * 128 + ((chunk ^ swz_rc(row)) << 4); }

enum JobKind { JOB_DX = 0, JOB_DW = 1 };

struct TileJob {
    const uint16_t *a; // operand giving output rows i
    const uint16_t *b; // operand giving output cols j
    void *c;           // output, row-major [I, J], leading dim J
    int64_t I, J, R;   // output rows, cols, reduction length
    int64_t lda, ldb;  // leading dims of a and b in elements
    uint32_t a_bytes, b_bytes; // operand sizes (each < 2 GiB on this path)
    int tiles_i, tiles_j, ntiles;
    int kind;          // JOB_DX: RC operands, bf16 out; JOB_DW: OC operands, fp32 out
};

struct MfmaParams {
    TileJob job[2];
    int njobs;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes) {
    // raw buffer: stride 0, num_records in bytes, gfx9 data-format word
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rs, LDS char *dst, uint32_t off) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LDS void *)dst, 16, (int)off, 0, 0, 0);
}

// RC slab: element (o, r) at base[o*ld + r].  Wave w, instruction p fills LDS
// rows 8(8w+p) .. +7; lane -> row (lane>>3), physical chunk (lane&7).
template <int P0, int NP>
__device__ __forceinline__ void dma_rc(__amdgpu_buffer_rsrc_t rs, LDS char *op, int64_t ld, int64_t O,
                                       int64_t R, int64_t o0, int64_t r0, int w, int lane) {
#pragma unroll
    for (int p = P0; p < P0 + NP; ++p) {
        const int row = (w * 8 + p) * 8 + (lane >> 3);
        const int lc = (lane & 7) ^ swz_rc(row);
        const int64_t o = o0 + row;
        const int64_t r = r0 + 8 * lc;
        const uint32_t off = (o < O && r < R) ? (uint32_t)((o * ld + r) * 2) : kOOB;
        dma16(rs, op + (w * 8 + p) * 1024, off);
    }
}

// OC slab: element (r, o) at base[r*ld + o].  Wave w, instruction p fills LDS
// rows 2(8w+p), +1; lane -> row (lane>>5), physical chunk (lane&31).
template <int P0, int NP>
__device__ __forceinline__ void dma_oc(__amdgpu_buffer_rsrc_t rs, LDS char *op, int64_t ld, int64_t O,
                                       int64_t R, int64_t r0, int64_t o0, int w, int lane) {
#pragma unroll
    for (int p = P0; p < P0 + NP; ++p) {
        const int row = (w * 8 + p) * 2 + (lane >> 5);
        const int lc = (lane & 31) ^ swz_oc(row);
        const int64_t r = r0 + row;
        const int64_t o = o0 + 8 * lc;
        const uint32_t off = (o < O && r < R) ? (uint32_t)((r * ld + o) * 2) : kOOB;
        dma16(rs, op + (w * 8 + p) * 1024, off);
    }
}

// MFMA fragment (8 consecutive r of outer index `ob + (lane&31)`, r half
// chosen by lane>>5) for k-step ks of the slab.
__device__ __forceinline__ bf16x8_t frag_rc(const LDS char *op, int ob, int ks, int lane) {
    const int row = ob + (lane & 31);
    return *reinterpret_cast<const LDS bf16x8_t *>(op + rc_off(row, 2 * ks + (lane >> 5)));
}

__device__ __forceinline__ bf16x8_t frag_oc(const LDS char *op, int ob, int ks, int lane) {
    const int g = lane >> 4, s = lane & 15;
    const int row = ks * 16 + 8 * (g >> 1) + (s >> 2);
    const int col = ob + 16 * (g & 1) + 4 * (s & 3);
    const int lc = col >> 3;
    const int a0 = row * 512 + ((lc ^ swz_oc(row)) << 4) + (col & 7) * 2;
    const int a1 = (row + 4) * 512 + ((lc ^ swz_oc(row + 4)) << 4) + (col & 7) * 2;
    // Issued as inline asm: the compiler's wait insertion treats the builtin as
    // aliasing the in-flight DMA into the other stage buffer and would stall on
    // it.  The caller waits for these reads with lgkm_wait() before use.
    bf16x4_t lo, hi;
    asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(lo) : "v"(op + a0));
    asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(hi) : "v"(op + a1));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Wait for all of this wave's LDS reads; the fragments are threaded through the
// asm so no MFMA that consumes them can be scheduled above the wait.
__device__ __forceinline__ void lgkm_wait(bf16x8_t (&a)[4], bf16x8_t (&b)[4]) {
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(b[0]), "+v"(b[1]), "+v"(b[2]),
                   "+v"(b[3])
                 :
                 : "memory");
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
__device__ __forceinline__ void run_tile(const TileJob &jb, int t_index, LDS char *smem) {
    int ti, tj;
    tile_coords(jb, t_index, ti, tj);
    const int64_t i0 = (int64_t)ti * kTile;
    const int64_t j0 = (int64_t)tj * kTile;
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int wm = w >> 1, wn = w & 1;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(jb.a, jb.a_bytes);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(jb.b, jb.b_bytes);

    f32x16_t acc[4][4];
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y)
            acc[x][y] = f32x16_t{};

    // DMA of slab s into its stage buffer, instructions [P0, P0+NP) of each operand
    auto issue = [&](int s, auto p0, auto np) {
        constexpr int P0 = decltype(p0)::value, NP = decltype(np)::value;
        LDS char *st = smem + (s & 1) * kStageBytes;
        const int64_t r0 = (int64_t)s * kBK;
        if (KIND == JOB_DX) {
            dma_rc<P0, NP>(ra, st, jb.lda, jb.I, jb.R, i0, r0, w, lane);
            dma_rc<P0, NP>(rb, st + kOperandBytes, jb.ldb, jb.J, jb.R, j0, r0, w, lane);
        } else {
            dma_oc<P0, NP>(ra, st, jb.lda, jb.I, jb.R, r0, i0, w, lane);
            dma_oc<P0, NP>(rb, st + kOperandBytes, jb.ldb, jb.J, jb.R, r0, j0, w, lane);
        }
    };
    auto frag = [&](const LDS char *op, int ob, int ks) {
        return KIND == JOB_DX ? frag_rc(op, ob, ks, lane) : frag_oc(op, ob, ks, lane);
    };
    using C0 = std::integral_constant<int, 0>;
    using C2 = std::integral_constant<int, 2>;
    using C8 = std::integral_constant<int, 8>;
    // LDS reads per fragment: one b128 (RC) or two transposing b64 (OC)
    constexpr int kReadsPerFrag = KIND == JOB_DX ? 1 : 2;

    const int nslab = (int)((jb.R + kBK - 1) / kBK);
    if (nslab > 0)
        issue(0, C0{}, C8{});
    for (int s = 0; s < nslab; ++s) {
        // this wave's DMA of slab s has landed; after the barrier, everyone's has,
        // and every wave is done reading the buffer that slab s+1 will fill
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        const bool more = s + 1 < nslab;
        const LDS char *la = smem + (s & 1) * kStageBytes;
        const LDS char *lb = la + kOperandBytes;
        bf16x8_t af[4], bf[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            af[x] = frag(la, wm * 128 + x * 32, 0);
            bf[x] = frag(lb, wn * 128 + x * 32, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            // one scheduling region per k-step: the next step's fragment reads and a
            // quarter of the next slab's DMA are interleaved with this step's 16 MFMAs
            if (KIND == JOB_DW)
                lgkm_wait(af, bf); // the asm transposing reads of this step's fragments
            bf16x8_t an[4], bn[4];
            if (ks + 1 < 4) {
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    an[x] = frag(la, wm * 128 + x * 32, ks + 1);
                    bn[x] = frag(lb, wn * 128 + x * 32, ks + 1);
                }
            }
            if (more) {
                if (ks == 0) issue(s + 1, std::integral_constant<int, 0>{}, C2{});
                if (ks == 1) issue(s + 1, std::integral_constant<int, 2>{}, C2{});
                if (ks == 2) issue(s + 1, std::integral_constant<int, 4>{}, C2{});
                if (ks == 3) issue(s + 1, std::integral_constant<int, 6>{}, C2{});
            }
#pragma unroll
            for (int x = 0; x < 4; ++x)
#pragma unroll
                for (int y = 0; y < 4; ++y)
                    acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[y], af[x], acc[x][y], 0, 0, 0);
            if (ks + 1 < 4) {
                // 8 fragments = 8 (RC) or 16 (OC) LDS reads spread over the 16 MFMAs
#pragma unroll
                for (int i = 0; i < 8 * kReadsPerFrag; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 16 / (8 * kReadsPerFrag), 0); // MFMA
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                        // DS read
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            if (ks + 1 < 4) {
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    af[x] = an[x];
                    bf[x] = bn[x];
                }
            }
        }
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
    __shared__ __attribute__((aligned(1024))) char smem_raw[kLdsBytes];
    LDS char *smem = (LDS char *)smem_raw;
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
    // RC operands have I (resp. J) rows of ld elements; OC operands have R rows
    const int64_t a_rows = kind == JOB_DX ? I : R;
    const int64_t b_rows = kind == JOB_DX ? J : R;
    j.a_bytes = (uint32_t)(a_rows * lda * 2);
    j.b_bytes = (uint32_t)(b_rows * ldb * 2);
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

    // buffer offsets are 32-bit with 2^31 marking "out of range": each operand
    // of the MFMA path must be smaller than 2 GiB
    const int64_t lim = (int64_t)1 << 31;
    if (2 * a.M * a.K >= lim || 2 * a.K * a.N >= lim || 2 * a.M * a.N >= lim)
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
