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
//   k_lin_bwd_mfma   bf16 MFMA (v_mfma_f32_16x16x32_bf16, fp32 accumulate), 256x256
//                    output tile per 4-wave workgroup (128x128 per wave).  The reduction
//                    runs in slabs of 32 that global->LDS DMA streams into a 4-slot,
//                    XOR-swizzled LDS ring three slabs ahead of the MFMAs; one barrier
//                    per slab.  For dX both operands are reduction-contiguous rows (one
//                    16-byte LDS read per fragment); for dW the reduction index is the
//                    slow index of both operands, and the transposing LDS read
//                    (ds_read_b64_tr_b16) turns the row-major slab into MFMA fragments.
//                    One launch runs the tiles of both products; blocks are ordered
//                    longest reduction first and mapped so that each XCD works on a
//                    compact group of tiles.
//   k_lin_bwd_mfma_split  the same with dX's reduction split into ranges whose
//                    tiles write fp32 partials (where few, long dX tiles would
//                    outlast the launch: M from 257, or 160 with both products and
//                    K, N >= 2048, up to 2048); k_dx_smallm_reduce adds them.
//   k_dx_smallm      dX for M <= 256 (decode-like and small batches; up to 1024
//                    on request): streams W once per 256-row group, the reduction
//                    over n split across blocks; the fp32 partials are added in
//                    split order by the first blocks of k_dw_smallm (M <= 256),
//                    else by k_dx_smallm_reduce.
//   k_dw_smallm      dW for M <= 256: bound by writing the fp32 output at small M;
//                    small tiles, several per CU, so stores overlap other tiles' loads.
//   k_smallm_pair    the blocks of both in one launch, two per CU (M <= 64, N and
//                    K*N not too large), so W's read stream and dW's write stream
//                    overlap; the dX partials are then added by k_dx_smallm_reduce.
//   k_dx_rows16, k_smallm_pair16  the same for M <= 16 on small calls, with dX
//                    blocks that each sum a whole reduction: no partials and no
//                    summing launch.
//   k_lin_bwd_fused_small  both products for M <= 64 in one launch (on request).
//   k_repack         zero-padded copies for bf16 calls whose K or N is not a
//                    multiple of 8 or whose pointers are not 16-byte aligned.
//   k_lin_bwd_simt   any dtype / alignment / shape: the fp32 path.
#include "device.h"
#include "dispatch.h"
#include "kernels.h"

#include <algorithm>
#include <type_traits>

namespace lb {
namespace {

// ------------------------------------------------------------------------
// MFMA tile kernel
// ------------------------------------------------------------------------
constexpr int kTile = 256;                        // output tile edge (i and j)
constexpr int kBK = 32;                           // reduction slab per stage
constexpr int kStages = 4;                        // LDS ring: 3 slabs in flight
constexpr int kThreads = 256;                     // 4 waves, 2x2, 128x128 each
constexpr int kOperandBytes = kTile * kBK * 2;    // one operand slab in LDS: 16 KiB
constexpr int kStageBytes = 2 * kOperandBytes;    // A and B
constexpr int kBOffset = kStages * kOperandBytes;  // all A slabs first, then all B slabs
constexpr int kLdsBytes = kStages * kStageBytes;  // 128 KiB
constexpr int kDmaPerOp = kBK / 8;                // DMA instructions per wave per operand per slab
constexpr int kGroupI = 4;                        // tile rows per raster group
constexpr int kGroupIRot = 2;                     // ... for a job whose reduction starts are rotated
constexpr int kCUs = 256;                         // compute units of the part (8 XCDs x 32)
constexpr uint32_t kOOB = 0x80000000u;            // buffer offset past num_records: reads 0

#define LDS __attribute__((address_space(3)))
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));

// Operand slabs live in LDS in one of two layouts, both written by
// global->LDS DMA (buffer_load_dwordx4 ... lds: lane l of a wave
// instruction writes 16 bytes at M0 + 16*l, so one instruction fills 1 KiB).
// The XOR swizzles are applied by choosing which global chunk each lane
// fetches; the LDS side is always contiguous.  Both are free of bank
// conflicts for the fragment reads, as measured with the LDS bank-conflict
// counter on in-bounds probes of the exact read patterns.
//
//  RC ("reduction contiguous", dX operands dY and W): slab pairs, described
//     with the dX pipeline below.
//  OC ("outer contiguous", dW operands X and dY): 32 rows (r) x 256 outer
//     indices, 512 B per row; chunk c of row r is stored at chunk
//     c ^ swz_oc(r).  MFMA fragment = two ds_read_b64_tr_b16: within each
//     16-lane group the instruction reads a 4-row x 16-column block (each
//     lane addresses 4 columns of one row) and hands lane i column i, so a
//     lane receives 4 consecutive r of its own outer index.
static_assert(kBK == 32, "an RC slab pair is one 128-byte line per row");
__device__ __forceinline__ int swz_oc(int row) {
    // 32-byte segment s of row r moves to s ^ ((r & 3) | 4*((r >> 3) & 1)): the
    // rows r..r+3 and r+8..r+11 that one 32-lane read touches land on eight
    // different segments (chunk pairs stay together)
    return 2 * ((row & 3) | (((row >> 3) & 1) << 2));
}

enum JobKind { JOB_DX = 0, JOB_DW = 1 };

struct TileJob {
    const uint16_t *a; // operand giving output rows i
    const uint16_t *b; // operand giving output cols j
    void *c;           // output, row-major [I, J], leading dim J
    int64_t I, J, R;   // output rows, cols, reduction length
    int64_t lda, ldb;  // leading dims of a and b in elements
    int tiles_i, tiles_j, ntiles; // ntiles = tiles_i * tiles_j * splits
    int kind;          // JOB_DX: RC operands, bf16 out; JOB_DW: OC operands, fp32 out
    // k rotation (slabs), dX (RC) jobs only: the tile at (ti, tj) walks the
    // slabs starting at rot * ((tj / 2) % 4) mod nslab (0 for a ragged
    // reduction)
    int rot;
    // dX jobs only: the reduction split into `splits` ranges of split_len
    // elements (a whole number of 64-element pairs; the last range may be
    // shorter); with splits > 1 the tiles of range s write fp32 partial sums
    // to part + s*I*J, which a later launch adds in range order, instead of
    // bf16 sums to c
    int splits;
    int64_t split_len;
    float *part;
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
// The same for data read once: the non-temporal cache policy (aux bit 1).
__device__ __forceinline__ void dma16_nt(__amdgpu_buffer_rsrc_t rs, LDS char *dst, uint32_t off) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LDS void *)dst, 16, (int)off, 0, 0, 2);
}

// A buffer offset (below 2^31) marked out of range when !ok: bit 31 set puts
// it past any descriptor size used here.  Written as arithmetic, not a
// select, so the compiler emits no branch around the memory instruction (a
// branch would skip a zero-filling DMA, or duplicate a store).
__device__ __forceinline__ uint32_t oob_unless(bool ok, uint32_t off) {
    return off | ((uint32_t)!ok << 31);
}

// Output stores (never re-read by the kernel that writes them): 16 bytes
// through a buffer descriptor, so that out-of-range lanes are dropped by the
// hardware without a branch, non-temporal.  (A store-only probe wrote 64 MiB
// faster with the sc1 policy than non-temporal, 10.2 vs 11.1 us, but in the
// kernels sc1 was slower: M = 2048 123.7 vs 119.1 us, the block's projections
// 1390 vs 1413 TFLOP/s, M = 32 24.3 vs 22.7 us, A/B in one process.)
#ifndef LB_OUT_AUX
#define LB_OUT_AUX 2 // nt
#endif
template <typename T>
__device__ __forceinline__ void store_out(__amdgpu_buffer_rsrc_t rs, uint32_t off, const T &v) {
    static_assert(sizeof(T) == 16, "16-byte stores");
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), rs, (int)off, 0, LB_OUT_AUX);
}

// Per-lane DMA source offsets of an OC slab, fixed for a tile.  Instruction p
// of wave w fills LDS rows 2q, 2q+1 (r) of the slab, q = kDmaPerOp*w + p: lane
// l takes physical chunk l&31 of row 2q + l/32, i.e. outer chunk
// (l&31) ^ swz_oc(row).  Offset (row*ld + o)*2 relative to the slab's first
// row; outer chunks outside the operand get kOOB.
__device__ __forceinline__ uint32_t dma_oc_off(int p, int64_t ld, int64_t O, int64_t o0, int w, int lane) {
    const int q = w * kDmaPerOp + p;
    const int row = q * 2 + (lane >> 5);
    const int lc = (lane & 31) ^ swz_oc(row);
    const int64_t o = o0 + 8 * lc;
    return o < O ? (uint32_t)((row * ld + o) * 2) : kOOB;
}

// Per-lane LDS byte offsets (within an OC slab) of the fragment for the 16
// outer indices ob..ob+15, all 32 r of the slab: lane l holds outer index
// ob + l%16 and r = 8*(l/16) .. +7 (the operand layout of a 16x16x32 MFMA),
// read as two ds_read_b64_tr_b16 (half h = r 4h..4h+3 of each 8): each
// 16-lane group reads a 4-row x 16-column block.
__device__ __forceinline__ int frag_off_oc(int ob, int lane, int half) {
    const int g = lane >> 4, s = lane & 15;
    const int row = 8 * g + 4 * half + (s >> 2);
    const int col = ob + 4 * (s & 3);
    const int lc = col >> 3;
    return row * 512 + ((lc ^ swz_oc(row)) << 4) + (col & 7) * 2;
}

// LDS fragment reads are issued as inline asm: the compiler's wait insertion
// treats them as aliasing the in-flight DMA into other stage buffers and would
// stall on it, or would place a wait before every MFMA.  Callers wait for these
// reads with lgkm_wait() before use.
template <int OFF>
__device__ __forceinline__ bf16x8_t read_rc(const LDS char *p) {
    static_assert(OFF >= 0 && OFF < 65536, "ds offset is 16 bits");
    bf16x8_t v;
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(p), "n"(OFF));
    return v;
}
template <int OFF>
__device__ __forceinline__ bf16x4_t read_tr(const LDS char *p) {
    static_assert(OFF >= 0 && OFF < 65536, "ds offset is 16 bits");
    bf16x4_t v;
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(v) : "v"(p), "n"(OFF));
    return v;
}

constexpr int kFrags = 8; // fragments per operand per wave (128 outer indices / 16)

// acc += A·B on a 16x16x32 block.  Written as inline asm so the 64
// accumulators of a wave stay in AGPRs: with the builtin the register
// allocator splits them between register files and shuffles them inside the
// main loop.  The accumulators are only read after mfma_drain().
__device__ __forceinline__ void mfma16(f32x4_t &acc, const bf16x8_t &a, const bf16x8_t &b) {
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// Wait states between the last MFMA and any other instruction reading its
// accumulator (more than the deepest MFMA pipeline needs).
__device__ __forceinline__ void mfma_drain() {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
}
typedef bf16x8_t Frags[kFrags];

typedef bf16x4_t TrHalves[kFrags][2];

// Wait for all of this wave's LDS reads; the fragments are threaded through the
// asm so no instruction that consumes them can be placed above the wait.
__device__ __forceinline__ void lgkm_wait_tr(TrHalves &t) {
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(t[0][0]), "+v"(t[0][1]), "+v"(t[1][0]), "+v"(t[1][1]), "+v"(t[2][0]), "+v"(t[2][1]),
                   "+v"(t[3][0]), "+v"(t[3][1]), "+v"(t[4][0]), "+v"(t[4][1]), "+v"(t[5][0]), "+v"(t[5][1]),
                   "+v"(t[6][0]), "+v"(t[6][1]), "+v"(t[7][0]), "+v"(t[7][1])
                 :
                 : "memory");
}
__device__ __forceinline__ void lgkm_wait_tr_x(TrHalves &t, bf16x4_t &x0, bf16x4_t &x1) {
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(t[0][0]), "+v"(t[0][1]), "+v"(t[1][0]), "+v"(t[1][1]), "+v"(t[2][0]), "+v"(t[2][1]),
                   "+v"(t[3][0]), "+v"(t[3][1]), "+v"(t[4][0]), "+v"(t[4][1]), "+v"(t[5][0]), "+v"(t[5][1]),
                   "+v"(t[6][0]), "+v"(t[6][1]), "+v"(t[7][0]), "+v"(t[7][1]), "+v"(x0), "+v"(x1)
                 :
                 : "memory");
}
__device__ __forceinline__ void lgkm_wait(Frags &a, Frags &b) {
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(a[4]), "+v"(a[5]), "+v"(a[6]),
                   "+v"(a[7]), "+v"(b[0]), "+v"(b[1]), "+v"(b[2]), "+v"(b[3]), "+v"(b[4]), "+v"(b[5]),
                   "+v"(b[6]), "+v"(b[7])
                 :
                 : "memory");
}

// Wait for this wave's LDS reads of one W fragment and MB dY fragments.
template <int MB>
__device__ __forceinline__ void lgkm_wait_n(bf16x8_t &w, bf16x8_t (&g)[MB]) {
    if constexpr (MB == 1)
        asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(w), "+v"(g[0])::"memory");
    else if constexpr (MB == 2)
        asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(w), "+v"(g[0]), "+v"(g[1])::"memory");
    else
        asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(w), "+v"(g[0]), "+v"(g[1]), "+v"(g[2]), "+v"(g[3])::"memory");
}

// Wait for this wave's LDS reads of XW W fragments and MW dY fragments.
template <int XW, int MW>
__device__ __forceinline__ void lgkm_wait_wg(bf16x8_t (&w)[XW], bf16x8_t (&g)[MW]) {
    if constexpr (XW == 1) {
        lgkm_wait_n<MW>(w[0], g);
    } else if constexpr (MW == 2) {
        asm volatile("s_waitcnt lgkmcnt(0)"
                     : "+v"(w[0]), "+v"(w[1]), "+v"(w[2]), "+v"(w[3]), "+v"(g[0]), "+v"(g[1])::"memory");
    } else {
        static_assert(XW == 4 && MW == 4, "fragment counts of the small-M dX kernel");
        asm volatile("s_waitcnt lgkmcnt(0)"
                     : "+v"(w[0]), "+v"(w[1]), "+v"(w[2]), "+v"(w[3]), "+v"(g[0]), "+v"(g[1]), "+v"(g[2]),
                       "+v"(g[3])::"memory");
    }
}

// Wait until at most `n` (a multiple of 8, <= 24) of this wave's DMA
// instructions are still in flight (DMA completes in issue order).
__device__ __forceinline__ void dma_wait(int n) {
    if (n >= 24)
        asm volatile("s_waitcnt vmcnt(24)" ::: "memory");
    else if (n >= 16)
        asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
    else if (n >= 8)
        asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    else
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Workgroup barrier that publishes this wave's landed DMA and retires its LDS
// reads.  A plain s_barrier: __syncthreads() would add a release fence that
// waits for *all* outstanding DMA (vmcnt(0)) and drains the ring.  The memory
// clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void slab_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Tile index within a job -> (ti, tj).  Consecutive block ids land on
// different XCDs (round-robin dispatch), so first gather each XCD's blocks
// into one contiguous range of tiles, then raster that range in groups of
// kGroupI tile rows so concurrently running tiles share operand panels in L2.
// A job with rotated reduction starts (rows 32 KiB apart) takes groups of
// kGroupIRot rows: measured on M = 16384, N = 16384 (K = 4096) dX alone 1307
// -> 1407 TFLOP/s, both products 1414 -> 1439, and N = 32768 1349 -> 1428;
// level (within 0.5%) at M <= 8192 or K = 1024; the same bits.  For all jobs
// two-row groups made the QKV and down projections 1-1.6% slower.  So does a
// dW job of at most 16 x 16 tiles over a reduction of at most 2048 (K, N <=
// 4096, M <= 2048: the calls of a data-parallel shard), where it measured,
// both products, K = N = 4096: M = 512 56.1 -> 51.9 us, 1024 82.9 -> 80.1,
// 2048 115.8 -> 113.5 (level with K or N = 2048; 0.5-1.3% slower at M = 4096
// and 8192, which keep four rows).
__device__ __forceinline__ void tile_coords(const TileJob &jb, int t, int &ti, int &tj, int &sp) {
    int u = t;
    if ((jb.ntiles & 7) == 0)
        u = (t & 7) * (jb.ntiles >> 3) + (t >> 3);
    // the reduction range: consecutive tiles of an XCD share it (and their panels)
    const int tps = jb.tiles_i * jb.tiles_j;
    sp = u / tps;
    u -= sp * tps;
    const bool short_dw = jb.kind == JOB_DW && jb.tiles_i <= 16 && jb.tiles_j <= 16 && jb.R <= 2048;
    const int gi = jb.rot != 0 || short_dw ? kGroupIRot : kGroupI;
    const int per_group = gi * jb.tiles_j;
    const int group = u / per_group;
    const int first_i = group * gi;
    const int rows = min(jb.tiles_i - first_i, gi);
    const int in_group = u - group * per_group;
    ti = first_i + in_group % rows;
    tj = in_group / rows;
}

// Epilogue.  Block (x, y) of lane l holds C[i][j..j+3] for i = 16x + l%16,
// j = 16y + 4*(l/16) within the wave's 128x128 quadrant, so a direct store
// instruction would write 16 rows x 32 or 64 bytes: partial-line requests,
// which, issued by every CU at the end of its tile at once, made the epilogue
// cost as much as several k-steps.  Instead each wave passes its quadrant
// through its own 8 KiB of LDS beyond the operand ring (no barrier: nothing
// else touches it) in rounds of 32 rows (dX, bf16: 4 rounds) or 16 rows (dW,
// fp32: 8 rounds), row-major with 16-byte chunk c of row r at chunk c ^ (r % 16)
// (16 consecutive rows of one chunk hit distinct banks), reads each round
// back a row segment per lane group and stores whole 128-byte lines.
// Each round issues its eight LDS reads before its first store.  FULL: the
// whole 128x128 quadrant lies inside the output, and no store has a range
// check.  (With a check per store the compiler moved each LDS read into its
// store's branch and waited for it there, and without the checks it still
// alternated read, wait, store: one LDS round trip per 1 KiB store, 4.4 us per
// dX and 4.6-5.4 us per dW tile at M = 2048.)
constexpr int kEpiBytes = 8192; // per wave
// An output: row-major [I, J], leading dimension J (bf16 for KIND == JOB_DX,
// fp32 for JOB_DW).
struct OutView {
    void *c;
    int64_t I, J;
};
template <int KIND, bool FULL>
__device__ __forceinline__ void store_quadrant(const f32x4_t (&acc)[kFrags][kFrags], const OutView &jb,
                                               int64_t ib, int64_t jb0, int w, int lane, LDS char *smem) {
    LDS char *const reg = smem + kLdsBytes + w * kEpiBytes;
    if constexpr (KIND == JOB_DX) {
        // round h: fragment rows x = 2h, 2h+1 (quadrant rows 32h .. 32h+31), 256 B each
#pragma unroll
        for (int h = 0; h < kFrags / 2; ++h) {
#pragma unroll
            for (int xx = 0; xx < 2; ++xx)
#pragma unroll
                for (int y = 0; y < kFrags; ++y) {
                    const int r = 16 * xx + (lane & 15);
                    const int c = 16 * y + 4 * (lane >> 4); // bf16 column, 4 per lane
                    const f32x4_t &a = acc[2 * h + xx][y];
                    const u32x2_t pk = {pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3])};
                    *reinterpret_cast<LDS u32x2_t *>(reg + r * 256 + (((c >> 3) ^ (r & 15)) << 4) + (c & 4) * 2) =
                        pk;
                }
            u32x4_t v[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int r = 4 * q + (lane >> 4);
                const int k = lane & 15; // 8 bf16 columns
                v[q] = *reinterpret_cast<const LDS u32x4_t *>(reg + r * 256 + ((k ^ (r & 15)) << 4));
            }
            __builtin_amdgcn_sched_barrier(0); // all eight reads before the first store
            // the round's 32 rows from column jb0 on; rows past I lie past the size
            const int64_t i0 = ib + 32 * h;
            const __amdgpu_buffer_rsrc_t rs = make_rsrc(static_cast<uint16_t *>(jb.c) + i0 * jb.J + jb0,
                                                        (uint32_t)(2 * max<int64_t>(0, min<int64_t>(32, jb.I - i0)) * jb.J));
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int r = 4 * q + (lane >> 4);
                const int k = lane & 15; // J % 8 == 0: columns j..j+7 all in or all out
                const uint32_t off = (uint32_t)(2 * (r * jb.J + 8 * k));
                store_out(rs, FULL ? off : oob_unless(jb0 + 8 * k < jb.J, off), v[q]);
            }
        }
    } else {
        // round x: fragment row x (quadrant rows 16x .. 16x+15), 512 B each
#pragma unroll
        for (int x = 0; x < kFrags; ++x) {
#pragma unroll
            for (int y = 0; y < kFrags; ++y) {
                const int r = lane & 15;
                const int c = 16 * y + 4 * (lane >> 4); // fp32 column, 4 per lane
                *reinterpret_cast<LDS f32x4_t *>(reg + r * 512 + (((c >> 2) ^ r) << 4)) = acc[x][y];
            }
            f32x4_t v[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int r = 2 * q + (lane >> 5);
                const int k = lane & 31; // 4 fp32 columns
                v[q] = *reinterpret_cast<const LDS f32x4_t *>(reg + r * 512 + ((k ^ r) << 4));
            }
            __builtin_amdgcn_sched_barrier(0); // all eight reads before the first store
            const int64_t i0 = ib + 16 * x;
            const __amdgpu_buffer_rsrc_t rs = make_rsrc(static_cast<float *>(jb.c) + i0 * jb.J + jb0,
                                                        (uint32_t)(4 * max<int64_t>(0, min<int64_t>(16, jb.I - i0)) * jb.J));
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int r = 2 * q + (lane >> 5);
                const int k = lane & 31;
                const uint32_t off = (uint32_t)(4 * (r * jb.J + 4 * k));
                store_out(rs, FULL ? off : oob_unless(jb0 + 4 * k < jb.J, off), v[q]);
            }
        }
    }
}
template <int KIND>
__device__ __forceinline__ void store_tile(const f32x4_t (&acc)[kFrags][kFrags], const OutView &jb, int64_t i0,
                                           int64_t j0, int w, int wm, int wn, int lane, LDS char *smem) {
    const int64_t ib = i0 + wm * 128;
    const int64_t jb0 = j0 + wn * 128;
    if (ib + 128 <= jb.I && jb0 + 128 <= jb.J)
        store_quadrant<KIND, true>(acc, jb, ib, jb0, w, lane, smem);
    else
        store_quadrant<KIND, false>(acc, jb, ib, jb0, w, lane, smem);
}

// ---- RC operands (dX): slab pairs ----
// Two consecutive 32-deep slabs are stored together, as 256 rows of 128 B
// (r 0..63 of the pair), so each 8-lane group of a DMA instruction fetches one
// whole 128-byte line: half-line requests would double the L1->L2 request
// count.  The 128 KiB hold two such pairs per operand.  16-byte chunk c of row
// o is stored at chunk c ^ (o % 8), so the 8 rows of one chunk that a fragment
// read serves together sit on distinct banks (measured with the LDS conflict
// counter: 0 conflict cycles; also folding bit 3 of the row into the XOR, as
// an earlier layout did, gave conflicts in a quarter of the active cycles).
constexpr int kPairBytes = 2 * kOperandBytes; // 32 KiB per operand
constexpr int kDmaPerOpPair = 8;              // DMA instructions per wave per operand per pair
__device__ __forceinline__ int swz_rcp(int row) { return row & 7; }
__device__ __forceinline__ int rcp_off(int o, int c) { return o * 128 + ((c ^ swz_rcp(o)) << 4); }
// fragment of outer block ob (16 wide) for slab half h of a pair
__device__ __forceinline__ int frag_off_rcp(int ob, int lane, int h) {
    return rcp_off(ob + (lane & 15), 4 * h + (lane >> 4));
}
// DMA instruction p of wave w fills pair rows 8q .. 8q+7, q = 8w + p; lane l
// fetches logical chunk (l & 7) ^ swz_rcp(row) of row 8q + l/8.  Offset
// relative to the tile's first operand row and the pair's first r (so it
// stays below 2^31 for operands of any size: 256 rows of ld < 2^22); rows
// outside the operand (or, for the partial last pair, r >= R) read zero.
__device__ __forceinline__ uint32_t dma_rcp_off(int p, int64_t ld, int64_t O, int64_t o0, int w, int lane,
                                                int64_t k0 = 0, int64_t R = -1) {
    const int row = (w * kDmaPerOpPair + p) * 8 + (lane >> 3);
    const int lc = (lane & 7) ^ swz_rcp(row);
    const int64_t k = k0 + 8 * lc;
    const bool ok = o0 + row < O && (R < 0 || k < R);
    return oob_unless(ok, (uint32_t)((row * ld + (R < 0 ? 0 : k0) + 8 * lc) * 2));
}

// dX tile.  Slab t lives in pair t/2, ring slot (t/2)%2, half t%2.  During
// slab t the MFMAs use slab t's fragments (in registers) while slab t+1's are
// read; an odd slab t first waits for pair (t+1)/2 and barriers (after which
// the slot of pair (t-1)/2, whose fragments are all in registers, is free),
// then issues the DMA of pair (t+3)/2 into that slot, one instruction every
// fourth MFMA: a pair is fetched one to two slabs ahead of its first use, with
// one barrier per pair.  The spacing keeps the CU's address path at its rate
// (the four waves' 64 instructions of 1 KiB over 64 MFMAs); issued every
// second MFMA, or half of them in the next slab, the address FIFO filled, the
// waves stalled unevenly and the barrier paid for the skew (block 1.8% slower).
template <bool SPLIT> // SPLIT: the job's reduction is split (fp32 partials out)
__device__ __forceinline__ void run_tile_rc(const TileJob &jb, int t_index, LDS char *smem) {
    static_assert(kStages * kOperandBytes == 2 * kPairBytes, "two pairs per operand");
    constexpr int kReads = 2 * kFrags; // ds_read_b128 per wave per slab
    int ti, tj, sp;
    tile_coords(jb, t_index, ti, tj, sp);
    const int64_t i0 = (int64_t)ti * kTile;
    const int64_t j0 = (int64_t)tj * kTile;
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = w >> 1, wn = w & 1;

    uint32_t va[kDmaPerOpPair], vb[kDmaPerOpPair];
#pragma unroll
    for (int p = 0; p < kDmaPerOpPair; ++p) {
        va[p] = dma_rcp_off(p, jb.lda, jb.I, i0, w, lane);
        vb[p] = dma_rcp_off(p, jb.ldb, jb.J, j0, w, lane);
    }
    int fo[2][kFrags][2]; // [A/B][block][half]
#pragma unroll
    for (int x = 0; x < kFrags; ++x)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            fo[0][x][h] = frag_off_rcp(wm * 128 + x * 16, lane, h);
            fo[1][x][h] = kBOffset + frag_off_rcp(wn * 128 + x * 16, lane, h);
        }
    f32x4_t acc[kFrags][kFrags];
#pragma unroll
    for (int x = 0; x < kFrags; ++x)
#pragma unroll
        for (int y = 0; y < kFrags; ++y)
            acc[x][y] = f32x4_t{};

    // this tile's reduction range: [kb, kb + R) of the job's (one range unless split)
    const int64_t kb = (int64_t)sp * jb.split_len;
    const int64_t R = min<int64_t>(jb.split_len, jb.R - kb);
    const int npair = (int)((R + 63) / 64);
    const int nslab4 = (int)(((R + kBK - 1) / kBK + 3) / 4 * 4); // padded with zero slabs
    const int P = nslab4 / 2;                                     // pairs, padding included
    const bool ptail = (R % 64) != 0;                             // last real pair is partial
    // rotation of the reduction order (see TileJob), in whole pairs
    const int rotp = ptail || npair == 0 ? 0 : ((jb.rot * ((tj >> 1) & 3)) >> 1) % npair;
    LDS char *const wdst = smem + w * kDmaPerOpPair * 1024;
    // the tile's operand rows from the range's first column: windows of at
    // most 256 rows (2 * 256 * ld < 2^31), from a_t / b_t to the window's end
    const uint16_t *const a_t = jb.a + i0 * jb.lda + kb;
    const uint16_t *const b_t = jb.b + j0 * jb.ldb + kb;
    const uint32_t a_win = (uint32_t)(2 * (min<int64_t>(kTile, jb.I - i0) * jb.lda - kb));
    const uint32_t b_win = (uint32_t)(2 * (min<int64_t>(kTile, jb.J - j0) * jb.ldb - kb));

    struct PairSrc {
        __amdgpu_buffer_rsrc_t a, b;
    };
    auto pair_src = [&](int q) {
        PairSrc r;
        if (q >= npair) { // padding: every lane out of range, reads zero
            r.a = make_rsrc(jb.a, 0);
            r.b = make_rsrc(jb.b, 0);
            return r;
        }
        q += rotp;
        q = q >= npair ? q - npair : q;
        const int64_t k0 = (int64_t)q * 64;
        r.a = make_rsrc(a_t + k0, a_win - (uint32_t)(2 * k0));
        r.b = make_rsrc(b_t + k0, b_win - (uint32_t)(2 * k0));
        return r;
    };
    auto dma = [&](const PairSrc &src, int q, int op, int p, bool tail) {
        LDS char *st = wdst + (q & 1) * kPairBytes + p * 1024 + op * kBOffset;
        if (tail) {
            const int64_t k0 = (int64_t)q * 64;
            if (op == 0)
                dma16(make_rsrc(a_t, a_win), st, dma_rcp_off(p, jb.lda, jb.I, i0, w, lane, k0, R));
            else
                dma16(make_rsrc(b_t, b_win), st, dma_rcp_off(p, jb.ldb, jb.J, j0, w, lane, k0, R));
        } else {
            dma16(op == 0 ? src.a : src.b, st, op == 0 ? va[p] : vb[p]);
        }
    };
    // LDS read j (0..15) of the slab with t % 4 == TM
    auto read_frag = [&](auto tm, int j, Frags &an, Frags &bn) {
        constexpr int m = decltype(tm)::value;
        constexpr int off = ((m >> 1) & 1) * kPairBytes;
        const int op = j / kFrags, xb = j % kFrags;
        (op == 0 ? an : bn)[xb] = read_rc<off>(smem + fo[op][xb][m & 1]);
    };
    // slab t with t % 4 == TM (compile time); flags as described above (only
    // odd slabs issue DMAs: the 16 instructions of pair (t+3)/2, from `src`)
    auto slab = [&](int t, auto tm, bool dmas, bool tail, bool N, const PairSrc &src, Frags &af, Frags &bf,
                    Frags &an, Frags &bn) {
        constexpr int m = decltype(tm)::value;
        constexpr bool odd = m & 1;
        const int q = (t + 3) / 2;
        if (odd && N) {
            dma_wait(0);
            slab_barrier();
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < kFrags * kFrags; ++i) {
            const int x = i / kFrags, y = i % kFrags;
            mfma16(acc[x][y], bf[y], af[x]);
            __builtin_amdgcn_sched_barrier(0);
            if (i % 2 == 0 && i / 2 < kReads)
                read_frag(std::integral_constant<int, (m + 1) % 4>{}, i / 2, an, bn);
            if (odd && dmas && i % 4 == 1) { // MFMAs 1, 5, ..., 61
                const int d = i / 4;
                dma(src, q, d & 1, d >> 1, tail);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        lgkm_wait(an, bn);
        __builtin_amdgcn_sched_barrier(0);
    };

    Frags af, bf, an, bn;
    if (nslab4 > 0) {
        // prologue: pairs 0 and 1 fill both slots; wait for pair 0 and read slab 0
        for (int q = 0; q < 2; ++q) {
            const PairSrc src = pair_src(q);
            const bool tail = ptail && q == npair - 1;
#pragma unroll
            for (int d = 0; d < 2 * kDmaPerOpPair; ++d)
                dma(src, q, d & 1, d >> 1, tail);
        }
        dma_wait(2 * kDmaPerOpPair);
        slab_barrier();
#pragma unroll
        for (int j = 0; j < kReads; ++j)
            read_frag(std::integral_constant<int, 0>{}, j, af, bf);
        lgkm_wait(af, bf);

        using C0 = std::integral_constant<int, 0>;
        using C1 = std::integral_constant<int, 1>;
        using C2 = std::integral_constant<int, 2>;
        using C3 = std::integral_constant<int, 3>;
        int s = 0;
        // steady state: the pairs issued (s/2 + 2, s/2 + 3) are full ones.
        // Their sources come from a cursor that advances base and window by a
        // pair (the general pair_src, between two slabs, held up the odd
        // slab's first MFMA): cq is the rotated index of the next pair fetched.
        if (npair > 4) {
            int cq = (2 + rotp) % npair;
            const uint16_t *ca = a_t + (int64_t)cq * 64, *cb = b_t + (int64_t)cq * 64;
            uint32_t cwa = a_win - 128u * (uint32_t)cq, cwb = b_win - 128u * (uint32_t)cq;
            auto next_pair = [&]() {
                const PairSrc r{make_rsrc(ca, cwa), make_rsrc(cb, cwb)};
                ++cq;
                ca += 64;
                cb += 64;
                cwa -= 128;
                cwb -= 128;
                if (cq == npair) { // the rotated order wraps to the first pair
                    cq = 0;
                    ca = a_t;
                    cb = b_t;
                    cwa = a_win;
                    cwb = b_win;
                }
                return r;
            };
            const PairSrc none{};
            for (; s / 2 + 4 < npair; s += 4) {
                slab(s + 0, C0{}, true, false, false, none, af, bf, an, bn);
                slab(s + 1, C1{}, true, false, true, next_pair(), an, bn, af, bf);
                slab(s + 2, C2{}, true, false, false, none, af, bf, an, bn);
                slab(s + 3, C3{}, true, false, true, next_pair(), an, bn, af, bf);
            }
        }
        auto flags = [&](int t, bool &dmas, bool &tail, bool &N) {
            const bool odd = t & 1;
            const int q = (t + 3) / 2;
            dmas = odd && q < P;
            tail = dmas && ptail && q == npair - 1;
            N = odd && t + 1 < nslab4;
        };
        for (; s < nslab4; s += 4) {
            bool d0, t0, n0, d1, t1, n1, d2, t2, n2, d3, t3, n3;
            flags(s + 0, d0, t0, n0);
            flags(s + 1, d1, t1, n1);
            flags(s + 2, d2, t2, n2);
            flags(s + 3, d3, t3, n3);
            const PairSrc none{};
            slab(s + 0, C0{}, d0, t0, n0, none, af, bf, an, bn);
            slab(s + 1, C1{}, d1, t1, n1, pair_src((s + 4) / 2), an, bn, af, bf);
            slab(s + 2, C2{}, d2, t2, n2, none, af, bf, an, bn);
            slab(s + 3, C3{}, d3, t3, n3, pair_src((s + 6) / 2), an, bn, af, bf);
        }
    }
    mfma_drain();
    // (one epilogue per instantiation: with both behind a run-time branch the
    // compiler copied the accumulators out of the AGPRs before it and spilled)
    if constexpr (SPLIT) // fp32 partial sums of range sp
        store_tile<JOB_DW>(acc, OutView{jb.part + (int64_t)sp * jb.I * jb.J, jb.I, jb.J}, i0, j0, w, wm, wn, lane,
                           smem);
    else
        store_tile<JOB_DX>(acc, OutView{jb.c, jb.I, jb.J}, i0, j0, w, wm, wn, lane, smem);
}

// dW tile (OC operands).  Wave w = 2*wm + wn owns the 128x128 quadrant
// (wm, wn) as 8x8 blocks of 16x16 (v_mfma_f32_16x16x32_bf16, fp32 accumulate).
// The reduction runs in slabs of 32 through a 4-slot LDS ring; one slab is one
// k-step of 64 MFMAs per wave.  The reduction order is never rotated here
// (rotation is for the dX job's operands only).
__device__ __forceinline__ void run_tile_oc(const TileJob &jb, int t_index, LDS char *smem) {
    static_assert(kDmaPerOp == 4 && kStages == 4, "pipeline below assumes 4 DMAs per operand, 4 stages");
    constexpr int kRPF = 2;                   // ds_read_b64_tr_b16 per fragment
    constexpr int kReads = 2 * kFrags * kRPF; // per wave per slab
    constexpr int kDmaPerSlab = 2 * kDmaPerOp;
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); // wave-uniform
    const int wm = w >> 1, wn = w & 1;

    // LDS fragment addresses: the same for every tile
    int fo[2][kFrags][kRPF]; // [A/B][block][half]
#pragma unroll
    for (int x = 0; x < kFrags; ++x)
#pragma unroll
        for (int h = 0; h < kRPF; ++h) {
            fo[0][x][h] = frag_off_oc(wm * 128 + x * 16, lane, h);
            fo[1][x][h] = kBOffset + frag_off_oc(wn * 128 + x * 16, lane, h);
        }

    const int nslab = (int)((jb.R + kBK - 1) / kBK);
    // The slab count is padded to a multiple of the ring size with slabs that
    // read zero, so every pass of the loops below runs four whole slabs with
    // compile-time ring slots and no early exit.
    const int nslab4 = (nslab + kStages - 1) / kStages * kStages;
    // per-slab source advance (elements) and a full slab's bytes, per operand
    // (32 rows of ld < 2^25: below 2^31 bytes)
    const int64_t step_a = (int64_t)kBK * jb.lda;
    const int64_t step_b = (int64_t)kBK * jb.ldb;
    const uint32_t full_a = (uint32_t)(2 * step_a);
    const uint32_t full_b = (uint32_t)(2 * step_b);
    LDS char *const wdst = smem + w * kDmaPerOp * 1024; // this wave's DMA destinations

    int ti, tj, sp;
    tile_coords(jb, t_index, ti, tj, sp); // one reduction range: sp = 0
    const int64_t i0 = (int64_t)ti * kTile;
    const int64_t j0 = (int64_t)tj * kTile;
    // slab-independent per-lane DMA source offsets
    uint32_t va[kDmaPerOp], vb[kDmaPerOp];
#pragma unroll
    for (int p = 0; p < kDmaPerOp; ++p) {
        va[p] = dma_oc_off(p, jb.lda, jb.I, i0, w, lane);
        vb[p] = dma_oc_off(p, jb.ldb, jb.J, j0, w, lane);
    }

    // Buffer descriptors for slab s: the base at the slab's first row, the size
    // the rows left, so rows past R read zero.  The general form (padding
    // slabs, a partial last slab) serves the prologue and the last groups;
    // the steady state advances two pointers by a slab instead (the general
    // form's 64-bit products, done between two slabs, held up the first MFMA
    // of every slab).
    struct SlabSrc {
        __amdgpu_buffer_rsrc_t a, b;
    };
    auto slab_src = [&](int s) {
        SlabSrc r;
        if (s >= nslab) { // padding slab: every lane out of range, reads zero
            r.a = make_rsrc(jb.a, 0);
            r.b = make_rsrc(jb.b, 0);
            return r;
        }
        const int64_t rows = min<int64_t>(kBK, jb.R - (int64_t)s * kBK);
        r.a = make_rsrc(jb.a + s * step_a, (uint32_t)(2 * rows * jb.lda));
        r.b = make_rsrc(jb.b + s * step_b, (uint32_t)(2 * rows * jb.ldb));
        return r;
    };
    // DMA instruction p of operand op for a slab in ring slot `slot`
    auto dma = [&](const SlabSrc &src, int slot, int op, int p) {
        LDS char *st = wdst + slot * kOperandBytes + p * 1024 + op * kBOffset;
        dma16(op == 0 ? src.a : src.b, st, op == 0 ? va[p] : vb[p]);
    };
    // Read LDS read number j (0 .. kReads-1) of a slab held in ring slot `stage`
    // (an int, or a compile-time constant that becomes the immediate offset).
    auto read_frag = [&](auto stage, int j, TrHalves (&tr)[2]) {
        const int op = j / (kFrags * kRPF), xb = (j % (kFrags * kRPF)) / kRPF, h = j % kRPF;
        const LDS char *base = smem + fo[op][xb][h];
        if constexpr (std::is_integral_v<decltype(stage)>) {
            tr[op][xb][h] = read_tr<0>(base + stage * kOperandBytes);
        } else {
            constexpr int off = decltype(stage)::value * kOperandBytes;
            tr[op][xb][h] = read_tr<off>(base);
        }
    };
    // wait for the slab's reads, then join the two transposed halves
    auto finish_reads = [&](Frags &an, Frags &bn, TrHalves (&tr)[2]) {
        lgkm_wait_tr(tr[0]);
        lgkm_wait_tr(tr[1]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int xb = 0; xb < kFrags; ++xb) {
            an[xb] = __builtin_shufflevector(tr[0][xb][0], tr[0][xb][1], 0, 1, 2, 3, 4, 5, 6, 7);
            bn[xb] = __builtin_shufflevector(tr[1][xb][0], tr[1][xb][1], 0, 1, 2, 3, 4, 5, 6, 7);
        }
    };

    // Slab s (fragments already in af/bf):
    //   if there is a slab s+1: wait for its DMA and barrier.  After the
    //   barrier every wave has its slab-s fragments in registers, so ring slot
    //   s%4 is free and takes the DMA (source src) of slab s+4;
    //   64 MFMAs on (af, bf); the LDS reads of slab s+1 into (an, bn) go with
    //   the first MFMAs, the DMA with later ones (sched_barrier pins the order,
    //   so the matrix pipe never waits behind address or memory work).
    //   The last slab reads its successor's ring slot too (stale data, never
    //   used): keeping the reads unconditional lets the transposed halves share
    //   registers with the fragments they form.
    // wait_n: this wave's DMA instructions issued after the following slab's.
    // stage: the ring slot of slab s, a compile-time constant; the next slab's
    // slot is derived from it.
    constexpr int kReadSlot = 1; // MFMA slots per LDS read
    // DMA j after MFMA kDmaSlot0 + kDmaStep*j (33, 37, ..., 61): spaced so the
    // four waves' instructions stay within the CU's address rate (every second
    // MFMA filled the address FIFO; block 1.9% slower)
    constexpr int kDmaSlot0 = 33;
    constexpr int kDmaStep = 4;
    f32x4_t acc[kFrags][kFrags];
#pragma unroll
    for (int x = 0; x < kFrags; ++x)
#pragma unroll
        for (int y = 0; y < kFrags; ++y)
            acc[x][y] = f32x4_t{};
    auto slab = [&](auto stage, bool dmas, const SlabSrc &src, bool N, int wait_n, Frags &af, Frags &bf,
                    Frags &an, Frags &bn) {
        constexpr int slot = decltype(stage)::value;
        using Next = std::integral_constant<int, (slot + 1) % kStages>;
        if (N) {
            dma_wait(wait_n);
            slab_barrier();
        }
        __builtin_amdgcn_sched_barrier(0);
        TrHalves tr[2];
#pragma unroll
        for (int i = 0; i < kFrags * kFrags; ++i) {
            const int x = i / kFrags, y = i % kFrags;
            mfma16(acc[x][y], bf[y], af[x]);
            __builtin_amdgcn_sched_barrier(0);
            if (i % kReadSlot == 0 && i / kReadSlot < kReads)
                read_frag(Next{}, i / kReadSlot, tr);
            if (dmas && i >= kDmaSlot0 && i < kDmaSlot0 + kDmaStep * kDmaPerSlab &&
                (i - kDmaSlot0) % kDmaStep == 0) {
                const int d = (i - kDmaSlot0) / kDmaStep;
                dma(src, slot, d & 1, d >> 1);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        finish_reads(an, bn, tr);
        __builtin_amdgcn_sched_barrier(0);
    };
    using C0 = std::integral_constant<int, 0>;
    using C1 = std::integral_constant<int, 1>;
    using C2 = std::integral_constant<int, 2>;
    using C3 = std::integral_constant<int, 3>;
    constexpr int kW = 2 * kDmaPerSlab; // steady state: the two slabs after the next may be in flight
    const SlabSrc none{};
    Frags af, bf, an, bn;
    if (nslab > 0) {
        // prologue: slabs 0..3 fill the ring; wait for slab 0 and read it
        for (int s = 0; s < kStages; ++s) {
            const SlabSrc src = slab_src(s);
#pragma unroll
            for (int p = 0; p < kDmaPerOp; ++p) {
                dma(src, s, 0, p);
                dma(src, s, 1, p);
            }
        }
        dma_wait(kDmaPerSlab * (kStages - 1));
        slab_barrier();
        {
            TrHalves tr[2];
#pragma unroll
            for (int j = 0; j < kReads; ++j)
                read_frag(0, j, tr);
            finish_reads(af, bf, tr);
        }
        int s = 0;
        // steady state: slab s+4 is a full slab, branch free; pa / pb point at
        // the slab the next DMA fetches
        const uint16_t *pa = jb.a + 4 * step_a;
        const uint16_t *pb = jb.b + 4 * step_b;
        auto next_src = [&]() {
            const SlabSrc r{make_rsrc(pa, full_a), make_rsrc(pb, full_b)};
            pa += step_a;
            pb += step_b;
            return r;
        };
        for (; s + 2 * kStages < nslab; s += kStages) {
            slab(C0{}, true, next_src(), true, kW, af, bf, an, bn);
            slab(C1{}, true, next_src(), true, kW, an, bn, af, bf);
            slab(C2{}, true, next_src(), true, kW, af, bf, an, bn);
            slab(C3{}, true, next_src(), true, kW, an, bn, af, bf);
        }
        // the groups whose DMA targets may be partial or padding slabs
        for (; s + kStages < nslab4; s += kStages) {
            slab(C0{}, true, slab_src(s + 4), true, kW, af, bf, an, bn);
            slab(C1{}, true, slab_src(s + 5), true, kW, an, bn, af, bf);
            slab(C2{}, true, slab_src(s + 6), true, kW, af, bf, an, bn);
            slab(C3{}, true, slab_src(s + 7), true, kW, an, bn, af, bf);
        }
        // draining: no more DMAs; slab t waits for t+1 while one exists
        slab(C0{}, false, none, true, kDmaPerSlab * 2, af, bf, an, bn);
        slab(C1{}, false, none, true, kDmaPerSlab * 1, an, bn, af, bf);
        slab(C2{}, false, none, true, 0, af, bf, an, bn);
        slab(C3{}, false, none, false, 0, an, bn, af, bf);
    }

    mfma_drain();
    store_tile<JOB_DW>(acc, OutView{jb.c, jb.I, jb.J}, i0, j0, w, wm, wn, lane, smem);
}

// One block = one tile of job 0 or job 1.  SPLIT: the dX job (if any) has its
// reduction split into several ranges (k_lin_bwd_mfma_split).
template <bool SPLIT>
__device__ __forceinline__ void lin_bwd_mfma_block(const MfmaParams &p) {
    __shared__ __attribute__((aligned(1024))) char smem_raw[kLdsBytes + 4 * kEpiBytes];
    LDS char *smem = (LDS char *)smem_raw;
    int b = blockIdx.x;
    const TileJob *jb = &p.job[0];
    if (b >= p.job[0].ntiles) {
        b -= p.job[0].ntiles;
        jb = &p.job[1];
    }
    if (jb->kind == JOB_DX)
        run_tile_rc<SPLIT>(*jb, b, smem);
    else
        run_tile_oc(*jb, b, smem);
}
__global__ __launch_bounds__(kThreads, 1) void k_lin_bwd_mfma(MfmaParams p) { lin_bwd_mfma_block<false>(p); }
__global__ __launch_bounds__(kThreads, 1) void k_lin_bwd_mfma_split(MfmaParams p) { lin_bwd_mfma_block<true>(p); }

// ------------------------------------------------------------------------
// small M: at M <= 64 both products are bound by HBM, not MFMA: dX streams W
// (2KN bytes), dW writes the fp32 output (4KN bytes).  Up to M = 256 dX takes
// the split-reduction kernel below and dW the small-tile kernel, as two
// launches, or at M <= 64 (up to an N and a K*N: plan::pair_fits) as one
// launch holding the blocks of both (k_smallm_pair); from M = 257, where dW
// returns to the tile kernel, dX joins it there with its reduction split over
// several tiles (the tile kernel with whole reductions would give dX only
// (M/256)(K/256) long tiles).
// (With dX's 144 KiB ring the one launch lost: the dX blocks took every CU
// first and the dW blocks ran at the merged kernel's occupancy of one block
// per CU.  With 72 KiB it wins up to N = 8192 and a dW of 128 MiB; at N = 16384
// or K = N = 8192 the mixed read and write streams still made it slower than
// the two launches in turn.)
// ------------------------------------------------------------------------
constexpr int kSmallMaxM = 256;   // dW: the small-tile kernel up to this M
constexpr int kSmallMaxDxM = 1024; // dX: the small-M kernel up to this M (split tile ranges: kDxSplitMaxM)

struct SmallParams {
    const uint16_t *X, *W, *G; // X[M,K], W[K,N], dY[M,N]
    uint16_t *dX;              // [M,K] bf16, or null
    float *dW;                 // [K,N] fp32, or null
    float *part;               // split partials [splits][M][K] (splits > 1)
    int64_t M, K, N;
    int64_t split_len;         // reduction elements per dX split (a whole number of chunks)
    int splits;                // dX splits per column group
    int mgroups;               // dX row groups of 16*MB rows; block b = ((group, row group), split):
                               // split b % splits, row group (b / splits) % mgroups, group b / splits / mgroups
    int dw_tiles_n;            // dW block b = (n tile, k tile) (b % dw_tiles_n, b / dw_tiles_n)
    int reduce_blocks;         // dW blocks that also add up dX partials
    int dx_blocks;             // k_smallm_pair: blocks below this run dX, the rest dW
};

// dW[k,n] = Σ_m X[m,k]·dY[m,n] for M <= 256: a rank-M product whose cost is
// writing the output.  Small 64x256 tiles (several resident per CU) let one
// tile's stores overlap other tiles' loads and MFMAs; a 256x256 tile of the
// main kernel holds a CU for its whole tile and every CU then stores at once.
// Per block the reduction runs in 32-row slabs through a two-slot LDS ring,
// both operands by DMA: dY[slab, n0:n0+256] as an OC slab (the main kernel's
// layout and fragment reads), X[slab, k0:k0+64] as 32 rows of 128 bytes.
// Wave w owns dW rows k0+16w .. +15 (16 blocks of 16x16, one MFMA per block
// and slab), then passes them through 4 KiB of LDS per wave in rounds of 64
// columns so that each store instruction writes 4 rows x 256 contiguous bytes.
constexpr int kDwsBK = 64;                 // dW rows per block (16 per wave)
constexpr int kDwsBN = kTile;              // dW columns per block (one OC slab row)
constexpr int kDwsXSlab = 32 * kDwsBK * 2; // X slab in LDS: 32 rows x 128 B
constexpr int kDwsSlot = kOperandBytes + kDwsXSlab;
constexpr int kDwsStage = 4096;            // per-wave epilogue staging: 16 rows x 256 B
constexpr int kDwsLds = 2 * kDwsSlot + 4 * kDwsStage;

__device__ __forceinline__ bf16x8_t join4(bf16x4_t lo, bf16x4_t hi) {
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ void dw_small_block(const SmallParams &p, int b, LDS char *smem) {
    const int64_t M = p.M, K = p.K, N = p.N;
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    LDS char *const stage = smem + 2 * kDwsSlot + w * kDwsStage;
    const int64_t n0 = (int64_t)(b % p.dw_tiles_n) * kDwsBN;
    const int64_t k0 = (int64_t)(b / p.dw_tiles_n) * kDwsBK;
    const int nslab = (int)((M + 31) / 32);
    // dY rows from the slab on (rows past M and columns past N read zero through
    // the descriptor's size or kOOB); X by row: lane l of wave w's instruction
    // fetches chunk l%8 of slab row 8w + l/8 (offsets are 32-bit: 2MK < 2^31)
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(p.X, (uint32_t)(2 * M * K));
    const int xrow = 8 * w + (lane >> 3);
    const int64_t xk = k0 + 8 * (lane & 7);
    auto issue = [&](int s) { // slab s into slot s % 2: 5 DMA instructions per wave
        LDS char *slot = smem + (s & 1) * kDwsSlot;
        const int64_t r0 = 32 * (int64_t)s;
        const __amdgpu_buffer_rsrc_t rg = make_rsrc(p.G + r0 * N, (uint32_t)(2 * min<int64_t>(32, M - r0) * N));
#pragma unroll
        for (int q = 0; q < kDmaPerOp; ++q)
            dma16(rg, slot + (w * kDmaPerOp + q) * 1024, dma_oc_off(q, N, N, n0, w, lane));
        const int64_t m = r0 + xrow;
        dma16(rx, slot + kOperandBytes + 8 * w * 128, m < M && xk < K ? (uint32_t)(2 * (m * K + xk)) : kOOB);
    };

    // fragments: lane l holds outer index ob + l%16 and r = 8(l/16) .. +7,
    // read as two transposing halves (r 4h .. 4h+3 of each 8)
    f32x4_t acc[16];
#pragma unroll
    for (int y = 0; y < 16; ++y)
        acc[y] = f32x4_t{};
    const int g = lane >> 4, sl = lane & 15;
    issue(0);
    if (nslab > 1)
        issue(1);
    for (int s = 0; s < nslab; ++s) {
        if (s + 1 < nslab)
            asm volatile("s_waitcnt vmcnt(5)" ::: "memory"); // the next slab may stay in flight
        else
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        slab_barrier();
        // fragment reads as inline asm with explicit waits: with the builtin the
        // compiler waits for all DMA in flight (the next slab's too) first
        const LDS char *gb = smem + (s & 1) * kDwsSlot;
        const LDS char *xb = gb + kOperandBytes;
        const int xcol = 16 * w + 4 * (sl & 3);
        bf16x4_t x0 = read_tr<0>(xb + (8 * g + (sl >> 2)) * 128 + xcol * 2);
        bf16x4_t x1 = read_tr<0>(xb + (8 * g + 4 + (sl >> 2)) * 128 + xcol * 2);
        TrHalves tr[2]; // all 16 dY fragments in registers of their own: no read overwrites an MFMA source
#pragma unroll
        for (int y = 0; y < 16; ++y)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                tr[y >> 3][y & 7][h] = read_tr<0>(gb + frag_off_oc(16 * y, lane, h));
        lgkm_wait_tr_x(tr[0], x0, x1);
        lgkm_wait_tr(tr[1]);
        const bf16x8_t xf = join4(x0, x1);
#pragma unroll
        for (int y = 0; y < 16; ++y) // lane l: dW[k0 + 16w + l%16][n0 + 16y + 4(l/16) .. +3]
            acc[y] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(join4(tr[y >> 3][y & 7][0], tr[y >> 3][y & 7][1]), xf,
                                                             acc[y], 0, 0, 0);
        if (s + 2 < nslab) {
            slab_barrier(); // every wave has read this slot
            issue(s + 2);
        }
    }

    // epilogue: round q covers columns 64q .. 64q+63 of the wave's 16 rows;
    // 16-byte chunk c of staging row r sits at chunk c ^ r.  The wave's rows
    // are one buffer window from column n0 on (rows past K lie past its size).
    const int64_t kw = k0 + 16 * w;
    const __amdgpu_buffer_rsrc_t rdw =
        make_rsrc(p.dW + kw * N + n0, (uint32_t)(4 * max<int64_t>(0, min<int64_t>(16, K - kw)) * N));
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#pragma unroll
        for (int yy = 0; yy < 4; ++yy) {
            const int r = sl, c = 4 * yy + g;
            *reinterpret_cast<LDS f32x4_t *>(stage + r * 256 + ((c ^ r) << 4)) = acc[4 * q + yy];
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int r = 4 * t + g, c = sl;
            const f32x4_t v = *reinterpret_cast<const LDS f32x4_t *>(stage + r * 256 + ((c ^ r) << 4));
            const int nl = 64 * q + 4 * c; // N % 8 == 0: n .. n+3 all in range or all out
            store_out(rdw, oob_unless(n0 + nl < N, (uint32_t)(4 * (r * N + nl))), v);
        }
    }
}

// dX[m,k] = Σ_n dY[m,n]·W[k,n] with M <= 16*MB, for small M (up to 256): the
// tile kernel would give it only K/256 tiles.  Bound by streaming W once at
// M <= 64, by both W and the MFMAs near 256.  Block (s, grp): dX columns
// k0 = 64grp .. +63 over the reduction range of split s, in chunks of CH n
// through an LDS ring of three slots where they fit (two otherwise).  Wave w
// streams rows k0+16w .. +15 of W: each DMA instruction fetches 1 KiB of
// whole rows (two rows x 512 bytes at CH = 256, four x 256 at CH = 128) with
// the non-temporal policy (W is read once; loading MFMA fragments straight
// from memory touches 16 rows x 64 bytes per instruction and was slower), and
// the wave only ever reads its own rows back.  dY[0:M, chunk] is shared by
// the four waves.  In both, 16-byte chunk c of an LDS row r sits at chunk
// c ^ (r % 16), so the 16 rows one fragment read serves hit distinct banks.
// Per chunk: wait for its DMA, barrier, DMA of the chunk kS-1 ahead into the
// slot the barrier freed, CH/32 MFMA steps.  With one split the block stores
// dX in bf16; with several it stores fp32 partial sums part[s][m][k] that are
// added in split order afterwards.  (A last-block-reduces variant, counting
// finished splits with a device-scope atomic, needs a device-scope release
// and acquire per block; on this part those write back and invalidate the
// XCD's L2, and dX took 5x longer.)
constexpr int kDxsBK = 64; // dX columns per block
template <int MB> // reduction elements per chunk: dY's slot stays within LDS
constexpr int dx_small_chunk() { return MB <= 4 ? 256 : 128; }
template <int MB, int CH = dx_small_chunk<MB>()>
constexpr int dx_small_slot() { return (64 + MB * 16) * CH * 2; }
template <int MB, int CH = dx_small_chunk<MB>()> // ring slots: three where they fit in LDS
constexpr int dx_small_slots() { return 3 * dx_small_slot<MB, CH>() <= 160 * 1024 ? 3 : 2; }
template <int MB, int CH = dx_small_chunk<MB>(), int S = dx_small_slots<MB, CH>()>
constexpr int dx_small_lds() { return S * dx_small_slot<MB, CH>(); }

// Wait until at most `c` chunks' DMA (kPerChunk instructions each) are in flight.
template <int kPerChunk>
__device__ __forceinline__ void dx_chunk_wait(int c) {
    if (c >= 2)
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * kPerChunk) : "memory");
    else if (c == 1)
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kPerChunk) : "memory");
    else
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

template <int MB, int kCH = dx_small_chunk<MB>(), int kS = dx_small_slots<MB, kCH>()>
__device__ __forceinline__ void dx_small_block(const SmallParams &p, int b, LDS char *smem) {
    constexpr int kRow = 2 * kCH;                // bytes per LDS row
    constexpr int kCPR = kRow / 16;              // 16-byte chunks per row
    constexpr int kRPI = 1024 / kRow;            // rows per DMA instruction
    constexpr int kWSlot = 64 * kRow;            // W part of a slot
    constexpr int kSlot = dx_small_slot<MB, kCH>();
    constexpr int kWInst = 16 / kRPI;            // W DMA instructions per wave per chunk
    constexpr int kGInst = MB * 16 / kRPI / 4;   // dY DMA instructions per wave per chunk
    constexpr int kPerChunk = kWInst + kGInst;
    static_assert(kCPR >= 16, "the XOR swizzle spans 16 chunks");
    static_assert((kS - 1) * kPerChunk <= 63, "the chunks in flight fit the vmcnt counter");
    const int64_t M = p.M, K = p.K, N = p.N;
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int s = b % p.splits, mg = (b / p.splits) % p.mgroups, grp = b / p.splits / p.mgroups;
    const int64_t k0 = (int64_t)grp * kDxsBK;
    const int64_t m0 = (int64_t)mg * 16 * MB; // this block's rows of dY and dX
    const int64_t n_beg = (int64_t)s * p.split_len;
    const int64_t n_end = min(N, n_beg + p.split_len);
    const int nc = (int)((n_end - n_beg + kCH - 1) / kCH);
    // W rows from k0 on, and dY; offsets are 32-bit (2KN, 2MN < 2^31) and
    // rows or columns out of range read zero through kOOB
    // windows: the block's 64 rows of W and 16 MB rows of dY (offsets below 2^31 for N < 2^22)
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(p.W + k0 * N, (uint32_t)(2 * min<int64_t>(64, K - k0) * N));
    const __amdgpu_buffer_rsrc_t rg = make_rsrc(p.G + m0 * N, (uint32_t)(2 * min<int64_t>(16 * MB, M - m0) * N));
    const int lrow = lane / kCPR, lchunk = lane % kCPR; // this lane's row and chunk within an instruction
    auto issue = [&](int j) { // chunk j into slot j % kS
        const int64_t c0 = n_beg + (int64_t)j * kCH;
        LDS char *slot = smem + (j % kS) * kSlot;
#pragma unroll
        for (int i = 0; i < kWInst; ++i) {
            const int r = 16 * w + kRPI * i + lrow;
            const int64_t n = c0 + 8 * (lchunk ^ (r & 15));
            const bool ok = k0 + r < K && n < n_end;
            dma16_nt(rw, slot + (16 * w + kRPI * i) * kRow, ok ? (uint32_t)(2 * (r * N + n)) : kOOB);
        }
#pragma unroll
        for (int i = 0; i < kGInst; ++i) {
            const int mr = kRPI * (w * kGInst + i);
            const int m = mr + lrow;
            const int64_t n = c0 + 8 * (lchunk ^ (m & 15));
            const bool ok = m0 + m < M && n < n_end;
            dma16(rg, slot + kWSlot + mr * kRow, ok ? (uint32_t)(2 * (m * N + n)) : kOOB);
        }
    };

    // Fragment layout.  MB <= 4: wave w owns dX columns k0+16w .. +15 and all
    // M rows (one W fragment and MB dY fragments per 32-deep step, MB MFMAs).
    // MB >= 8: wave w owns row blocks w*MW .. +MW-1 and all 64 columns (four W
    // fragments and MW dY fragments per step, 4*MW MFMAs): with one column
    // block per wave every MFMA would need a fresh dY fragment, more LDS
    // traffic than the LDS delivers.
    constexpr bool kWide = MB >= 8;
    constexpr int MW = kWide ? MB / 4 : MB; // dY fragments per step
    constexpr int XW = kWide ? 4 : 1;       // W fragments per step
    f32x4_t acc[MW][XW];
#pragma unroll
    for (int j = 0; j < MW; ++j)
#pragma unroll
        for (int x = 0; x < XW; ++x)
            acc[j][x] = f32x4_t{};
    const int sw = lane & 15; // row % 16 of every fragment row this lane reads
    // chunk j: wait for its DMA, barrier (after which every wave is done with
    // chunk j-1, so its slot takes chunk j + kS - 1), then its MFMA steps
    for (int i = 0; i < kS - 1 && i < nc; ++i)
        issue(i);
    for (int jc = 0; jc < nc; ++jc) {
        dx_chunk_wait<kPerChunk>(min(kS - 2, nc - 1 - jc));
        slab_barrier();
        if (jc + kS - 1 < nc)
            issue(jc + kS - 1);
        const LDS char *slot = smem + (jc % kS) * kSlot;
#pragma unroll
        for (int u = 0; u < kCH / 32; ++u) {
            const int c = 4 * u + (lane >> 4);
            bf16x8_t wf[XW], gf[MW];
#pragma unroll
            for (int x = 0; x < XW; ++x)
                wf[x] = read_rc<0>(slot + (16 * (kWide ? x : w) + sw) * kRow + ((c ^ sw) << 4));
#pragma unroll
            for (int j = 0; j < MW; ++j)
                gf[j] = read_rc<0>(slot + kWSlot + (16 * (kWide ? w * MW + j : j) + sw) * kRow + ((c ^ sw) << 4));
            lgkm_wait_wg<XW, MW>(wf, gf);
            // lane l: dX[row block's 16 rows: l%16][column block's 16: 4(l/16) .. +3]
#pragma unroll
            for (int j = 0; j < MW; ++j)
#pragma unroll
                for (int x = 0; x < XW; ++x)
                    acc[j][x] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[x], gf[j], acc[j][x], 0, 0, 0);
        }
    }
#pragma unroll
    for (int j = 0; j < MW; ++j)
#pragma unroll
        for (int x = 0; x < XW; ++x) {
            const int64_t m = m0 + 16 * (kWide ? w * MW + j : j) + (lane & 15);
            const int64_t k = k0 + 16 * (kWide ? x : w) + 4 * (lane >> 4);
            if (m >= M || k >= K) // K % 8 == 0: k .. k+3 all in range
                continue;
            if (p.splits == 1) {
                const u32x2_t pk = {pack_bf16x2(acc[j][x][0], acc[j][x][1]), pack_bf16x2(acc[j][x][2], acc[j][x][3])};
                *reinterpret_cast<u32x2_t *>(p.dX + m * K + k) = pk;
            } else {
                *reinterpret_cast<f32x4_t *>(p.part + ((int64_t)s * M + m) * K + k) = acc[j][x];
            }
        }
}

// dX = bf16(Σ_s part[s]) over the splits in order (splits <= kDxsMaxSplits)
// for entries 4i .. 4i+3 (M*K % 8 == 0), all loads issued at once.  Run by the
// first blocks of the dW kernel that follows the dX kernel on the stream (its
// write stream hides the reads), or, without dW, by a kernel of its own.
constexpr int kDxsMaxSplits = 16;
__device__ __forceinline__ void dx_reduce_quad(const SmallParams &p, int64_t q) {
    const int64_t MK = p.M * p.K;
    const int64_t i = 4 * q;
    if (i >= MK)
        return;
    f32x4_t v[kDxsMaxSplits];
#pragma unroll
    for (int t = 0; t < kDxsMaxSplits; ++t)
        v[t] = t < p.splits ? *reinterpret_cast<const f32x4_t *>(p.part + t * MK + i) : f32x4_t{};
    f32x4_t a = v[0];
#pragma unroll
    for (int t = 1; t < kDxsMaxSplits; ++t)
        if (t < p.splits)
            a += v[t];
    const u32x2_t pk = {pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3])};
    *reinterpret_cast<u32x2_t *>(p.dX + i) = pk;
}

__global__ __launch_bounds__(256) void k_dx_smallm_reduce(SmallParams p) {
    dx_reduce_quad(p, (int64_t)blockIdx.x * 256 + threadIdx.x);
}

template <int MB>
__global__ __launch_bounds__(256) void k_dx_smallm(SmallParams p) {
    __shared__ __attribute__((aligned(1024))) char smem_raw[dx_small_lds<MB>()];
    dx_small_block<MB>(p, blockIdx.x, (LDS char *)smem_raw);
}

// dX for M <= 16 on small calls (plan::rows16_fits) without split partials,
// so without the launch that sums them: block b owns dX columns k0 = 16b ..
// +15 over the whole reduction, and wave w takes the w-th quarter of n in
// chunks of 128: W's 16 rows come by DMA through a ring of its own (four
// slots of 16 rows x 256 bytes; 16-byte chunk c of row r at chunk c ^ r),
// dY's fragments straight from memory into registers three chunks ahead (dY
// is at most 16 rows and stays in the caches).  Every chunk is issued, the
// ones past the wave's range reading zero, so the loop has no branches and
// one wait count.  The four waves' sums are added in wave order through LDS.
// 64 KiB of LDS: two blocks per CU, beside dW's blocks in k_smallm_pair16.
constexpr int kR16CH = 128, kR16Row = 256, kR16S = 4, kR16Slot = 16 * kR16Row;
constexpr int kR16Lds = 4 * kR16S * kR16Slot;

__device__ __forceinline__ bf16x8_t load16(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
    return __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off, 0, 0));
}

__device__ __forceinline__ void dx_rows16_block(const SmallParams &p, int b, LDS char *smem) {
    constexpr int kPer = 4 + 4; // per chunk: 4 DMA instructions (4 rows x 256 B each), 4 fragment loads
    static_assert((kR16S - 1) * kPer <= 63, "the chunks in flight fit the vmcnt counter");
    const int64_t M = p.M, K = p.K, N = p.N;
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t k0 = (int64_t)b * 16;
    const int64_t qn = ((N + 3) / 4 + kR16CH - 1) / kR16CH * kR16CH;
    const int64_t n_beg = min(N, (int64_t)w * qn), n_end = min(N, n_beg + qn);
    const int nc = (int)((n_end - n_beg + kR16CH - 1) / kR16CH);
    const int nc4 = (nc + kR16S - 1) / kR16S * kR16S;
    LDS char *const ring = smem + w * (kR16S * kR16Slot);
    // windows: the block's 16 rows of W, all of dY (2MN < 2^31); out-of-range
    // rows and columns read zero through the window or kOOB
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(p.W + k0 * N, (uint32_t)(2 * min<int64_t>(16, K - k0) * N));
    const __amdgpu_buffer_rsrc_t rg = make_rsrc(p.G, (uint32_t)(2 * M * N));
    const int drow = lane >> 4, dchunk = lane & 15; // DMA: row within the instruction, LDS chunk
    const int sw = lane & 15, q4 = lane >> 4;       // fragments: row, 8-element group
    bf16x8_t gbuf[kR16S][4];
    f32x4_t acc = f32x4_t{};
    auto issue = [&](int j, auto slc) __attribute__((always_inline)) {
        constexpr int SL = decltype(slc)::value;
        const int64_t c0 = n_beg + (int64_t)j * kR16CH;
        LDS char *slot = ring + SL * kR16Slot;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * i + drow;
            const int64_t n = c0 + 8 * (dchunk ^ r);
            dma16_nt(rw, slot + i * 1024, oob_unless(k0 + r < K && n < n_end, (uint32_t)(2 * (r * N + n))));
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t n = c0 + 32 * u + 8 * q4;
            gbuf[SL][u] = load16(rg, oob_unless(sw < M && n < n_end, (uint32_t)(2 * (sw * N + n))));
        }
    };
    // chunk j from slot SL, after issuing chunk j + 3 into the slot chunk j - 1 used
    auto step = [&](int j, auto slc) __attribute__((always_inline)) {
        constexpr int SL = decltype(slc)::value;
        issue(j + kR16S - 1, std::integral_constant<int, (SL + kR16S - 1) % kR16S>{});
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"((kR16S - 1) * kPer) : "memory");
        const LDS char *slot = ring + SL * kR16Slot;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            bf16x8_t wf[1], gf[1];
            wf[0] = read_rc<0>(slot + sw * kR16Row + (((4 * u + q4) ^ sw) << 4));
            gf[0] = gbuf[SL][u];
            lgkm_wait_wg<1, 1>(wf, gf);
            // lane l: dX[m = l%16][k0 + 4(l/16) .. +3]
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[0], gf[0], acc, 0, 0, 0);
        }
    };
    issue(0, std::integral_constant<int, 0>{});
    issue(1, std::integral_constant<int, 1>{});
    issue(2, std::integral_constant<int, 2>{});
    for (int jc = 0; jc < nc4; jc += kR16S) {
        step(jc, std::integral_constant<int, 0>{});
        step(jc + 1, std::integral_constant<int, 1>{});
        step(jc + 2, std::integral_constant<int, 2>{});
        step(jc + 3, std::integral_constant<int, 3>{});
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); // the last (zero-reading) DMA into the ring too
    LDS f32x4_t *const sums = (LDS f32x4_t *)smem;
    __syncthreads(); // every wave is done with its ring
    sums[w * 64 + lane] = acc;
    __syncthreads();
    if (w != 0)
        return;
    f32x4_t t = sums[lane];
#pragma unroll
    for (int v = 1; v < 4; ++v)
        t += sums[v * 64 + lane];
    const int64_t k = k0 + 4 * q4; // K % 8 == 0: k .. k+3 all in range or all out
    if (sw < M && k < K) {
        const u32x2_t pk = {pack_bf16x2(t[0], t[1]), pack_bf16x2(t[2], t[3])};
        *reinterpret_cast<u32x2_t *>(p.dX + sw * K + k) = pk;
    }
}

__global__ __launch_bounds__(256) void k_dx_rows16(SmallParams p) {
    __shared__ __attribute__((aligned(1024))) char smem_raw[kR16Lds];
    dx_rows16_block(p, blockIdx.x, (LDS char *)smem_raw);
}

// both products for the same calls: blocks below dx_blocks run dx_rows16_block,
// the rest k_dw_smallm's blocks (LDS: the larger of the two, two blocks per CU)
__global__ __launch_bounds__(256) void k_smallm_pair16(SmallParams p) {
    static_assert(kR16Lds <= 80 * 1024 && kDwsLds <= 80 * 1024, "two blocks fit a CU's LDS");
    __shared__ __attribute__((aligned(1024))) char smem_raw[kR16Lds > kDwsLds ? kR16Lds : kDwsLds];
    if ((int)blockIdx.x < p.dx_blocks)
        dx_rows16_block(p, blockIdx.x, (LDS char *)smem_raw);
    else
        dw_small_block(p, blockIdx.x - p.dx_blocks, (LDS char *)smem_raw);
}

// Both small-M products in one launch (where plan::pair_fits: M <= 64 and
// limits on N and K*N): blocks below dx_blocks run dX blocks
// with a ring of 128-element chunks, the rest dW blocks.  At 128 elements a
// dX block needs at most 72 KiB of LDS (96 would leave no room beside it;
// MB = 4 keeps two slots, 64 KiB), so every CU holds two blocks of either
// kind: the dX blocks' read stream of W and the dW blocks' write stream of
// fp32 dW overlap, and the launch boundary between them goes.  Each block computes what it computes in k_dx_smallm /
// k_dw_smallm, in the same order, so results are the same bits; dX's split
// partials are added afterwards by k_dx_smallm_reduce.
template <int MB, int CH, int S>
__global__ __launch_bounds__(256) void k_smallm_pair(SmallParams p) {
    constexpr int kDx = dx_small_lds<MB, CH, S>();
    static_assert(kDx <= 80 * 1024 && kDwsLds <= 80 * 1024, "two blocks fit a CU's LDS");
    __shared__ __attribute__((aligned(1024))) char smem_raw[kDx > kDwsLds ? kDx : kDwsLds];
    if ((int)blockIdx.x < p.dx_blocks)
        dx_small_block<MB, CH, S>(p, blockIdx.x, (LDS char *)smem_raw);
    else
        dw_small_block(p, blockIdx.x - p.dx_blocks, (LDS char *)smem_raw);
}

// dW blocks; with reduce_blocks > 0 the first reduce_blocks blocks also finish
// the preceding dX launch's split reduction, 1024 entries each.
__global__ __launch_bounds__(256) void k_dw_smallm(SmallParams p) {
    __shared__ __attribute__((aligned(1024))) char smem_raw[kDwsLds];
    if ((int)blockIdx.x < p.reduce_blocks) {
        dx_reduce_quad(p, (int64_t)blockIdx.x * 256 + threadIdx.x);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); // the slab waits below count DMA only
    }
    dw_small_block(p, blockIdx.x, (LDS char *)smem_raw);
}

// ------------------------------------------------------------------------
// M <= 64: both products in one launch (LB_PATH_FUSED_SMALL_M; not chosen
// automatically, see launch_lin_bwd).  dX[m, k] needs row k of W over the
// whole reduction, and dW[k, :] is written row by row, so block (row group,
// split) owns 16 rows k0 .. k0+15: it streams those rows of W once (2N bytes
// each, non-temporal: read once) together with dY (shared by all blocks, from
// the caches), accumulates dX[0:M, k0:k0+16] over its part of the reduction
// and writes dW[k0:k0+16, its columns] chunk by chunk.  The W read stream and
// the dW write stream (4N bytes per row) then overlap on every CU, where two
// launches in turn ran them one after the other.  With one split (K >= 4096
// gives 256 such blocks) dX needs no partial sums; with more, the fp32
// partials go to part[s][m][k] and are added in split order by
// k_dx_smallm_reduce.
//
// Per chunk of 256 reduction columns n (a ring of kRsSlots slots in LDS, all
// by DMA: W[k0:k0+16, chunk] and dY[0:16MB, chunk], 512 B per row):
//   dX: wave w takes the chunk's 32-deep steps 2w, 2w+1 (one W fragment, MB
//       dY fragments, MB MFMAs each); the four waves' sums are added in wave
//       order at the end.
//   dW: wave w takes the chunk's 16-column blocks 4w .. 4w+3: one MFMA per
//       block and 32 rows of M (the X fragments are read once per block),
//       passes the 16 x 64 fp32 result through 4 KiB of LDS of its own and
//       stores four 4-row x 256-byte segments.
// The waits count the wave's vector-memory operations (DMA and stores, which
// the counter retires in issue order) issued after the chunk's DMA, so a
// chunk's stores never wait for later DMA and vice versa.  All LDS accesses in
// the loop are inline asm: the compiler would otherwise treat them as aliasing
// the DMA in flight and wait for all of it.
constexpr int kRsRows = 16;                  // W / dW rows per block
constexpr int kRsCH = 256;                   // reduction columns per chunk
constexpr int kRsRowBytes = kRsCH * 2;       // 512 B per LDS row
constexpr int kRsWBytes = kRsRows * kRsRowBytes;
constexpr int kRsXBytes = 4096;              // X[0:128, k0:k0+16], 32 B per row
constexpr int kRsStage = 4096;               // per wave: 16 rows x 64 fp32
template <int MB> constexpr int rs_slot() { return kRsWBytes + 16 * MB * kRsRowBytes; }
template <int MB> constexpr int rs_slots() { return MB >= 4 ? 3 : 5; }
template <int MB> constexpr int rs_ring() { return rs_slots<MB>() * rs_slot<MB>(); }
template <int MB> constexpr int rs_lds() { return rs_ring<MB>() + kRsXBytes + 4 * kRsStage; }
constexpr int kRsMaxM = 64;

// 16-byte chunk c of LDS row r sits at c ^ rs_swz(r): the 16 rows a fragment
// row read serves hit 16 different bank groups, and the rows {0..3, 8..11}
// (or {4..7, 12..15}) that half a transposing read serves hit 8 different
// 32-byte segments.
__device__ __forceinline__ int rs_swz(int r) { return (((r & 3) | (((r >> 3) & 1) << 2)) << 1) | ((r >> 2) & 1); }
__device__ __forceinline__ int rs_off(int r, int c) { return r * kRsRowBytes + ((c ^ rs_swz(r)) << 4); }

// s_waitcnt vmcnt(n) for a run-time n (clamped to 63: waiting longer is safe)
__device__ __forceinline__ void vm_wait(int n) {
    switch (n > 63 ? 63 : n) {
#define LB_VMW(i)                                              \
    case i: asm volatile("s_waitcnt vmcnt(" #i ")" ::: "memory"); break;
    LB_VMW(0) LB_VMW(1) LB_VMW(2) LB_VMW(3) LB_VMW(4) LB_VMW(5) LB_VMW(6) LB_VMW(7)
    LB_VMW(8) LB_VMW(9) LB_VMW(10) LB_VMW(11) LB_VMW(12) LB_VMW(13) LB_VMW(14) LB_VMW(15)
    LB_VMW(16) LB_VMW(17) LB_VMW(18) LB_VMW(19) LB_VMW(20) LB_VMW(21) LB_VMW(22) LB_VMW(23)
    LB_VMW(24) LB_VMW(25) LB_VMW(26) LB_VMW(27) LB_VMW(28) LB_VMW(29) LB_VMW(30) LB_VMW(31)
    LB_VMW(32) LB_VMW(33) LB_VMW(34) LB_VMW(35) LB_VMW(36) LB_VMW(37) LB_VMW(38) LB_VMW(39)
    LB_VMW(40) LB_VMW(41) LB_VMW(42) LB_VMW(43) LB_VMW(44) LB_VMW(45) LB_VMW(46) LB_VMW(47)
    LB_VMW(48) LB_VMW(49) LB_VMW(50) LB_VMW(51) LB_VMW(52) LB_VMW(53) LB_VMW(54) LB_VMW(55)
    LB_VMW(56) LB_VMW(57) LB_VMW(58) LB_VMW(59) LB_VMW(60) LB_VMW(61) LB_VMW(62)
    default: asm volatile("s_waitcnt vmcnt(63)" ::: "memory"); break;
#undef LB_VMW
    }
}

__device__ __forceinline__ void lds_write16(LDS char *p, const f32x4_t &v) {
    asm volatile("ds_write_b128 %0, %1" ::"v"(p), "v"(v) : "memory");
}
__device__ __forceinline__ f32x4_t lds_read16(const LDS char *p) {
    f32x4_t v;
    asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(p));
    return v;
}
template <int N>
__device__ __forceinline__ void lgkm_wait_f(f32x4_t (&v)[N]) {
    static_assert(N == 4, "four staged quads per round");
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3])::"memory");
}
template <int MW>
__device__ __forceinline__ void lgkm_wait_tr_n(bf16x4_t (&t)[MW][2]) {
    if constexpr (MW == 1)
        asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(t[0][0]), "+v"(t[0][1])::"memory");
    else
        asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(t[0][0]), "+v"(t[0][1]), "+v"(t[1][0]), "+v"(t[1][1])::"memory");
}
// Wait until at most N of this wave's LDS reads are in flight, with the two
// dX steps' fragments (or two column blocks' transposed halves) threaded
// through the asm so that no MFMA that reads them moves above the wait.
template <int MB, int N>
__device__ __forceinline__ void rs_wait_dx(bf16x8_t (&w)[2], bf16x8_t (&g)[2][MB]) {
    static_assert(N <= 15, "lgkmcnt is a 4-bit counter");
    if constexpr (MB == 2)
        asm volatile("s_waitcnt lgkmcnt(%[n])"
                     : "+v"(w[0]), "+v"(w[1]), "+v"(g[0][0]), "+v"(g[0][1]), "+v"(g[1][0]), "+v"(g[1][1])
                     : [n] "n"(N)
                     : "memory");
    else
        asm volatile("s_waitcnt lgkmcnt(%[n])"
                     : "+v"(w[0]), "+v"(w[1]), "+v"(g[0][0]), "+v"(g[0][1]), "+v"(g[0][2]), "+v"(g[0][3]),
                       "+v"(g[1][0]), "+v"(g[1][1]), "+v"(g[1][2]), "+v"(g[1][3])
                     : [n] "n"(N)
                     : "memory");
}
template <int MW, int N>
__device__ __forceinline__ void rs_wait_tr(bf16x4_t (&a)[MW][2], bf16x4_t (&b)[MW][2]) {
    static_assert(N <= 15, "lgkmcnt is a 4-bit counter");
    if constexpr (MW == 1)
        asm volatile("s_waitcnt lgkmcnt(%[n])"
                     : "+v"(a[0][0]), "+v"(a[0][1]), "+v"(b[0][0]), "+v"(b[0][1])
                     : [n] "n"(N)
                     : "memory");
    else
        asm volatile("s_waitcnt lgkmcnt(%[n])"
                     : "+v"(a[0][0]), "+v"(a[0][1]), "+v"(a[1][0]), "+v"(a[1][1]), "+v"(b[0][0]), "+v"(b[0][1]),
                       "+v"(b[1][0]), "+v"(b[1][1])
                     : [n] "n"(N)
                     : "memory");
}

struct FusedParams {
    const uint16_t *X, *W, *G; // X[M,K], W[K,N], dY[M,N]
    uint16_t *dX;              // [M,K] bf16
    float *dW;                 // [K,N] fp32
    float *part;               // split partials [splits][M][K] (splits > 1)
    int64_t M, K, N;
    int64_t split_len;         // reduction columns per split (a multiple of kRsCH)
    int splits;
};

template <int MB>
__device__ __forceinline__ void fused_small_block(const FusedParams &p, int b, LDS char *smem) {
    // the dW reduction reads dY in 32-row steps: the slot holds at least 32 rows
    static_assert(MB == 2 || MB == 4, "16 MB rows of dY per slot, 32 or 64");
    constexpr int kS = rs_slots<MB>();
    constexpr int kSlot = rs_slot<MB>();
    constexpr int kMW = MB >= 4 ? 2 : 1;      // 32-row steps of the dW reduction over m
    constexpr int kWInst = kRsWBytes / 1024 / 4;          // W DMA instructions per wave per chunk
    constexpr int kGInst = 16 * MB * kRsRowBytes / 1024 / 4; // dY DMA instructions per wave per chunk
    constexpr int kPerChunk = kWInst + kGInst;
    const int64_t M = p.M, K = p.K, N = p.N;
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int s = b % p.splits;
    const int64_t k0 = (int64_t)(b / p.splits) * kRsRows;
    const int64_t n_beg = (int64_t)s * p.split_len;
    const int64_t n_end = min(N, n_beg + p.split_len);
    const int nc = (int)((n_end - n_beg + kRsCH - 1) / kRsCH);
    LDS char *const xs = smem + rs_ring<MB>();
    LDS char *const stage = xs + kRsXBytes + w * kRsStage;

    // offsets are 32-bit (16 rows of W, and 2MN, 2MK < 2^31); rows or columns out of range read zero
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(p.W + k0 * N, (uint32_t)(2 * min<int64_t>(kRsRows, K - k0) * N));
    const __amdgpu_buffer_rsrc_t rg = make_rsrc(p.G, (uint32_t)(2 * M * N));
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(p.X, (uint32_t)(2 * M * K));
    // dW rows k0 .. k0+15 (a 64N-byte window, so 32-bit offsets); rows past K
    // lie past the descriptor's size and are not written
    const __amdgpu_buffer_rsrc_t rdw = make_rsrc(p.dW + k0 * N, (uint32_t)(4 * min<int64_t>(kRsRows, K - k0) * N));
    auto issue = [&](int j) { // chunk j into slot j % kS
        LDS char *slot = smem + (j % kS) * kSlot;
        const int64_t c0 = n_beg + (int64_t)j * kRsCH;
#pragma unroll
        for (int i = 0; i < kWInst; ++i) {
            const int q = w * kWInst + i; // 1 KiB = LDS rows 2q, 2q+1
            const int r = 2 * q + (lane >> 5);
            const int64_t n = c0 + 8 * ((lane & 31) ^ rs_swz(r));
            const bool ok = k0 + r < K && n < n_end;
            dma16_nt(rw, slot + q * 1024, oob_unless(ok, (uint32_t)(2 * (r * N + n))));
        }
#pragma unroll
        for (int i = 0; i < kGInst; ++i) {
            const int q = w * kGInst + i;
            const int r = 2 * q + (lane >> 5);
            const int64_t n = c0 + 8 * ((lane & 31) ^ rs_swz(r));
            const bool ok = r < M && n < n_end;
            dma16(rg, slot + kRsWBytes + q * 1024, oob_unless(ok, (uint32_t)(2 * (r * N + n))));
        }
    };
    {   // X[0:M, k0:k0+16]: wave w's instruction covers rows 32w .. 32w+31
        const int r = 32 * w + (lane >> 1);
        const int64_t k = k0 + 8 * (lane & 1);
        dma16(rx, xs + w * 1024, oob_unless(r < M && k < K, (uint32_t)(2 * (r * K + k))));
    }
    for (int j = 0; j < kS - 1 && j < nc; ++j)
        issue(j);

    f32x4_t accx[MB];
#pragma unroll
    for (int j = 0; j < MB; ++j)
        accx[j] = f32x4_t{};
    bf16x8_t xf[kMW];
    const int g = lane >> 4, sl = lane & 15;
    for (int jc = 0; jc < nc; ++jc) {
        // issued after chunk jc's DMA: the DMA of chunks jc+1 .. jc+kS-2 (those
        // that exist) and the stores of the last min(jc, kS-1) chunks
        vm_wait(kPerChunk * max(0, min(jc + kS - 2, nc - 1) - jc) + 4 * min(jc, kS - 1));
        slab_barrier(); // every wave's DMA of chunk jc landed; chunk jc-1's slot is free
        if (jc + kS - 1 < nc)
            issue(jc + kS - 1);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        const LDS char *slot = smem + (jc % kS) * kSlot;
        const LDS char *gs = slot + kRsWBytes;
        if (jc == 0) { // the X fragments (A side of dW), rows 32rr + 8g .. +7, column k0 + sl
#pragma unroll
            for (int rr = 0; rr < kMW; ++rr) {
                const int row = 32 * rr + 8 * g + (sl >> 2);
                const bf16x4_t lo = read_tr<0>(xs + row * 32 + 8 * (sl & 3));
                const bf16x4_t hi = read_tr<0>(xs + (row + 4) * 32 + 8 * (sl & 3));
                xf[rr] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            }
        }
        // All of the chunk's fragment reads go out first, in the order they are
        // used (LDS reads return in order): dX's, then dW's for column blocks
        // 0, 1, then 2, 3 of the wave; each group of MFMAs waits only for its own.
        // dX: steps 2w, 2w+1 (32 columns each); lane: dX[16j + l%16][k0 + 4(l/16) .. +3]
        bf16x8_t wf[2], gf[2][MB];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int c = 4 * (2 * w + u) + g; // this lane's 16-byte chunk of the step
            wf[u] = read_rc<0>(slot + rs_off(sl, c));
#pragma unroll
            for (int j = 0; j < MB; ++j)
                gf[u][j] = read_rc<0>(gs + rs_off(16 * j + sl, c));
        }
        // dW: column blocks 4w .. 4w+3; lane: dW[k0 + l%16][16nb + 4(l/16) .. +3]
        bf16x4_t tr[4][kMW][2];
        auto read_w = [&](int t) {
            const int col = 16 * (4 * w + t) + 4 * (sl & 3);
#pragma unroll
            for (int rr = 0; rr < kMW; ++rr)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int row = 32 * rr + 8 * g + 4 * h + (sl >> 2);
                    tr[t][rr][h] = read_tr<0>(gs + rs_off(row, col >> 3) + (col & 7) * 2);
                }
        };
        read_w(0);
        read_w(1);
        rs_wait_dx<MB, 4 * kMW>(wf, gf); // all but the 2 x 2 kMW reads of blocks 0, 1
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int j = 0; j < MB; ++j)
                accx[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[u], gf[u][j], accx[j], 0, 0, 0);
        read_w(2);
        read_w(3);
        f32x4_t accw[4];
        auto mfma_w = [&](int t) {
            accw[t] = f32x4_t{};
#pragma unroll
            for (int rr = 0; rr < kMW; ++rr)
                accw[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_shufflevector(tr[t][rr][0], tr[t][rr][1], 0, 1, 2, 3, 4, 5, 6, 7), xf[rr], accw[t], 0, 0,
                    0);
        };
        rs_wait_tr<kMW, 4 * kMW>(tr[0], tr[1]); // blocks 0, 1 landed; 2, 3 may be in flight
        mfma_w(0);
        mfma_w(1);
        rs_wait_tr<kMW, 0>(tr[2], tr[3]);
        mfma_w(2);
        mfma_w(3);
        // through the wave's staging area: row k (16), 16-byte chunk c at c ^ k
#pragma unroll
        for (int t = 0; t < 4; ++t)
            lds_write16(stage + sl * 256 + (((4 * t + g) ^ sl) << 4), accw[t]);
        f32x4_t v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int r = 4 * u + g;
            v[u] = lds_read16(stage + r * 256 + ((sl ^ r) << 4));
        }
        lgkm_wait_f(v);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        const int64_t nb0 = n_beg + (int64_t)jc * kRsCH + 64 * w + 4 * sl;
#pragma unroll
        for (int u = 0; u < 4; ++u) // N % 8 == 0: nb0 .. nb0+3 all in range
            store_out(rdw, oob_unless(nb0 < n_end, (uint32_t)(4 * ((4 * u + g) * N + nb0))), v[u]);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
    }
    // dX: the four waves' partial sums, added in wave order; the ring is reused
    // once every DMA has landed and every wave is past the loop
    vm_wait(0);
    slab_barrier();
    LDS float *red = reinterpret_cast<LDS float *>(smem);
    constexpr int M16 = 16 * MB;
#pragma unroll
    for (int j = 0; j < MB; ++j)
        *reinterpret_cast<LDS f32x4_t *>(red + ((w * M16 + 16 * j + sl) * 16 + 4 * g)) = accx[j];
    __syncthreads();
    const int t = threadIdx.x;
    if (t < M16 * 4) {
        const int m = t >> 2, kq = t & 3;
        f32x4_t a = *reinterpret_cast<const LDS f32x4_t *>(red + (m * 16 + 4 * kq));
#pragma unroll
        for (int ww = 1; ww < 4; ++ww)
            a += *reinterpret_cast<const LDS f32x4_t *>(red + ((ww * M16 + m) * 16 + 4 * kq));
        const int64_t k = k0 + 4 * kq;
        if (m < M && k < K) { // K % 8 == 0: k .. k+3 all in range
            if (p.splits == 1) {
                const u32x2_t pk = {pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3])};
                *reinterpret_cast<u32x2_t *>(p.dX + m * K + k) = pk;
            } else {
                *reinterpret_cast<f32x4_t *>(p.part + ((int64_t)s * M + m) * K + k) = a;
            }
        }
    }
}

template <int MB>
__global__ __launch_bounds__(256, 1) void k_lin_bwd_fused_small(FusedParams p) {
    static_assert(rs_lds<MB>() <= 160 * 1024, "LDS");
    static_assert(4 * 16 * MB * 16 * 4 <= rs_ring<MB>(), "the dX sums fit in the ring");
    __shared__ __attribute__((aligned(1024))) char smem_raw[rs_lds<MB>()];
    fused_small_block<MB>(p, blockIdx.x, (LDS char *)smem_raw);
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
// Ragged or unaligned bf16 operands
// ------------------------------------------------------------------------
// The MFMA kernels read rows in 16-byte chunks, so K and N must be multiples
// of 8 and the pointers 16-byte aligned.  Other bf16 calls run on zero-padded
// copies: the padded problem (M, K8, N8) has the same sums (zero columns add
// nothing), its extra output rows and columns are dropped when dX and dW are
// copied back.  k_repack copies a row-major matrix into another with a
// different row length, writing zero where the source has no entry.  A thread
// moves 16 bytes of one destination row: its source elements are loaded one
// by one (a ragged source row has no 16-byte alignment) but all before any
// store, so each thread keeps 16 bytes of loads in flight; the store is one
// 16-byte vector when the destination rows allow it.  Grid: x over 16-byte
// chunks of a row, y over rows (a block-stride loop beyond 65535 rows).
template <typename T>
__global__ __launch_bounds__(256) void k_repack(const T *src, int64_t src_rows, int64_t src_cols, T *dst,
                                                int64_t dst_rows, int64_t dst_cols, bool dst_vec) {
    constexpr int V = 16 / sizeof(T);
    typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
    const int64_t c0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * V;
    if (c0 >= dst_cols)
        return;
    for (int64_t r = blockIdx.y; r < dst_rows; r += gridDim.y) {
        const T *s = src + r * src_cols;
        T *d = dst + r * dst_cols;
        T v[V];
#pragma unroll
        for (int j = 0; j < V; ++j)
            v[j] = r < src_rows && c0 + j < src_cols ? s[c0 + j] : T(0);
        if (dst_vec) { // dst_cols % V == 0 and dst 16-byte aligned: c0 .. c0+V-1 in range
            u32x4v q;
            __builtin_memcpy(&q, v, 16);
            *reinterpret_cast<u32x4v *>(d + c0) = q;
        } else {
#pragma unroll
            for (int j = 0; j < V; ++j)
                if (c0 + j < dst_cols)
                    d[c0 + j] = v[j];
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
    j.rot = 0;
    j.splits = 1;
    j.split_len = R;
    j.part = nullptr;
    return j;
}

// From this M on (up to kSmallMaxDxM), dX takes the tile kernel with a split
// reduction instead of the small-M kernel when the path is chosen
// automatically: there dW has left the small-tile kernel, and the split dX
// tiles share one launch with the dW tiles (measured at K = N = 4096, both
// products: M = 320 64.1 -> 49.2 us, 512 69.2 -> 57.6, 768 105.0 -> 78.2,
// 1024 101.4 -> 82.7; M = 1024, K = 16384 377.8 -> 251.9).  At M <= 256 the
// split tiles were no faster than the small-M kernel for dX alone, and slower
// with K = 16384 (75.9 vs 66.6 us at M = 256).
constexpr int64_t kTileSplitMinDxM = kSmallMaxM + 1;
// Below that, down to this M, both products take the tile kernel (one launch,
// dX split) when both are requested and K, N >= kTileBothMinKN: there the two
// small-M launches lost (tile / small-M, whole call: 0.82-1.00 on 11 seeded
// shapes with K, N >= 2048 between M = 145 and 254, e.g. M = 204, K = 12288,
// N = 16384 424.6 -> 350.1 us), while with K or N <= 1024, at M <= 128 or for
// one product alone the small-M kernels stayed as fast or faster (M = 128,
// K = N = 4096: 35.3 vs 42.3 us).
constexpr int64_t kTileBothMinM = 160;
constexpr int64_t kTileBothMinKN = 2048;

// The host-side sizing decisions (range counts, the launch-length model, the
// pair limits) live in dispatch.h; its constants must be the kernels'.
static_assert(plan::kCUs == kCUs && plan::kSlab == kBK && plan::kMaxSplits == kDxsMaxSplits,
              "dispatch.h sizes the kernels in this file");

// Which MFMA kernel can run which product.  Every kernel reads 16-byte chunks
// of bf16 rows (K and N multiples of 8, 16-byte aligned pointers) through
// buffer descriptors with 32-bit offsets, 2^31 and beyond meaning "out of
// range"; each descriptor covers only the rows its block reads (a tile's 256
// operand rows, a 32-row slab, a block's rows of W), so operands and outputs
// may be larger than 2 GiB as long as each such window stays below 2 GiB.
struct Eligible {
    bool tile_dx, tile_dw;   // the 256x256 tile kernel
    bool small_dx, small_dw; // split-reduction dX (M <= 1024), small-tile dW (M <= 256)
    bool fused;              // both products in one launch (M <= 64)
};

Eligible eligible(const LinBwdArgs &a, bool need_dx, bool need_dw) {
    const int64_t lim = (int64_t)1 << 31;
    const bool rows8 = a.bf16 && (a.K % 8 == 0) && (a.N % 8 == 0);
    // output windows: 32 rows of dX (2K bytes each), 16 of dW (4N); slabs of
    // 32 rows of X (2K) and dY (2N)
    const bool win = 64 * a.K < lim && 64 * a.N < lim;
    const bool dx_ok = rows8 && win && is_aligned16(a.dX) && (a.N == 0 || (is_aligned16(a.dY) && is_aligned16(a.W)));
    const bool dw_ok = rows8 && win && is_aligned16(a.dW) && (a.M == 0 || (is_aligned16(a.X) && is_aligned16(a.dY)));
    Eligible e;
    // dX reads 256 rows of dY or W (2N bytes each) per tile / row group
    e.tile_dx = dx_ok && 512 * a.N < lim;
    e.tile_dw = dw_ok;
    e.small_dx = e.tile_dx && a.M <= kSmallMaxDxM;
    // the small-tile dW kernel addresses X (M <= 256 rows) as a whole
    e.small_dw = dw_ok && a.M >= 1 && a.M <= kSmallMaxM && 2 * a.M * a.K < lim;
    // the fused kernel addresses X and dY (M <= 64 rows) as wholes
    e.fused = need_dx && need_dw && dx_ok && dw_ok && a.M >= 1 && a.M <= kRsMaxM && a.N > 0 &&
              2 * a.M * a.K < lim && 2 * a.M * a.N < lim;
    return e;
}

// Both products for M <= 64 in one launch (plus, with several splits of the
// reduction, the launch that adds the dX partials in split order).
hipError_t launch_fused_small(const LinBwdArgs &a, hipStream_t s) {
    FusedParams fp{};
    fp.X = static_cast<const uint16_t *>(a.X);
    fp.W = static_cast<const uint16_t *>(a.W);
    fp.G = static_cast<const uint16_t *>(a.dY);
    fp.dX = static_cast<uint16_t *>(a.dX);
    fp.dW = a.dW;
    fp.M = a.M;
    fp.K = a.K;
    fp.N = a.N;
    // splits of the reduction: toward 256 blocks (one per CU), each a whole
    // number of chunks, at most kDxsMaxSplits, partials within the workspace
    const int64_t rblocks = (a.K + kRsRows - 1) / kRsRows;
    const plan::Split sl = plan::reduction_split(
        a.N, kRsCH, rblocks, a.M, a.K, a.dx_partial ? std::min(a.dx_partial_floats, kSmallDxPartialFloats) : 0);
    const int64_t splits = sl.splits, split_len = sl.len;
    fp.split_len = split_len;
    fp.splits = (int)splits;
    fp.part = a.dx_partial;
    const int64_t blocks = rblocks * splits;
    if (blocks > 0x7fffffff)
        return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)blocks);
    if (a.M <= 32) // rows M .. 31 of the dY slot read zero
        hipLaunchKernelGGL(k_lin_bwd_fused_small<2>, grid, dim3(256), 0, s, fp);
    else
        hipLaunchKernelGGL(k_lin_bwd_fused_small<4>, grid, dim3(256), 0, s, fp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || splits == 1)
        return e;
    SmallParams sp{};
    sp.dX = fp.dX;
    sp.part = fp.part;
    sp.M = a.M;
    sp.K = a.K;
    sp.N = a.N;
    sp.splits = (int)splits;
    const int64_t quads = a.M * a.K / 4;
    hipLaunchKernelGGL(k_dx_smallm_reduce, dim3((unsigned)((quads + 255) / 256)), dim3(256), 0, s, sp);
    return hipGetLastError();
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

// Which buffers a bf16 call has to copy before the MFMA kernels can take it
// (none: it runs as it is).  K8, N8: K and N rounded up to multiples of 8.
struct Staging {
    bool any;
    bool g, w, x, dx, dw; // padded copies of dY [M,N8], W [K8,N8], X [M,K8]; dX [M,K8], dW [K8,N8]
    int64_t K8, N8;
};

Staging staging(const LinBwdArgs &a, bool need_dx, bool need_dw) {
    Staging st{};
    if (!a.bf16 || !a.may_stage || a.path == PATH_GENERAL || a.M <= 0 || a.K <= 0 || a.N <= 0 ||
        (!need_dx && !need_dw))
        return st;
    st.K8 = (a.K + 7) / 8 * 8;
    st.N8 = (a.N + 7) / 8 * 8;
    const bool kr = st.K8 != a.K, nr = st.N8 != a.N;
    st.g = nr || !is_aligned16(a.dY);
    st.w = need_dx && (kr || nr || !is_aligned16(a.W));
    st.x = need_dw && (kr || !is_aligned16(a.X));
    st.dx = need_dx && (kr || !is_aligned16(a.dX));
    st.dw = need_dw && (kr || nr || !is_aligned16(a.dW));
    st.any = st.g || st.w || st.x || st.dx || st.dw;
    return st;
}

// The padded call as the MFMA dispatch sees it; `base` holds the copies (with
// base == nullptr only the pointers' alignment is meaningful: for the checks).
LinBwdArgs padded_call(const LinBwdArgs &a, const Staging &st, bool need_dx, bool need_dw, char *base,
                       int64_t (&off)[5]) {
    char *const b = base ? base : reinterpret_cast<char *>(256);
    LinBwdArgs in = a;
    in.K = st.K8;
    in.N = st.N8;
    in.may_stage = false;
    in.dY = st.g ? b + off[0] : a.dY;
    in.W = st.w ? b + off[1] : a.W;
    in.X = st.x ? b + off[2] : a.X;
    in.dX = need_dx ? (st.dx ? b + off[3] : a.dX) : nullptr;
    in.dW = need_dw ? (st.dw ? reinterpret_cast<float *>(b + off[4]) : a.dW) : nullptr;
    return in;
}

// Byte offsets of the copies in one allocation (256-byte aligned); returns the total.
int64_t staging_layout(const LinBwdArgs &a, const Staging &st, int64_t (&off)[5]) {
    const int64_t bytes[5] = {st.g ? 2 * a.M * st.N8 : 0, st.w ? 2 * st.K8 * st.N8 : 0, st.x ? 2 * a.M * st.K8 : 0,
                              st.dx ? 2 * a.M * st.K8 : 0, st.dw ? 4 * st.K8 * st.N8 : 0};
    int64_t total = 0;
    for (int i = 0; i < 5; ++i) {
        off[i] = total;
        total += (bytes[i] + 255) / 256 * 256;
    }
    return total;
}

template <typename T>
hipError_t repack(const void *src, int64_t src_rows, int64_t src_cols, void *dst, int64_t dst_rows,
                  int64_t dst_cols, hipStream_t s) {
    constexpr int V = 16 / sizeof(T);
    const int64_t per_block = 256 * V;
    const dim3 grid((unsigned)((dst_cols + per_block - 1) / per_block), (unsigned)std::min<int64_t>(dst_rows, 65535));
    const bool vec = dst_cols % V == 0 && is_aligned16(dst);
    hipLaunchKernelGGL(k_repack<T>, grid, dim3(256), 0, s, static_cast<const T *>(src), src_rows, src_cols,
                       static_cast<T *>(dst), dst_rows, dst_cols, vec);
    return hipGetLastError();
}

hipError_t launch_lin_bwd_aligned(const LinBwdArgs &a, bool need_dx, bool need_dw, hipStream_t s);

// Pads, runs the padded call, copies dX / dW back; the copies live in one
// stream-ordered allocation from the library's pool, released behind the last
// kernel.  When that
// allocation fails, an automatic call takes the element-wise kernel instead
// and a forced path returns the error.
hipError_t launch_staged(const LinBwdArgs &a, const Staging &st, bool need_dx, bool need_dw, hipStream_t s) {
    int64_t off[5];
    const int64_t total = staging_layout(a, st, off);
    void *base = nullptr;
    hipMemPool_t pool = nullptr;
    hipError_t ea = staging_pool(&pool);
    if (ea == hipSuccess)
        ea = hipMallocFromPoolAsync(&base, (size_t)total, pool, s);
    if (ea == hipSuccess && !is_aligned16(base))
        ea = hipErrorInvalidValue;
    if (ea != hipSuccess) {
        if (base)
            (void)hipFreeAsync(base, s);
        (void)hipGetLastError();
        return a.path == PATH_AUTO ? launch_simt(a, need_dx, need_dw, s) : ea;
    }
    char *const b = static_cast<char *>(base);
    hipError_t e = hipSuccess;
    if (st.g)
        e = repack<uint16_t>(a.dY, a.M, a.N, b + off[0], a.M, st.N8, s);
    if (e == hipSuccess && st.w)
        e = repack<uint16_t>(a.W, a.K, a.N, b + off[1], st.K8, st.N8, s);
    if (e == hipSuccess && st.x)
        e = repack<uint16_t>(a.X, a.M, a.K, b + off[2], a.M, st.K8, s);
    const LinBwdArgs in = padded_call(a, st, need_dx, need_dw, b, off);
    if (e == hipSuccess)
        e = launch_lin_bwd_aligned(in, need_dx, need_dw, s);
    if (e == hipSuccess && st.dx)
        e = repack<uint16_t>(b + off[3], a.M, st.K8, a.dX, a.M, a.K, s);
    if (e == hipSuccess && st.dw)
        e = repack<float>(b + off[4], st.K8, st.N8, a.dW, a.K, a.N, s);
    const hipError_t ef = hipFreeAsync(base, s);
    return e != hipSuccess ? e : ef;
}

} // namespace

const char *lin_bwd_path_refusal(const LinBwdArgs &a) {
    if (a.path == PATH_AUTO || a.path == PATH_GENERAL)
        return nullptr;
    const bool need_dx = a.dX != nullptr && a.M > 0 && a.K > 0;
    const bool need_dw = a.dW != nullptr && a.K > 0 && a.N > 0;
    if (!need_dx && !need_dw)
        return nullptr;
    if (a.path != PATH_TILE && a.path != PATH_SMALL_M && a.path != PATH_FUSED_SMALL_M)
        return "unknown path";
    // a ragged or unaligned call runs padded: check the padded call
    const Staging st = staging(a, need_dx, need_dw);
    int64_t off[5] = {0, 0, 0, 0, 0};
    const Eligible e = st.any ? eligible(padded_call(a, st, need_dx, need_dw, nullptr, off), need_dx, need_dw)
                              : eligible(a, need_dx, need_dw);
    static const char *kNeed = "the MFMA kernels need bf16 operands (K and N multiples of 8 and 16-byte aligned "
                               "pointers, or a call that may copy its operands padded), K and N below 2^25 and, "
                               "for dX, N below 2^22";
    if (a.path == PATH_TILE && ((need_dx && !e.tile_dx) || (need_dw && !e.tile_dw)))
        return kNeed;
    if (a.path == PATH_SMALL_M) {
        if (need_dx && !e.small_dx)
            return a.M > kSmallMaxDxM ? "the small-M dX kernel takes M <= 1024" : kNeed;
        if (need_dw && !e.small_dw)
            return a.M > kSmallMaxM ? "the small-M dW kernel takes M <= 256" : kNeed;
    }
    if (a.path == PATH_FUSED_SMALL_M && !e.fused)
        return "the fused small-M kernel computes both products (dX and dW requested), with bf16 operands, "
               "K and N multiples of 8, 16-byte aligned pointers, 1 <= M <= 64 and N > 0";
    return nullptr;
}

hipError_t launch_lin_bwd(const LinBwdArgs &a, hipStream_t s) {
    const bool need_dx = a.dX != nullptr && a.M > 0 && a.K > 0;
    const bool need_dw = a.dW != nullptr && a.K > 0 && a.N > 0;
    if (!need_dx && !need_dw)
        return hipSuccess;
    if (a.path == PATH_GENERAL)
        return launch_simt(a, need_dx, need_dw, s);
    const Staging st = staging(a, need_dx, need_dw);
    if (st.any)
        return launch_staged(a, st, need_dx, need_dw, s);
    return launch_lin_bwd_aligned(a, need_dx, need_dw, s);
}

namespace {

hipError_t launch_lin_bwd_aligned(const LinBwdArgs &a, bool need_dx, bool need_dw, hipStream_t s) {
    // the fused small-M kernel runs when asked for: measured against the two
    // launches below it was 5% slower at K = N = 4096 (M = 1 .. 32) and 20-25%
    // slower with K or N = 16384; its one 140 KiB block per CU leaves each
    // chunk's LDS round trips and barrier unhidden
    const Eligible e = eligible(a, need_dx, need_dw);
    if (a.path == PATH_FUSED_SMALL_M && e.fused)
        return launch_fused_small(a, s);
    // per product: the small-M kernel (not for the empty sums, N = 0 for dX and
    // M = 0 for dW, which the tile kernel writes as zeros), else the tile
    // kernel, else the element-wise kernel.  From M = kTileSplitMinDxM on, dX
    // takes the tile kernel with its reduction split over several tiles (fp32
    // partials in the workspace) instead of the small-M kernel; from
    // kTileBothMinM with large K and N, both products do (both_tile).
    const bool both_tile = a.path == PATH_AUTO && need_dx && need_dw && a.dx_partial != nullptr &&
                           a.M >= kTileBothMinM && a.K >= kTileBothMinKN && a.N >= kTileBothMinKN &&
                           e.tile_dx && e.tile_dw;
    const bool small_ok = a.path != PATH_TILE && !both_tile;
    const bool small_dx = need_dx && a.N > 0 && small_ok && e.small_dx &&
                          !(a.path == PATH_AUTO && a.M >= kTileSplitMinDxM && a.dx_partial != nullptr);
    const bool small_dw = need_dw && small_ok && e.small_dw;
    const bool tile_dx = need_dx && !small_dx && e.tile_dx;
    const bool tile_dw = need_dw && !small_dw && e.tile_dw;
    const bool simt_dx = need_dx && !small_dx && !tile_dx;
    const bool simt_dw = need_dw && !small_dw && !tile_dw;
    if (simt_dx || simt_dw) {
        hipError_t e2 = launch_simt(a, simt_dx, simt_dw, s);
        if (e2 != hipSuccess)
            return e2;
    }
    MfmaParams p{};
    int nj = 0;
    TileJob jx{}, jw{};
    bool have_x = false, have_w = false;
    if (tile_dx) {
        jx = make_tile_job(JOB_DX, a.dY, a.W, a.dX, a.M, a.K, a.N, a.N, a.N);
        // Rows of both RC operands are 2N bytes apart.  When that is a multiple
        // of 32 KiB, the same k of every row maps to one small group of L2 sets:
        // the 32 tiles running together on an XCD (4 tile rows x 8 tile columns)
        // touch about 3072 such lines per slab pair, the sets hold about 2048,
        // and the tiles evict each other's lines.  Four groups of tiles (by tile
        // column) start 32 slabs apart: each group's lines fit and are shared
        // within the group (measured on 16384x4096x16384: dX 860 -> 1090 TFLOP/s
        // for a distinct start per tile, 1289 -> 1327 for the four groups over
        // that).  Other strides are left alone: there the lockstep order shares
        // lines in L2 best.
        if ((2 * a.N) % 32768 == 0)
            jx.rot = 32;
        have_x = true;
    }
    if (tile_dw) {
        jw = make_tile_job(JOB_DW, a.X, a.dY, a.dW, a.K, a.N, a.M, a.K, a.N);
        have_w = true;
    }
    if (have_x && a.dx_partial != nullptr && a.N > 0) {
        const int sx = plan::tile_dx_splits(a.M, a.K, jx.ntiles, jx.R, have_w ? jw.ntiles : 0, have_w ? jw.R : 0,
                                            a.dx_partial_floats);
        if (sx > 1) {
            const plan::Split sl = plan::tile_split_len(a.N, sx);
            jx.split_len = sl.len;
            jx.splits = (int)sl.splits;
            if ((int64_t)jx.splits * a.M * a.K > a.dx_partial_floats) // the ranges' partials must fit
                return hipErrorInvalidValue;
            jx.part = a.dx_partial;
            jx.ntiles *= jx.splits;
        }
    }
    // longest reduction first: those tiles start on the first wave of CUs
    if (have_x && have_w) {
        if (jw.R > (jx.splits > 1 ? jx.split_len : jx.R)) {
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
        if (have_x && jx.splits > 1)
            hipLaunchKernelGGL(k_lin_bwd_mfma_split, dim3((unsigned)blocks), dim3(kThreads), 0, s, p);
        else
            hipLaunchKernelGGL(k_lin_bwd_mfma, dim3((unsigned)blocks), dim3(kThreads), 0, s, p);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    // the dX partials of a split tile job are added (in range order) by the
    // small-M dW launch when there is one, else by a launch of their own
    const int tile_splits = have_x && jx.splits > 1 ? jx.splits : 1;
    if (small_dx || small_dw || tile_splits > 1) {
        SmallParams sp{};
        sp.X = static_cast<const uint16_t *>(a.X);
        sp.W = static_cast<const uint16_t *>(a.W);
        sp.G = static_cast<const uint16_t *>(a.dY);
        sp.dX = small_dx || tile_splits > 1 ? static_cast<uint16_t *>(a.dX) : nullptr;
        sp.dW = small_dw ? a.dW : nullptr;
        sp.M = a.M;
        sp.K = a.K;
        sp.N = a.N;
        sp.splits = tile_splits;
        sp.part = a.dx_partial;
        int64_t reduce_quads = tile_splits > 1 ? a.M * a.K / 4 : 0;
        if (small_dx) {
            // splits of the reduction: aim at ~256 blocks (one per CU; a block
            // streams its chunks through its ring), each split a whole number of
            // chunks, at most kDxsMaxSplits, partials within the workspace
            const int mb = a.M <= 16 ? 1 : a.M <= 32 ? 2 : a.M <= 64 ? 4 : a.M <= 128 ? 8 : 16;
            sp.mgroups = (int)((a.M + 16 * mb - 1) / (16 * mb)); // above 256 rows: groups of 256
            const int64_t chunk = mb <= 4 ? dx_small_chunk<4>() : dx_small_chunk<8>();
            const int64_t groups = (a.K + kDxsBK - 1) / kDxsBK;
            const plan::Split sl =
                plan::reduction_split(a.N, chunk, groups * sp.mgroups, a.M, a.K,
                                      a.dx_partial ? std::min(a.dx_partial_floats, kSmallDxPartialFloats) : 0);
            const int64_t splits = sl.splits, split_len = sl.len;
            sp.split_len = split_len;
            sp.splits = (int)splits;
            sp.part = a.dx_partial;
            const int64_t blocks = groups * sp.mgroups * splits;
            if (blocks > 0x7fffffff)
                return hipErrorInvalidConfiguration;
            if (plan::rows16_fits(a.M, a.K, a.N)) {
                // no split partials: dX alone, or dX and dW in one launch
                sp.splits = 1;
                sp.part = nullptr;
                sp.dx_blocks = (int)((a.K + 15) / 16);
                int64_t total = sp.dx_blocks;
                if (small_dw) {
                    sp.dw_tiles_n = ceil_div(a.N, kDwsBN);
                    total += (int64_t)sp.dw_tiles_n * ceil_div(a.K, kDwsBK);
                    hipLaunchKernelGGL(k_smallm_pair16, dim3((unsigned)total), dim3(256), 0, s, sp);
                } else {
                    hipLaunchKernelGGL(k_dx_rows16, dim3((unsigned)total), dim3(256), 0, s, sp);
                }
                return hipGetLastError();
            }
            if (small_dw && plan::pair_fits(a.M, a.K, a.N)) {
                // both products in one launch (mb <= 4); the dX split partials,
                // if any, are added by a launch of their own
                sp.dx_blocks = (int)blocks;
                sp.dw_tiles_n = ceil_div(a.N, kDwsBN);
                const int64_t total = blocks + (int64_t)sp.dw_tiles_n * ceil_div(a.K, kDwsBK);
                if (total > 0x7fffffff)
                    return hipErrorInvalidConfiguration;
                const dim3 g2((unsigned)total);
                switch (mb) {
                case 1: hipLaunchKernelGGL((k_smallm_pair<1, 128, 3>), g2, dim3(256), 0, s, sp); break;
                case 2: hipLaunchKernelGGL((k_smallm_pair<2, 128, 3>), g2, dim3(256), 0, s, sp); break;
                default: hipLaunchKernelGGL((k_smallm_pair<4, 128, 2>), g2, dim3(256), 0, s, sp); break;
                }
                hipError_t e = hipGetLastError();
                if (e != hipSuccess || splits == 1)
                    return e;
                hipLaunchKernelGGL(k_dx_smallm_reduce, dim3((unsigned)((a.M * a.K / 4 + 255) / 256)), dim3(256), 0, s, sp);
                return hipGetLastError();
            }
            const dim3 grid((unsigned)blocks);
            switch (mb) {
            case 1: hipLaunchKernelGGL(k_dx_smallm<1>, grid, dim3(256), 0, s, sp); break;
            case 2: hipLaunchKernelGGL(k_dx_smallm<2>, grid, dim3(256), 0, s, sp); break;
            case 4: hipLaunchKernelGGL(k_dx_smallm<4>, grid, dim3(256), 0, s, sp); break;
            case 8: hipLaunchKernelGGL(k_dx_smallm<8>, grid, dim3(256), 0, s, sp); break;
            default: hipLaunchKernelGGL(k_dx_smallm<16>, grid, dim3(256), 0, s, sp); break;
            }
            hipError_t e = hipGetLastError();
            if (e != hipSuccess)
                return e;
            if (splits > 1)
                reduce_quads = a.M * a.K / 4;
        }
        const int64_t reduce_blocks = (reduce_quads + 255) / 256;
        if (small_dw) {
            sp.dw_tiles_n = ceil_div(a.N, kDwsBN);
            const int64_t blocks = (int64_t)sp.dw_tiles_n * ceil_div(a.K, kDwsBK);
            if (blocks > 0x7fffffff)
                return hipErrorInvalidConfiguration;
            if (reduce_blocks <= blocks) { // else the reduction gets its own launch below
                sp.reduce_blocks = (int)reduce_blocks;
                reduce_quads = 0;
            }
            hipLaunchKernelGGL(k_dw_smallm, dim3((unsigned)blocks), dim3(256), 0, s, sp);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess)
                return e;
        }
        if (reduce_quads > 0) {
            hipLaunchKernelGGL(k_dx_smallm_reduce, dim3((unsigned)reduce_blocks), dim3(256), 0, s, sp);
            return hipGetLastError();
        }
        return hipSuccess;
    }
    return hipSuccess;
}

} // namespace
} // namespace lb
