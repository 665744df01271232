// Host-side sizing decisions of the lin_bwd launchers: how many ranges a
// reduction is split into, and when the two small-M products share a launch.
// Pure integer arithmetic with no HIP dependency, so that the decisions can be
// built and checked on a host without a GPU; lin_bwd.hip includes this file
// and ties the constants below to the kernels' own with static_asserts.
#pragma once

#include <algorithm>
#include <cstdint>

namespace lb {
namespace plan {

constexpr int64_t kCUs = 256;       // compute units of the part (8 XCDs x 32)
constexpr int64_t kSlab = 32;       // reduction elements per slab of the 256x256 tile kernel
constexpr int64_t kMaxSplits = 16;  // most ranges a dX reduction is cut into
constexpr int64_t kTileFixedSlabs = 4; // a tile's fixed work (first operand round trip, epilogue) in slabs

// Length, in slabs, of a launch of n0 tiles of l0 slabs then n1 tiles of l1:
// each tile starts on the CU that frees first and takes its slabs plus the
// fixed work.  CUs that free at the same time are kept as one group; a launch
// that would need more groups than tracked counts as endless.
inline int64_t launch_span(int64_t n0, int64_t l0, int64_t n1, int64_t l1) {
    constexpr int kG = 16;
    int64_t t[kG] = {0}, c[kG] = {kCUs};
    int g = 1;
    const int64_t n[2] = {n0, n1}, len[2] = {l0 + kTileFixedSlabs, l1 + kTileFixedSlabs};
    for (int j = 0; j < 2; ++j) {
        for (int64_t left = n[j]; left > 0;) {
            int e = 0;
            for (int i = 1; i < g; ++i)
                if (t[i] < t[e])
                    e = i;
            const int64_t k = std::min(c[e], left), end = t[e] + len[j];
            left -= k;
            c[e] -= k;
            int f = -1;
            for (int i = 0; i < g; ++i)
                if (t[i] == end)
                    f = i;
            if (f >= 0) {
                c[f] += k;
            } else if (c[e] == 0) {
                t[e] = end;
                c[e] = k;
                continue;
            } else if (g < kG) {
                t[g] = end;
                c[g++] = k;
            } else {
                return INT64_MAX;
            }
            if (c[e] == 0) {
                t[e] = t[g - 1];
                c[e] = c[g - 1];
                --g;
            }
        }
    }
    int64_t span = 0;
    for (int i = 0; i < g; ++i)
        span = std::max(span, t[i]);
    return span;
}

// launch_span of ntx dX tiles of xs slabs cut into sx ranges beside wtiles dW
// tiles of ws slabs, the longer tiles launched first
inline int64_t split_span(int64_t ntx, int64_t sx, int64_t xs, int64_t wtiles, int64_t ws) {
    const int64_t lx = (xs + sx - 1) / sx;
    return lx >= ws ? launch_span(ntx * sx, lx, wtiles, ws) : launch_span(wtiles, ws, ntx * sx, lx);
}

// Reduction ranges for a dX job of ntx 256x256 tiles, each over a reduction
// of rx elements, beside ntw dW tiles over rw elements (ntw = 0: dX alone),
// with M*K fp32 partials per range and room for cap floats of them.  With few
// dX tiles (small M) one tile's reduction would outlast the launch, so it is
// split, in powers of two up to kMaxSplits, while a dX tile is longer than the
// launch's average per CU (or than a dW tile in the same launch), each range
// keeps at least 8 slabs, and the ranges' partials fit.  Splitting costs the
// partials (written, then read back) and, once the tiles no longer run in one
// wave (more tiles than CUs), a tile's fixed work per range: so the first
// split, and any split beyond one wave, needs a tile longer than that target
// by more than a quarter (at least 8 slabs); and a launch that runs in one
// wave is split into more than one only where that shortens its scheduled
// length (launch_span; one wave: at most a sixteenth more tiles than CUs,
// whose few extra tiles start as the shortest finish).
// Measured with forced range counts (calls back to back on cold inputs):
//   M = 1800, K = N = 4096 (tile 6% above the average): 1 range 106.6 us, 2 131.2
//   M = 1959, K = N = 2048 (tile 3% above a dW tile): 1 44.5, 2 55.5, 4 79.0
//   M = 200, K = N = 4096 (272 tiles unsplit, 16 dX): 4 49.1, 8 44.3, 16 51.4
//   M = 1000, K = 520, N = 4104 (one wave): 2 57.9, 4 37.9, 8 31.3, 16 36.0
//   M = 160, K = N = 2048 (one wave): 2 29.9, 4 23.1, 8 21.7, 16 25.9
//   M = 2048, K = 1024, N = 16384: 1 356.1, 4 (chosen) 131.9
//   M = 549, K = 8192, N = 1024 (one wave unsplit, two with 2): 1 31.0, 2 50.7
//   M = 200, K = 2048, N = 4104 (264 tiles with 16): 8 31.1, 16 27.9
//   M = 2048, K = N = 4096: 1 115.1, 2 136.2
inline int tile_dx_splits(int64_t M, int64_t K, int64_t ntx, int64_t rx, int64_t ntw, int64_t rw, int64_t cap) {
    const int64_t xs = (rx + kSlab - 1) / kSlab;               // slabs per dX tile
    const int64_t other = ntw > 0 ? (rw + kSlab - 1) / kSlab : 0; // slabs per dW tile
    const int64_t total = ntx * xs + ntw * other;
    const int64_t target = std::max((total + kCUs - 1) / kCUs, other);
    const int64_t limit = target + std::max<int64_t>(8, target / 4);
    const int64_t wave = kCUs + kCUs / 16;
    int sx = 1;
    while (sx < kMaxSplits) {
        const int64_t cur = (xs + sx - 1) / sx;            // a dX tile's slabs now
        const int64_t next = (xs + 2 * sx - 1) / (2 * sx); // ... with twice the ranges
        if (cur <= target || next < 8 || 2 * sx * M * K > cap)
            break;
        const bool one_wave = ntx * 2 * sx + ntw <= wave;
        if ((sx == 1 || !one_wave) && cur <= limit)
            break;
        if (!one_wave && ntx * sx + ntw <= wave &&
            split_span(ntx, 2 * sx, xs, ntw, other) >= split_span(ntx, sx, xs, ntw, other))
            break;
        sx *= 2;
    }
    return sx;
}

// The range length (elements, a whole number of 64-element pairs) and count
// for a dX reduction of N elements cut toward sx ranges.
struct Split {
    int64_t splits, len;
};
inline Split tile_split_len(int64_t N, int sx) {
    const int64_t len = ((N + sx - 1) / sx + 63) / 64 * 64;
    return {(N + len - 1) / len, len};
}

// Splits of a small-M kernel's reduction of N elements, read in chunks of
// `chunk`, by `units` blocks per split: toward one block per CU, each split a
// whole number of chunks, at most kMaxSplits, the splits' M*K fp32 partials
// within cap floats (cap 0: no partials, one split).
inline Split reduction_split(int64_t N, int64_t chunk, int64_t units, int64_t M, int64_t K, int64_t cap) {
    const int64_t chunks = (N + chunk - 1) / chunk;
    int64_t s = std::min(chunks, std::max<int64_t>(1, (kCUs + units - 1) / units));
    s = std::min<int64_t>(s, kMaxSplits);
    s = cap > 0 ? std::min(s, cap / (M * K)) : 1;
    s = std::max<int64_t>(s, 1);
    const int64_t len = (chunks + s - 1) / s * chunk;
    return {(N + len - 1) / len, len};
}

// Both small-M products in one launch (k_smallm_pair) with M up to kPairMaxM,
// N up to kPairMaxN and K*N up to kPairMaxKN (dW of 128 MiB), or
// kPairMaxKNWide above N = 4096 (measured against the two launches: M = 1 /
// 32, K = 4096, N = 8192 1.044 / 1.013 of their time, M = 28, K = 2056,
// N = 8192 0.79, M = 64, K = 8192, N = 4096 0.91; K = N = 8192 1.00 and
// N = 16384 1.00-1.12).
constexpr int64_t kPairMaxM = 64;
constexpr int64_t kPairMaxN = 8192;
constexpr int64_t kPairMaxKN = 1LL << 25;
constexpr int64_t kPairMaxKNWide = 5LL << 22;
inline bool pair_fits(int64_t M, int64_t K, int64_t N) {
    return M >= 1 && M <= kPairMaxM && N >= 1 && N <= kPairMaxN && K * N <= (N <= 4096 ? kPairMaxKN : kPairMaxKNWide);
}

// dX for M <= 16 without split partials (dx_rows16_block; with dW in one
// launch) on small calls: K from kRows16MinK (at least 32 blocks of 16 rows),
// N from kRows16MinN to kRows16MaxN and at most 4K (enough blocks for the
// reduction's length), K*N up to kRows16MaxKN.  Measured per call against the
// split kernel and its summing launch, on 90 seeded shapes with M <= 16:
// within these limits 0.70-1.00 of its time (M = 1, K = N = 1024: 8.8 ->
// 6.5 us; M = 6, K = 1912, N = 1080, dX alone: 8.8 -> 6.2); outside them
// 1.04-1.67 (K <= 632 with N >= 3152, K <= 370 with N >= 4600: too few blocks
// for long reductions; N = 176: a quarter of n is less than one chunk) or
// mixed for larger K*N (0.90 at M = 8, K = N = 4096; 1.22 at M = 16,
// K = 1024, N = 4096).
constexpr int64_t kRows16MaxM = 16;
constexpr int64_t kRows16MinK = 512;
constexpr int64_t kRows16MinN = 256;
constexpr int64_t kRows16MaxN = 4096;
constexpr int64_t kRows16MaxKN = 1LL << 21;
inline bool rows16_fits(int64_t M, int64_t K, int64_t N) {
    return M >= 1 && M <= kRows16MaxM && K >= kRows16MinK && N >= kRows16MinN && N <= kRows16MaxN &&
           N <= 4 * K && K * N <= kRows16MaxKN;
}

} // namespace plan
} // namespace lb
