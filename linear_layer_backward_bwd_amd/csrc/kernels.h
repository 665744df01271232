// Host-side launchers shared between the kernel files and the C ABI (api.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lb {

// ---- fused unscale + AdamW ---------------------------------------------
enum GradType { GRAD_F32 = 0, GRAD_F16 = 1, GRAD_BF16 = 2 };

enum ShadowType { SHADOW_NONE = 0, SHADOW_BF16 = 1, SHADOW_F16 = 2 };

struct AdamWArgs {
    float *W;
    const void *g;
    float *m;
    float *v;
    int64_t n;
    float lr, b1, b2, eps, wd;
    float one_minus_b1, one_minus_b2; // 1 - b, rounded to float
    float bc1, bc2;                   // 1 - b^t, computed in double, rounded once
    float inv_scale;
    const float *clip;   // device scalar multiplying the unscaled gradient, or null
    const int32_t *skip; // device flag: nonzero -> write nothing, or null
    uint16_t *W16;       // 16-bit copy of the updated W, or null (then shadow = NONE)
};

hipError_t launch_adamw(const AdamWArgs &a, GradType gt, ShadowType shadow, hipStream_t s);

// ---- gradient norm ------------------------------------------------------
constexpr int kNormMaxBlocks = 16384; // workspace: this many fp64 partials and int flags

struct NormArgs {
    const void *g;
    int64_t n;
    float inv_scale, max_norm;
    double *partial; // workspace, kNormMaxBlocks entries
    int *flag;       // workspace, kNormMaxBlocks entries
    float *out;      // [0] norm, [1] clip factor
    int32_t *found_inf; // or null
};

hipError_t launch_grad_norm(const NormArgs &a, GradType gt, hipStream_t s);

// ---- Linear backward ----------------------------------------------------
// Which kernels run the two products (LB_PATH_* of linbwd.h).
enum LinPath {
    PATH_AUTO = 0,    // chosen by dtype, alignment and M
    PATH_TILE = 1,    // the 256x256 MFMA tile kernel for both products
    PATH_SMALL_M = 2, // split-reduction dX (M <= 1024) and small-tile dW (M <= 256)
    PATH_GENERAL = 3, // the element-wise kernel (any dtype, alignment, size)
    PATH_FUSED_SMALL_M = 4, // both products in one launch streaming W and dW (M <= 64)
};

struct LinBwdArgs {
    const void *X, *W, *dY;
    void *dX;  // may be null (skip)
    float *dW; // may be null (skip)
    int64_t M, K, N;
    bool bf16; // operands bf16 (else fp32)
    // workspace for the split reduction of the small-M dX path (fp32 partials),
    // or null: then that path runs unsplit
    float *dx_partial;
    int64_t dx_partial_floats;
    int path = PATH_AUTO; // a LinPath
    // bf16 calls with K or N not a multiple of 8, or with unaligned pointers,
    // may run on zero-padded copies allocated on the stream (false: they take
    // the element-wise kernel, nothing is allocated)
    bool may_stage = true;
};

constexpr int64_t kDxPartialFloats = 1 << 24; // 64 MiB of dX partials (split tile ranges, 1 <= M <= 2048)
// what the small-M dX kernels' splits may use of it (their split counts were
// measured within this capacity)
constexpr int64_t kSmallDxPartialFloats = 1 << 23;
// dX partials are passed to the dispatch for bf16 calls with 1 <= M <= this
constexpr int64_t kDxSplitMaxM = 2048;


// The current device's pool for the padded copies of ragged or unaligned
// calls (it keeps its memory across synchronisations; lb_shutdown frees it).
hipError_t staging_pool(hipMemPool_t *out);

// Chooses kernels by dtype, alignment and M (or a.path); enqueues 1-3 launches.
hipError_t launch_lin_bwd(const LinBwdArgs &a, hipStream_t s);

// nullptr when a.path can run this call, else why it cannot (checked on the
// host before anything is enqueued).
const char *lin_bwd_path_refusal(const LinBwdArgs &a);

// ---- bias gradient ------------------------------------------------------
constexpr int kBiasMaxSplits = 256;              // row splits per launch
constexpr int64_t kBiasWorkspaceFloats = 1 << 20; // workspace: splits * N fp32 partials

struct BiasArgs {
    const void *dY; // [M,N] bf16 or fp32
    float *db;      // [N] fp32
    int64_t M, N;
    bool bf16;
    float *partial; // workspace, kBiasWorkspaceFloats entries
};

// db[n] = sum_m dY[m,n]; one or two launches; N = 0 launches nothing.
hipError_t launch_bias_grad(const BiasArgs &a, hipStream_t s);

// ---- softmax backward ---------------------------------------------------
constexpr int64_t kSoftmaxWaveMaxCols = 4096; // longest row one wave holds in registers

struct SoftmaxArgs {
    const void *P, *dY; // [rows, cols] bf16 or fp32
    void *dX;           // [rows, cols], same type; may be P or dY
    int64_t rows, cols;
    bool bf16;
};

hipError_t launch_softmax_bwd(const SoftmaxArgs &a, hipStream_t s);

} // namespace lb
