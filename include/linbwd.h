/*
 * linbwd.h -- C ABI of liblinbwd.so: the backward-and-update step of a
 * Linear layer on one AMD MI355X (gfx950).
 *
 * A Linear layer computes Y = X·W with X[M,K] (batch and sequence flattened
 * into M rows), W[K,N].  Given the upstream gradient dY = dL/dY [M,N] the
 * library computes the two backward products and then updates an fp32
 * master copy of the weights with AdamW.
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers on the current HIP device,
 *    owned by the caller; the library never allocates, frees or retains them.
 *  - Matrices are row-major and contiguous (no leading-dimension arguments).
 *  - Work is enqueued asynchronously on the stream set with lb_set_stream()
 *    (per calling thread; the null stream by default).  No call synchronises.
 *  - Argument errors are detected on the host before anything is enqueued or
 *    written, and return a negative code; lb_last_error() then describes it.
 *    A failed kernel launch returns LB_EHIP.  Faults during execution surface
 *    at the caller's next synchronisation, as for any HIP kernel.
 *  - Outputs must not alias inputs or each other.
 *  - Calls enqueued on different streams that write the same memory race.
 *  - The few calls that need temporary device memory (noted below) take it
 *    from a library-owned workspace of about 68.2 MiB per (device, stream)
 *    pair, allocated on the first such call on that stream and kept until the
 *    process ends or lb_shutdown(): calls on one stream run in order and share
 *    it, calls on different streams use different workspaces and may overlap.
 */
#ifndef LINBWD_H
#define LINBWD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element type of X, W, dY and dX in lin_bwd() */
#define LB_F32 0  /* IEEE binary32 */
#define LB_BF16 1 /* bfloat16 (upper half of a binary32) */
#define LB_F16 2  /* IEEE binary16 (gradients and 16-bit weight copies only) */

/* return codes */
#define LB_OK 0
#define LB_EINVAL (-1) /* bad size, null pointer or hyper-parameter */
#define LB_EDTYPE (-2) /* unknown dtype code */
#define LB_EHIP (-4)   /* the HIP runtime refused a launch or a query */

/*
 * lin_bwd -- the two backward products of a Linear layer:
 *     dX = dY·Wᵀ     dX[m,k] = Σ_n dY[m,n]·W[k,n]     [M,K]
 *     dW = Xᵀ·dY     dW[k,n] = Σ_m X[m,k]·dY[m,n]     [K,N]
 * Pages: "GPU 优化实战 Part 2", section "反向传播——Linear 层的梯度" (each
 * forward product becomes these two products in the backward pass);
 * "GPU 如何训练模型：从算子到 Kernel", section "一个线性层，前向和反向到底在算
 * 什么" (shapes X[M,K], W[K,N], G = dL/dY [M,N]; the input gradient is only
 * needed when the layer below is trained; transposes through strides).
 *
 *   X   [M,K]  dtype        read only
 *   W   [K,N]  dtype        read only
 *   dY  [M,N]  dtype        read only
 *   dX  [M,K]  dtype        written (overwritten, not accumulated); NULL skips dX
 *   dW  [K,N]  fp32 always  written (overwritten, not accumulated); NULL skips dW
 *   dtype      LB_BF16: bf16 operands, fp32 accumulation, dX rounded to bf16
 *              (nearest even); LB_F32: fp32 operands and outputs.
 *
 * Sizes: 0 <= M, K, N < 2^31.  With M = 0 the sums are empty and dW is filled
 * with zeros; with N = 0 dX is filled with zeros; K = 0 writes nothing.
 * Any pointer alignment and any sizes are accepted.  bf16 calls run on the
 * MFMA kernels, which read rows in 16-byte chunks: a bf16 call whose K or N is
 * not a multiple of 8, or whose pointers are not 16-byte aligned, first copies
 * the operands that need it into zero-padded buffers (rows of a multiple of 8
 * elements, 16-byte aligned), runs the padded problem and copies dX and dW
 * back.  Those buffers come from a library-owned stream-ordered memory pool
 * of the current device (hipMallocFromPoolAsync on the calling thread's
 * stream, released behind the call's last kernel with hipFreeAsync); the pool
 * keeps the memory it has mapped across synchronisations, up to the largest
 * such call's copies, until lb_shutdown().  If the allocation fails, the call
 * takes the element-wise kernel instead (a forced path returns LB_EHIP).
 * fp32 calls take the element-wise kernel.
 * For bf16 with 1 <= M <= 2048 (decode-like and small batches, and batches
 * too small to fill the GPU with whole dX tiles), dX may sum over n in
 * several blocks whose fp32 partial sums go to the library-owned workspace of
 * the calling thread's stream and are added in a fixed order (results repeat
 * bit for bit).  The kernels are chosen by dtype, alignment,
 * M, K, N and the outputs requested unless lb_set_lin_bwd_path() forces a
 * path; every choice computes the same sums, rounded once.
 * Errors: LB_EINVAL for a negative size, a NULL operand that a requested
 * output needs (X for dW; W for dX; dY for either), or a forced kernel path
 * that cannot run the call; LB_EDTYPE for another dtype; LB_EHIP when the
 * workspace cannot be allocated or a launch fails.
 * Both outputs NULL is a no-op (LB_OK).
 */
int lin_bwd(const void *X, const void *W, const void *dY, void *dX, float *dW,
            int64_t M, int64_t K, int64_t N, int dtype);

/*
 * lin_bwd_ex -- lin_bwd plus the bias gradient of Y = X·W + b, where b [N] is
 * added to every row ("GPU 优化实战 Part 2", section "反向传播——Linear 层的
 * 梯度", which writes the forward with a bias; its AdamW section then updates
 * with dW and db):
 *     db[n] = Σ_m dY[m,n]                                    [N]
 *
 *   db  [N]  fp32 always  written (overwritten); NULL makes this call lin_bwd
 * Every other argument, size rule and error is lin_bwd's.  db is summed in
 * fp32 per row range and the partials in fp64, in a fixed order (results
 * repeat bit for bit); M = 0 fills db with zeros.  X and W may be NULL when
 * only db is requested.  Additional error: LB_EINVAL for a NULL dY with db
 * requested and M, N > 0.  db's row partials go to the library-owned
 * workspace of the calling thread's stream.
 */
int lin_bwd_ex(const void *X, const void *W, const void *dY, void *dX, float *dW, float *db,
               int64_t M, int64_t K, int64_t N, int dtype);

/*
 * lin_bwd_ex_noalloc -- lin_bwd_ex for callers that cannot allocate device
 * memory: code being captured into a HIP graph, tight serving loops, harnesses
 * that forbid hipMalloc.  It computes exactly what lin_bwd_ex computes (the
 * same kernels, splits and summation order, so the same bits), with the same
 * arguments, sizes and errors, but calls no allocating routine: its
 * temporaries (the small-M dX split partials and db's row partials) live in a
 * static device array of 68 MiB (16 Mi + 1 Mi floats) that the library holds on
 * every device it runs on until the process ends.  The kernels size their
 * splits to that array, so no size is refused for want of room.  Nothing in it
 * needs to start at zero: every partial is written before it is read.
 * All calls on one device share the one array, whatever their stream or
 * thread: calls that overlap on a device race (unlike lin_bwd_ex, whose
 * workspace is per stream), so the caller keeps them in one stream order.
 * The first call on a device looks up the array's device address
 * (hipGetSymbolAddress); LB_EHIP if that fails.  For HIP graph capture, make
 * that first call before capturing; the calls then record kernel launches
 * only (no allocation, no memset).  One exception to "the same
 * kernels": a bf16 call with K or N not a multiple of 8 or with unaligned
 * pointers, which lin_bwd_ex runs on padded copies it allocates, takes the
 * element-wise kernel here (the same bars, not the same bits), and a forced
 * MFMA path refuses it (LB_EINVAL).
 */
int lin_bwd_ex_noalloc(const void *X, const void *W, const void *dY, void *dX, float *dW,
                       float *db, int64_t M, int64_t K, int64_t N, int dtype);

/*
 * adamw_step -- one fused pass over n parameters that unscales the gradient
 * and applies AdamW with decoupled weight decay to the fp32 master weights:
 *     g  = float(grad[i]) · inv_scale
 *     m  = b1·m + (1 − b1)·g
 *     v  = b2·v + (1 − b2)·g·g
 *     m̂ = m / (1 − b1^step)      v̂ = v / (1 − b2^step)
 *     W  = W − lr·( m̂ / (√v̂ + eps) + wd·W )        (W on the right: before the step)
 * Pages: "GPU 优化实战 Part 2", sections "AdamW 优化器——融合内核" (the fused
 * per-parameter update with bias corrections) and "混合精度训练（FP16 / BF16）"
 * (fp32 master weights; a loss-scaled gradient is multiplied by 1/scale
 * before the update); "Mastering LLM Training with CUDA and ROCm", section
 * "AdamW Algorithm" (the same update as θ − η·m̂/(√v̂+ε) − η·λ·θ).
 *
 *   W, m, v  [n] fp32   read and written once each, in place
 *   grad     [n]        read only (not zeroed); fp32 for adamw_step, IEEE
 *                       binary16 bit patterns for adamw_step_f16, bfloat16
 *                       bit patterns for adamw_step_bf16
 *   step     the 1-based step number t; the bias corrections 1 − b^t are
 *            computed once per call on the host in double and rounded to float
 *   inv_scale  1 / loss scale (1 for an unscaled gradient)
 *
 * The fp32 arithmetic is done in the order written above, without fused
 * multiply-add contraction, with IEEE division and square root.
 * n = 0 is a no-op.  Any alignment of the element types is accepted (one
 * parameter per thread).  NaN and infinity propagate (no skip, no detection).
 * Errors: LB_EINVAL for n < 0, a NULL buffer with n > 0, step < 1, or b1 / b2
 * outside [0, 1); LB_EHIP when the launch fails.
 */
int adamw_step(float *W, const float *grad, float *m, float *v, int64_t n,
               float lr, float b1, float b2, float eps, float wd, int step,
               float inv_scale);
int adamw_step_f16(float *W, const uint16_t *grad, float *m, float *v, int64_t n,
                   float lr, float b1, float b2, float eps, float wd, int step,
                   float inv_scale);
int adamw_step_bf16(float *W, const uint16_t *grad, float *m, float *v, int64_t n,
                    float lr, float b1, float b2, float eps, float wd, int step,
                    float inv_scale);

/*
 * adamw_step_ex -- the AdamW pass with the optional parts of the training
 * step around it, in the order of the pages' complete loop ("GPU 优化实战
 * Part 2", section "完整训练循环（整合一切）": unscale, clip, AdamW on the fp32
 * master weights, 16-bit copy of the updated weights for the next forward
 * pass; section "混合精度训练（FP16 / BF16）" for the 16-bit forward weights).
 * Per parameter:
 *   g   = (float(grad) * inv_scale) * clip        clip = *d_clip, or 1 if NULL
 *   ... the AdamW update of adamw_step ...
 *   W16 = W rounded to nearest even, as w16_dtype  (if W16 is not NULL)
 * and nothing at all is written when d_skip is not NULL and *d_skip != 0.
 *
 *   W, m, v, grad, n, lr .. inv_scale   as for adamw_step
 *   grad_dtype  LB_F32, LB_F16 or LB_BF16 (element type of grad)
 *   d_clip      device pointer to one float, read by the kernel (so a factor
 *               computed on the device needs no host round trip), or NULL
 *   d_skip      device pointer to one int32, read by the kernel, or NULL
 *   W16         [n] 16-bit copy of the updated W (written), or NULL
 *   w16_dtype   LB_BF16 or LB_F16; ignored when W16 is NULL
 *
 * All pointers are device memory owned by the caller; W16 must not alias the
 * other buffers.  Any alignment of the element types is accepted.
 * Asynchronous on the thread's stream, like adamw_step.
 * Errors: those of adamw_step; LB_EDTYPE for another grad_dtype, or a W16
 * with a w16_dtype other than LB_BF16 / LB_F16.
 */
int adamw_step_ex(float *W, const void *grad, int grad_dtype, float *m, float *v, int64_t n,
                  float lr, float b1, float b2, float eps, float wd, int step, float inv_scale,
                  const float *d_clip, const int32_t *d_skip, void *W16, int w16_dtype);

/*
 * grad_norm -- the L2 norm of the unscaled gradient and the clip factor of the
 * pages' complete loop ("GPU 优化实战 Part 2", section "完整训练循环（整合
 * 一切）": the norm of the fp32 gradient, and a scale of max_norm / norm when it
 * exceeds max_norm), with an inf/NaN flag, written to device memory so that
 * adamw_step_ex can consume them without a host round trip:
 *   g32 = float(grad[i]) * inv_scale                  (fp32)
 *   d_out[0] = sqrt(sum g32^2)      exact squares summed in fp64, rounded once
 *   d_out[1] = d_out[0] > max_norm ? max_norm / d_out[0] : 1    (max_norm <= 0: 1)
 *   *d_found_inf = 1 if some g32 is inf or NaN, else 0         (if not NULL)
 * Pass d_out + 1 as adamw_step_ex's d_clip and d_found_inf as its d_skip.
 *
 *   grad         [n] device, read only; grad_dtype LB_F32, LB_F16 or LB_BF16
 *   d_out        device float[2], written
 *   d_found_inf  device int32, written, or NULL
 *
 * The summation order is fixed for a given n and 16-byte alignment of grad
 * (the result is reproducible).
 * The per-block partials go to the library-owned workspace of the calling
 * thread's stream.  Asynchronous on the thread's stream.  Errors: LB_EDTYPE for another
 * grad_dtype; LB_EINVAL for n < 0, NULL d_out, or NULL grad with n > 0;
 * LB_EHIP when the workspace cannot be allocated or a launch fails.
 */
int grad_norm(const void *grad, int grad_dtype, int64_t n, float inv_scale, float max_norm,
              float *d_out, int32_t *d_found_inf);

/*
 * softmax_bwd -- backward of a row softmax P = softmax(z), with respect to the
 * logits z ("GPU 优化实战 Part 2", section "Softmax 和 LayerNorm 的梯度（自定义
 * 内核）", softmax backward):
 *     dX[r,i] = P[r,i] * (dY[r,i] - Σ_j P[r,j]*dY[r,j])
 *
 *   P   [rows, cols]  dtype  read only (the forward's output)
 *   dY  [rows, cols]  dtype  read only
 *   dX  [rows, cols]  dtype  written; may be the same buffer as P or dY (in
 *                            place), must not overlap them otherwise
 *   dtype  LB_F32, or LB_BF16 (bf16 in and out, fp32 arithmetic, dX rounded
 *          to nearest even)
 *
 * Row-major, contiguous.  Each row's dot product is summed in fp32 in a fixed
 * order (results repeat bit for bit).  Any sizes and alignment; rows of up to
 * 4096 columns are held in registers (one read of P and dY), longer rows are
 * read twice.  rows = 0 or cols = 0 writes nothing.  Asynchronous on the
 * thread's stream.  Errors: LB_EDTYPE for another dtype; LB_EINVAL for a
 * negative size, a size of 2^40 or more, or a NULL buffer with rows, cols > 0;
 * LB_EHIP when a launch fails.
 */
int softmax_bwd(const void *P, const void *dY, void *dX, int64_t rows, int64_t cols, int dtype);

/*
 * lb_set_stream -- the HIP stream (a hipStream_t, passed as void*) on which
 * the calling thread's later calls enqueue their kernels; NULL selects the
 * null stream.  The setting is per thread.  Returns LB_OK.
 * ("GPU 优化实战 Part 2", section "完整训练循环（整合一切）": the step's kernels
 * are launched asynchronously in stream order, with one synchronisation at
 * the end.)
 */
int lb_set_stream(void *hip_stream);

/*
 * lb_set_lin_bwd_path -- forces which kernels lin_bwd / lin_bwd_ex use for
 * the calling thread's later calls (per thread, like the stream), so that
 * the kernels can be compared with each other on the same inputs and a
 * caller can pin a choice; every path computes the same sums, rounded once.
 *   LB_PATH_AUTO     chosen by dtype, alignment, M, K, N and the outputs
 *                    requested (the default)
 *   LB_PATH_TILE     both products on the 256x256 MFMA tile kernel (for
 *                    M <= 2048 with dX's reduction split over several tiles
 *                    when that shortens the launch)
 *   LB_PATH_SMALL_M  dX on the split-reduction kernel (M <= 1024), dW on the
 *                    small-tile kernel (M <= 256); at M <= 64 with both
 *                    products and moderate K*N, the blocks of both in one
 *                    launch; at M <= 16 on small calls, dX blocks that each
 *                    sum a whole reduction (no partials)
 *   LB_PATH_GENERAL  both products on the element-wise kernel
 *   LB_PATH_FUSED_SMALL_M  both products in one launch in which each block
 *                    streams 16 rows of W and writes the same 16 rows of dW
 *                    (1 <= M <= 64, dX and dW both requested; never chosen
 *                    automatically: slower than the SMALL_M pair on the
 *                    shapes measured)
 * A forced MFMA path (TILE, SMALL_M, FUSED_SMALL_M) needs bf16 operands and
 * the M limits above.  K or N not a multiple of 8, or unaligned pointers, run
 * on zero-padded copies (see lin_bwd; lin_bwd_ex_noalloc cannot make them and
 * refuses such calls); the limits of the buffer windows are then those of the
 * padded call: K, N < 2^25, for dX on the tile kernel N < 2^22, and for the
 * small-M dW and fused kernels X (and dY) below 2 GiB.  A call the path
 * cannot run fails with LB_EINVAL before anything is enqueued.  Returns LB_OK,
 * or LB_EINVAL for another value.
 */
#define LB_PATH_AUTO 0
#define LB_PATH_TILE 1
#define LB_PATH_SMALL_M 2
#define LB_PATH_GENERAL 3
#define LB_PATH_FUSED_SMALL_M 4
int lb_set_lin_bwd_path(int path);

/*
 * lb_last_error -- a description of the calling thread's last non-zero
 * return, or "" if there was none.  (The pages' listings check no error;
 * every entry point here validates its arguments on the host and reports
 * why it refused a call.)  The string is owned by the library and
 * valid until the thread's next call.
 */
const char *lb_last_error(void);

/* lb_version -- the library's version string (static storage). */
const char *lb_version(void);

/*
 * lb_shutdown -- frees the library-owned workspaces of every device and
 * stream (the gradient norm's partial sums, lin_bwd_ex's bias partials and
 * lin_bwd's dX partials for bf16 with 1 <= M <= 2048, allocated on first use
 * per device and stream; without this call they are kept until the process
 * ends) and destroys each device's memory pool of lin_bwd's padded copies
 * (ragged or unaligned bf16 calls).  A later call that needs a workspace or
 * a pool makes it again.  The static array of lin_bwd_ex_noalloc is not
 * freed: it lives as long as the process.  No call of this library may be in
 * flight on any device, on any stream, nor may another thread call into the
 * library meanwhile: the caller synchronizes first.  The calling thread's
 * current device is unchanged.  Returns LB_OK, or LB_EHIP
 * when a free fails (the remaining workspaces are still freed and forgotten).
 */
int lb_shutdown(void);

#ifdef __cplusplus
}
#endif

#endif /* LINBWD_H */
