/*
 * CPU oracle for the Linear-layer backward and the fused unscale + AdamW update.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the tests, the smoke check and the bench's CPU
 * baseline leg use it.  It shares no code, header, table or constant with the
 * HIP library; it is built by gcc with -O2 -ffp-contract=off and no fast-math,
 * so every float operation below is one IEEE-754 operation, rounded to
 * nearest even, in the order written.
 *
 * What it computes, and where the pages define it:
 *
 *  - Linear layer Y = X·W with X[M,K], W[K,N] (batch and sequence flattened
 *    into M) and upstream gradient G = dL/dY [M,N]:
 *        dX = G·Wᵀ      dX[m,k] = Σ_n G[m,n]·W[k,n]
 *        dW = Xᵀ·G      dW[k,n] = Σ_m X[m,k]·G[m,n]
 *        db = 1ᵀ·G      db[n]   = Σ_m G[m,n]       (bias b added to every row)
 *  - Softmax backward over rows: dX = P ⊙ (dY − rowsum(P ⊙ dY)).
 *    Pages: "GPU 优化实战 Part 2", section "反向传播——Linear 层的梯度"
 *    (the two backward products of a Linear layer); "GPU 如何训练模型：从算子
 *    到 Kernel", section "一个线性层，前向和反向到底在算什么" (shapes with batch
 *    and sequence merged into M, transposes expressed through strides).
 *    The oracle evaluates both sums in fp64 on the exact decoded input values,
 *    as plain loops with no blocking: every entry is its sum taken in index
 *    order from 0.0 (the whole-row functions add the terms of one output row
 *    side by side, which changes no entry's operations or their order).
 *
 *  - AdamW with decoupled weight decay on an fp32 master copy, after
 *    unscaling a loss-scaled gradient:
 *        g  = float(g_in) * inv_scale
 *        m  = b1*m + (1-b1)*g
 *        v  = b2*v + (1-b2)*g*g
 *        mh = m / (1 - b1^t)        vh = v / (1 - b2^t)
 *        W  = W - lr*( mh/(sqrt(vh)+eps) + wd*W )      (W on the right: old W)
 *    Pages: "GPU 优化实战 Part 2", sections "AdamW 优化器——融合内核" (the
 *    per-parameter update and its bias corrections) and "混合精度训练（FP16 /
 *    BF16）" (loss scale, unscale by multiplying with 1/scale before the
 *    update); "Mastering LLM Training with CUDA and ROCm", section "AdamW
 *    Algorithm" (the same update written as θ − η·m̂/(√v̂+ε) − η·λ·θ).
 *    The oracle is a scalar fp32 loop.  The bias corrections are evaluated
 *    once per call in double and rounded to float once.
 *
 *  - The training step's optional parts around that update, in the order of
 *    the pages' complete loop ("GPU 优化实战 Part 2", section "完整训练循环
 *    （整合一切）": unscale to fp32, optional clipping of the gradient by a
 *    factor, the AdamW step on the fp32 master weights, then a 16-bit copy of
 *    the updated weights for the next forward pass; section "混合精度训练
 *    （FP16 / BF16）" for the 16-bit forward weights):
 *        g  = (float(g_in) * inv_scale) * clip          (clip given: two roundings)
 *        ... the AdamW update above ...
 *        W16 = round_to_nearest_even(W) as fp16 or bf16
 *    and a skip flag that leaves every array untouched.  The 16-bit roundings
 *    are written from the IEEE definitions below.
 *
 *  - The loop's gradient clipping (same section, its step 7: the L2 norm of
 *    the unscaled fp32 gradient; when it exceeds max_norm the gradient is
 *    scaled by max_norm / norm):
 *        g32  = float(g_in) * inv_scale                       (fp32, as above)
 *        norm = sqrt( sum g32^2 )     squares and sum in fp64, rounded to fp32 once
 *        clip = norm > max_norm ? max_norm / norm : 1         (fp32; max_norm <= 0: 1)
 *        found_inf = some g32 is inf or NaN
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* element types of the caller's buffers */
#define ORACLE_F32 0
#define ORACLE_BF16 1
#define ORACLE_F16 2

/* ---- exact decoders ---------------------------------------------------- */

/* bf16 is the upper half of an IEEE binary32: widening is a 16-bit shift. */
static double bf16_value(uint16_t h)
{
    uint32_t bits = (uint32_t)h << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 mantissa bits. */
static double f16_value(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int mant = h & 0x3ff;
    double mag;
    if (e == 0)
        mag = ldexp((double)mant, -24); /* subnormal: mant * 2^-14 * 2^-10 */
    else if (e == 31)
        mag = mant ? NAN : INFINITY;
    else
        mag = ldexp((double)(mant | 0x400), e - 25); /* 1.mant * 2^(e-15) */
    return sign ? -mag : mag;
}

/* The decoders, exported for the pins (the loops below use the static ones,
 * which the compiler can inline). */
double oracle_bf16_to_f64(uint16_t h)
{
    return bf16_value(h);
}

double oracle_f16_to_f64(uint16_t h)
{
    return f16_value(h);
}

static double elt(const void *p, int dtype, int64_t i)
{
    if (dtype == ORACLE_F32)
        return (double)((const float *)p)[i];
    if (dtype == ORACLE_BF16)
        return bf16_value(((const uint16_t *)p)[i]);
    return f16_value(((const uint16_t *)p)[i]);
}

void oracle_decode(const void *p, int dtype, int64_t n, double *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = elt(p, dtype, i);
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---- Linear backward, fp64 ---------------------------------------------- */

/* acc[j] += x * value(p[off + j]) for j = 0 .. n-1: one fp64 product and one
 * fp64 addition per j (the element type is tested once, outside the loop).
 * Built twice, for AVX2 and for any x86-64, and picked at load time by the CPU:
 * wider vectors, the same IEEE operations (no contraction, no reassociation). */
__attribute__((target_clones("avx2", "default")))
static void add_scaled_row(double *acc, double x, const void *p, int dtype, int64_t off, int64_t n)
{
    if (dtype == ORACLE_F32) {
        const float *q = (const float *)p + off;
        for (int64_t j = 0; j < n; ++j)
            acc[j] += x * (double)q[j];
    } else if (dtype == ORACLE_BF16) {
        const uint16_t *q = (const uint16_t *)p + off;
        for (int64_t j = 0; j < n; ++j)
            acc[j] += x * bf16_value(q[j]);
    } else {
        const uint16_t *q = (const uint16_t *)p + off;
        for (int64_t j = 0; j < n; ++j)
            acc[j] += x * f16_value(q[j]);
    }
}

/* Output rows that the whole-row functions build side by side, so that one
 * pass over the shared operand serves them all (each row's own operations and
 * their order do not depend on it). */
#define ORACLE_ROW_GROUP 8

/* Size in bytes of one stored element. */
static size_t elt_size(int dtype)
{
    return dtype == ORACLE_F32 ? 4 : 2;
}

/*
 * Whole rows of dX: out[i*K + k] = dX[rows[i], k] = Σ_n G[rows[i],n]·W[k,n] for
 * every k (rows == NULL: every row m = i of dX, nrows = M).
 *
 * Each entry is the plain sum over n = 0, 1, ..., N-1, started from 0.0, one
 * fp64 product (exact for bf16, fp16 and fp32 inputs) and one fp64 addition per
 * term, in that order: the same operations as the dot product of oracle_dx_at.
 * The terms of all k of a few rows are added side by side (n outer, k inner),
 * so that memory is read in order; for that W's elements are first copied into
 * Wt[n,k] = W[k,n] (a copy of the stored values, no arithmetic).
 * Returns 0, or -1 when the copy cannot be allocated.
 */
int oracle_dx_rows(const void *G, const void *W, int dtype,
                   int64_t M, int64_t K, int64_t N,
                   const int64_t *rows, int64_t nrows, double *out)
{
    (void)M;
    const size_t es = elt_size(dtype);
    char *Wt = malloc((size_t)(K * N > 0 ? K * N : 1) * es);
    if (!Wt)
        return -1;
#pragma omp parallel for schedule(static)
    for (int64_t k = 0; k < K; ++k)
        for (int64_t n = 0; n < N; ++n)
            memcpy(Wt + (size_t)(n * K + k) * es, (const char *)W + (size_t)(k * N + n) * es, es);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i0 = 0; i0 < nrows; i0 += ORACLE_ROW_GROUP) {
        const int64_t cnt = nrows - i0 < ORACLE_ROW_GROUP ? nrows - i0 : ORACLE_ROW_GROUP;
        for (int64_t i = i0; i < i0 + cnt; ++i)
            for (int64_t k = 0; k < K; ++k)
                out[i * K + k] = 0.0;
        for (int64_t n = 0; n < N; ++n)
            for (int64_t i = i0; i < i0 + cnt; ++i) {
                const int64_t m = rows ? rows[i] : i;
                add_scaled_row(out + i * K, elt(G, dtype, m * N + n), Wt, dtype, n * K, K);
            }
    }
    free(Wt);
    return 0;
}

/*
 * Whole rows of dW: out[i*N + n] = dW[rows[i], n] = Σ_m X[m,rows[i]]·G[m,n] for
 * every n (rows == NULL: every row k = i of dW, nrows = K).  Each entry is the
 * plain sum over m = 0, 1, ..., M-1 from 0.0, the same operations in the same
 * order as the dot product of oracle_dw_at; the terms of all n of a few rows
 * are added side by side (m outer, n inner).
 */
void oracle_dw_rows(const void *X, const void *G, int dtype,
                    int64_t M, int64_t K, int64_t N,
                    const int64_t *rows, int64_t nrows, double *out)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i0 = 0; i0 < nrows; i0 += ORACLE_ROW_GROUP) {
        const int64_t cnt = nrows - i0 < ORACLE_ROW_GROUP ? nrows - i0 : ORACLE_ROW_GROUP;
        for (int64_t i = i0; i < i0 + cnt; ++i)
            for (int64_t n = 0; n < N; ++n)
                out[i * N + n] = 0.0;
        for (int64_t m = 0; m < M; ++m)
            for (int64_t i = i0; i < i0 + cnt; ++i) {
                const int64_t k = rows ? rows[i] : i;
                add_scaled_row(out + i * N, elt(X, dtype, m * K + k), G, dtype, m * N, N);
            }
    }
}

/* dX[m,k] = Σ_n G[m,n]·W[k,n], all M·K entries.  Row-major, contiguous.
 * Returns 0, or -1 when out of host memory. */
int oracle_dx(const void *G, const void *W, int dtype,
              int64_t M, int64_t K, int64_t N, double *dX)
{
    return oracle_dx_rows(G, W, dtype, M, K, N, NULL, M, dX);
}

/* dW[k,n] = Σ_m X[m,k]·G[m,n], all K·N entries. */
void oracle_dw(const void *X, const void *G, int dtype,
               int64_t M, int64_t K, int64_t N, double *dW)
{
    oracle_dw_rows(X, G, dtype, M, K, N, NULL, K, dW);
}

/* The same sums at a list of (row, col) positions only: out[i] = dX[rows[i], cols[i]]. */
void oracle_dx_at(const void *G, const void *W, int dtype,
                  int64_t M, int64_t K, int64_t N,
                  const int64_t *rows, const int64_t *cols, int64_t cnt, double *out)
{
    (void)M;
    (void)K;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t i = 0; i < cnt; ++i) {
        int64_t m = rows[i], k = cols[i];
        double s = 0.0;
        for (int64_t n = 0; n < N; ++n)
            s += elt(G, dtype, m * N + n) * elt(W, dtype, k * N + n);
        out[i] = s;
    }
}

/* out[i] = dW[rows[i], cols[i]] (rows index K, cols index N). */
void oracle_dw_at(const void *X, const void *G, int dtype,
                  int64_t M, int64_t K, int64_t N,
                  const int64_t *rows, const int64_t *cols, int64_t cnt, double *out)
{
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t i = 0; i < cnt; ++i) {
        int64_t k = rows[i], n = cols[i];
        double s = 0.0;
        for (int64_t m = 0; m < M; ++m)
            s += elt(X, dtype, m * K + k) * elt(G, dtype, m * N + n);
        out[i] = s;
    }
}

/* ---- bias gradient, fp64 -------------------------------------------------- */

/* db[n] = Σ_m G[m,n]: the gradient of the bias b in Y = X·W + b, where b is
 * added to every one of the M rows ("GPU 优化实战 Part 2", section
 * "反向传播——Linear 层的梯度", which writes the forward with a bias; the
 * section "AdamW 优化器——融合内核" then speaks of dW and db). */
void oracle_db(const void *G, int dtype, int64_t M, int64_t N, double *db)
{
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        double s = 0.0;
        for (int64_t m = 0; m < M; ++m)
            s += elt(G, dtype, m * N + n);
        db[n] = s;
    }
}

/* ---- softmax backward, fp64 ---------------------------------------------- */

/* Rows of P = softmax(z) (probabilities, row-major [rows, cols]) and of the
 * upstream gradient dY: dX[r,i] = P[r,i]·(dY[r,i] − Σ_j P[r,j]·dY[r,j]), the
 * gradient with respect to the logits z ("GPU 优化实战 Part 2", section
 * "Softmax 和 LayerNorm 的梯度（自定义内核）", softmax backward). */
void oracle_softmax_bwd(const void *P, const void *dY, int dtype, int64_t rows, int64_t cols,
                        double *dX)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        double dot = 0.0;
        for (int64_t j = 0; j < cols; ++j)
            dot += elt(P, dtype, r * cols + j) * elt(dY, dtype, r * cols + j);
        for (int64_t i = 0; i < cols; ++i)
            dX[r * cols + i] = elt(P, dtype, r * cols + i) * (elt(dY, dtype, r * cols + i) - dot);
    }
}

/* ---- unscale + AdamW, scalar fp32 --------------------------------------- */

static float grad_f32(const void *g, int gtype, int64_t i)
{
    if (gtype == ORACLE_F32)
        return ((const float *)g)[i];
    /* bf16 and fp16 values are exactly representable in binary32 */
    return (float)elt(g, gtype, i);
}

/*
 * One AdamW step over n parameters, in place on W, m, v.  g is read only.
 * Returns 0, or -1 for arguments under which the update is undefined
 * (step < 1, or a beta outside [0,1) which makes a bias correction zero or
 * meaningless).
 */
/* ---- 16-bit roundings of an fp32 value (IEEE round to nearest, ties to even) ---- */

/* bf16 keeps the upper 16 bits of the binary32 pattern: add half of the
 * dropped part, plus one when the kept part is odd (ties to even), then
 * truncate; a carry into the exponent is the correct rounding, including to
 * infinity.  NaN stays NaN (quiet bit set, sign kept). */
uint16_t oracle_f32_to_bf16(float f)
{
    uint32_t b;
    memcpy(&b, &f, sizeof b);
    if ((b & 0x7fffffffu) > 0x7f800000u)
        return (uint16_t)((b >> 16) | 0x0040u);
    const uint32_t lsb = (b >> 16) & 1u;
    return (uint16_t)((b + 0x7fffu + lsb) >> 16);
}

/* binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits; normal values
 * 2^-14 <= |x| <= 65504, subnormals k*2^-24.  Computed on the exact value in
 * double with nearbyint (round to nearest even in the default mode). */
uint16_t oracle_f32_to_f16(float f)
{
    const uint16_t sign = signbit(f) ? 0x8000u : 0u;
    if (isnan(f))
        return (uint16_t)(sign | 0x7e00u);
    const double a = fabs((double)f);
    if (isinf(f))
        return (uint16_t)(sign | 0x7c00u);
    if (a < ldexp(1.0, -14)) {                 /* subnormal range: k * 2^-24 */
        const double k = nearbyint(ldexp(a, 24)); /* exact scaling; k <= 1024 */
        return (uint16_t)(sign | (uint16_t)k); /* k == 1024 is the smallest normal */
    }
    int e;
    (void)frexp(a, &e);                        /* a = fr * 2^e, 0.5 <= fr < 1 */
    e -= 1;                                    /* 2^e <= a < 2^(e+1) */
    double q = nearbyint(ldexp(a, 10 - e));    /* 1024 <= q <= 2048 */
    if (q >= 2048.0) {
        q = 1024.0;
        e += 1;
    }
    if (e > 15)
        return (uint16_t)(sign | 0x7c00u);     /* rounds past 65504: infinity */
    return (uint16_t)(sign | (uint16_t)((e + 15) << 10) | (uint16_t)(q - 1024.0));
}

void oracle_round16(const float *in, int64_t n, int type, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = type == ORACLE_BF16 ? oracle_f32_to_bf16(in[i]) : oracle_f32_to_f16(in[i]);
}

int oracle_adamw(float *W, const void *g, int gtype, float *m, float *v, int64_t n,
                 float lr, float b1, float b2, float eps, float wd, int step,
                 float inv_scale)
{
    if (step < 1 || !(b1 >= 0.0f && b1 < 1.0f) || !(b2 >= 0.0f && b2 < 1.0f) || n < 0)
        return -1;
    const float bc1 = (float)(1.0 - pow((double)b1, (double)step));
    const float bc2 = (float)(1.0 - pow((double)b2, (double)step));
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        float gi = grad_f32(g, gtype, i) * inv_scale;
        m[i] = b1 * m[i] + (1.0f - b1) * gi;
        v[i] = b2 * v[i] + (1.0f - b2) * gi * gi;
        float mh = m[i] / bc1;
        float vh = v[i] / bc2;
        W[i] = W[i] - lr * (mh / (sqrtf(vh) + eps) + wd * W[i]);
    }
    return 0;
}

/* Global L2 norm of the unscaled gradient, its clip factor and an inf/NaN
 * flag: out[0] = norm, out[1] = clip factor, *found_inf = 0 or 1.  A plain
 * sequential fp64 sum of the exact squares of the fp32 values. */
void oracle_grad_norm(const void *g, int gtype, int64_t n, float inv_scale, float max_norm,
                      float *out, int *found_inf)
{
    double sum = 0.0;
    int bad = 0;
    for (int64_t i = 0; i < n; ++i) {
        const float x = grad_f32(g, gtype, i) * inv_scale;
        if (!isfinite(x))
            bad = 1;
        sum += (double)x * (double)x;
    }
    const float norm = (float)sqrt(sum);
    out[0] = norm;
    out[1] = (max_norm > 0.0f && norm > max_norm) ? max_norm / norm : 1.0f;
    *found_inf = bad;
}

/* The update with the loop's optional parts: clip (NULL: none) multiplies the
 * unscaled gradient, skip != 0 leaves W, m, v and W16 untouched, W16 (NULL:
 * none) receives the updated W rounded to w16type (ORACLE_BF16 / ORACLE_F16). */
int oracle_adamw_ex(float *W, const void *g, int gtype, float *m, float *v, int64_t n,
                    float lr, float b1, float b2, float eps, float wd, int step,
                    float inv_scale, const float *clip, int skip, uint16_t *W16, int w16type)
{
    if (step < 1 || !(b1 >= 0.0f && b1 < 1.0f) || !(b2 >= 0.0f && b2 < 1.0f) || n < 0)
        return -1;
    if (W16 && w16type != ORACLE_BF16 && w16type != ORACLE_F16)
        return -1;
    if (skip)
        return 0;
    const float bc1 = (float)(1.0 - pow((double)b1, (double)step));
    const float bc2 = (float)(1.0 - pow((double)b2, (double)step));
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        float gi = grad_f32(g, gtype, i) * inv_scale;
        if (clip)
            gi = gi * *clip;
        m[i] = b1 * m[i] + (1.0f - b1) * gi;
        v[i] = b2 * v[i] + (1.0f - b2) * gi * gi;
        float mh = m[i] / bc1;
        float vh = v[i] / bc2;
        W[i] = W[i] - lr * (mh / (sqrtf(vh) + eps) + wd * W[i]);
        if (W16)
            W16[i] = w16type == ORACLE_BF16 ? oracle_f32_to_bf16(W[i]) : oracle_f32_to_f16(W[i]);
    }
    return 0;
}
