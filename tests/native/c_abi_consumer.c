/*
 * A plain C program that uses liblinbwd.so through include/linbwd.h only, with
 * the HIP runtime for device memory: no Python, no torch.
 *
 *   1. lin_bwd on integer-valued bf16 operands (values -2 .. 2), on a shape
 *      that runs on the MFMA kernels and on a ragged one (K, N not multiples
 *      of 8: zero-padded copies).  Every product and every sum is exact in
 *      fp32, so dW must equal the exact sums bit for bit and dX their bf16
 *      rounding to nearest even.
 *   2. adamw_step with lr = 0 and m = v = 0 at step 1: W unchanged bit for
 *      bit, m = (1-b1)·g and v = (1-b2)·g·g as computed here in the same order.
 *   3. An unknown dtype: LB_EDTYPE and a message from lb_last_error().
 *
 * Built by the package's build step (gcc, no HIP compiler needed); prints
 * "c_abi_consumer: ok" and exits 0 when every check passes.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "linbwd.h"

#define HIP_OK(x)                                                              \
    do {                                                                       \
        hipError_t e_ = (x);                                                   \
        if (e_ != hipSuccess) {                                                \
            fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, hipGetErrorString(e_)); \
            exit(2);                                                           \
        }                                                                      \
    } while (0)

static uint32_t lcg = 12345u;
static int small_int(void) { /* -2 .. 2 */
    lcg = lcg * 1664525u + 1013904223u;
    return (int)((lcg >> 16) % 5u) - 2;
}
static uint16_t bf16_of_small_int(int v) { /* exact: the top 16 bits of the float */
    float f = (float)v;
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}
static uint16_t bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

static int check_lin_bwd(int64_t M, int64_t K, int64_t N) {
    size_t nx = (size_t)(M * K), nw = (size_t)(K * N), ng = (size_t)(M * N);
    int *x = malloc(nx * sizeof(int)), *w = malloc(nw * sizeof(int)), *g = malloc(ng * sizeof(int));
    uint16_t *hx = malloc(nx * 2), *hw = malloc(nw * 2), *hg = malloc(ng * 2), *hdx = malloc(nx * 2);
    float *hdw = malloc(nw * sizeof(float));
    for (size_t i = 0; i < nx; ++i) hx[i] = bf16_of_small_int(x[i] = small_int());
    for (size_t i = 0; i < nw; ++i) hw[i] = bf16_of_small_int(w[i] = small_int());
    for (size_t i = 0; i < ng; ++i) hg[i] = bf16_of_small_int(g[i] = small_int());
    void *dx_in, *dw_in, *dg_in, *ddx;
    float *ddw;
    HIP_OK(hipMalloc(&dx_in, nx * 2));
    HIP_OK(hipMalloc(&dw_in, nw * 2));
    HIP_OK(hipMalloc(&dg_in, ng * 2));
    HIP_OK(hipMalloc(&ddx, nx * 2));
    HIP_OK(hipMalloc((void **)&ddw, nw * sizeof(float)));
    HIP_OK(hipMemcpy(dx_in, hx, nx * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dw_in, hw, nw * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dg_in, hg, ng * 2, hipMemcpyHostToDevice));
    int rc = lin_bwd(dx_in, dw_in, dg_in, ddx, ddw, M, K, N, LB_BF16);
    if (rc != LB_OK) {
        fprintf(stderr, "lin_bwd(%lld, %lld, %lld) = %d: %s\n", (long long)M, (long long)K, (long long)N, rc,
                lb_last_error());
        return 1;
    }
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipMemcpy(hdx, ddx, nx * 2, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(hdw, ddw, nw * sizeof(float), hipMemcpyDeviceToHost));
    int bad = 0;
    for (int64_t m = 0; m < M && !bad; ++m)
        for (int64_t k = 0; k < K; ++k) { /* dX[m,k] = sum_n G[m,n] W[k,n] */
            long s = 0;
            for (int64_t n = 0; n < N; ++n) s += (long)g[m * N + n] * w[k * N + n];
            if (hdx[m * K + k] != bf16_rne((float)s)) { bad = 1; break; }
        }
    for (int64_t k = 0; k < K && !bad; ++k)
        for (int64_t n = 0; n < N; ++n) { /* dW[k,n] = sum_m X[m,k] G[m,n] */
            long s = 0;
            for (int64_t m = 0; m < M; ++m) s += (long)x[m * K + k] * g[m * N + n];
            if (hdw[k * N + n] != (float)s) { bad = 1; break; }
        }
    if (bad)
        fprintf(stderr, "lin_bwd(%lld, %lld, %lld): result differs from the exact sums\n", (long long)M, (long long)K,
                (long long)N);
    HIP_OK(hipFree(dx_in)); HIP_OK(hipFree(dw_in)); HIP_OK(hipFree(dg_in)); HIP_OK(hipFree(ddx)); HIP_OK(hipFree(ddw));
    free(x); free(w); free(g); free(hx); free(hw); free(hg); free(hdx); free(hdw);
    return bad;
}

static int check_adamw(void) {
    enum { n = 4099 };
    static float W[n], m[n], v[n], g[n], W2[n], m2[n], v2[n];
    for (int i = 0; i < n; ++i) {
        W[i] = 0.01f * (float)small_int() + 0.001f * (float)i;
        g[i] = 0.5f * (float)small_int();
        m[i] = v[i] = 0.0f;
    }
    float *dW, *dm, *dv, *dg;
    HIP_OK(hipMalloc((void **)&dW, sizeof W)); HIP_OK(hipMalloc((void **)&dm, sizeof m));
    HIP_OK(hipMalloc((void **)&dv, sizeof v)); HIP_OK(hipMalloc((void **)&dg, sizeof g));
    HIP_OK(hipMemcpy(dW, W, sizeof W, hipMemcpyHostToDevice)); HIP_OK(hipMemcpy(dm, m, sizeof m, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dv, v, sizeof v, hipMemcpyHostToDevice)); HIP_OK(hipMemcpy(dg, g, sizeof g, hipMemcpyHostToDevice));
    const float b1 = 0.9f, b2 = 0.95f;
    int rc = adamw_step(dW, dg, dm, dv, n, 0.0f, b1, b2, 1e-8f, 0.1f, 1, 1.0f);
    if (rc != LB_OK) {
        fprintf(stderr, "adamw_step = %d: %s\n", rc, lb_last_error());
        return 1;
    }
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipMemcpy(W2, dW, sizeof W, hipMemcpyDeviceToHost)); HIP_OK(hipMemcpy(m2, dm, sizeof m, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(v2, dv, sizeof v, hipMemcpyDeviceToHost));
    int bad = 0;
    for (int i = 0; i < n; ++i) {
        const float gi = g[i] * 1.0f;
        const float mi = b1 * 0.0f + (1.0f - b1) * gi;
        const float vi = b2 * 0.0f + (1.0f - b2) * gi * gi;
        if (memcmp(&W2[i], &W[i], 4) || memcmp(&m2[i], &mi, 4) || memcmp(&v2[i], &vi, 4)) { bad = 1; break; }
    }
    if (bad)
        fprintf(stderr, "adamw_step with lr = 0: W changed or m, v differ\n");
    HIP_OK(hipFree(dW)); HIP_OK(hipFree(dm)); HIP_OK(hipFree(dv)); HIP_OK(hipFree(dg));
    return bad;
}

int main(void) {
    int bad = 0;
    bad |= check_lin_bwd(300, 264, 520);  /* split-reduction dX, tile-kernel dW */
    bad |= check_lin_bwd(1100, 264, 520); /* both products on the tile kernel */
    bad |= check_lin_bwd(300, 100, 70);   /* ragged: zero-padded copies */
    bad |= check_adamw();
    int rc = lin_bwd(NULL, NULL, NULL, NULL, NULL, 1, 1, 1, 7);
    if (rc != LB_EDTYPE || lb_last_error()[0] == '\0') {
        fprintf(stderr, "unknown dtype: got %d, message '%s'\n", rc, lb_last_error());
        bad = 1;
    }
    if (lb_shutdown() != LB_OK) {
        fprintf(stderr, "lb_shutdown: %s\n", lb_last_error());
        bad = 1;
    }
    if (bad)
        return 1;
    printf("c_abi_consumer: ok (%s)\n", lb_version());
    return 0;
}
