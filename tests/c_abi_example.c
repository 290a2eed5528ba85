/*
 * The C ABI used from plain C, without Python or PyTorch: device buffers from
 * the HIP runtime, the library's calls on a stream the program creates, and
 * the results checked against the C oracle (oracle/oracle.c, linked in as
 * test infrastructure) within |y - y_ref| <= 1e-4 * sum|w x| + 1e-6.
 *
 * Cases: a Q4_K GEMV (512 x 512, batch 1), a Q6_K GEMV through the
 * LDS-streaming kernel (256 x 8192, batch 2), the whole decode FFN with the
 * residual added in place (hidden 512, FF 1024), activations quantized to
 * int8 (codes and scales equal to the oracle's bit for bit) and the Q8_0
 * GEMV on them (300 x 2560, batch 3), and a rejected call that must return
 * QD_ESHAPE without enqueuing anything.  Built by
 * __graft_entry__.build() into tests/c_abi_example.bin (gcc, host code
 * only); run by tests/test_gpu_c_abi.py.  Prints one "ok" line and exits 0.
 */
#define __HIP_PLATFORM_AMD__ 1
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../include/qdecode.h"
#include "../oracle/oracle.h"

static uint64_t rng = 0xC0FFEEull;
static uint32_t next_u32(void) {
    uint64_t z = (rng += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return (uint32_t)((z ^ (z >> 31)) >> 32);
}
static float unit(void) { return (float)(next_u32() >> 8) / 16777216.0f; }
static float normalish(void) { return (unit() + unit() + unit() - 1.5f) * 2.0f; }

/* f16 bits of v (v a small positive normal number, rounded by truncation:
 * any f16 value is a valid scale) */
static uint16_t f16_bits(float v) {
    uint32_t b;
    memcpy(&b, &v, 4);
    const int e = (int)((b >> 23) & 0xFF) - 127 + 15;
    return (uint16_t)((e << 10) | ((b >> 13) & 0x3FF));
}

/* Blocks with random quants and scales in the synthetic distributions. */
static void fill_q4k(uint8_t *W, int64_t nblk) {
    for (int64_t i = 0; i < nblk; i++) {
        uint8_t *b = W + 144 * i;
        for (int k = 0; k < 144; k++) b[k] = (uint8_t)next_u32();
        const uint16_t d = f16_bits(1e-3f + 9e-3f * unit()), dm = f16_bits(1e-3f + 9e-3f * unit());
        memcpy(b, &d, 2);
        memcpy(b + 2, &dm, 2);
    }
}
static void fill_q6k(uint8_t *W, int64_t nblk) {
    for (int64_t i = 0; i < nblk; i++) {
        uint8_t *b = W + 210 * i;
        for (int k = 0; k < 208; k++) b[k] = (uint8_t)next_u32();
        for (int k = 192; k < 208; k++) b[k] = (uint8_t)(int8_t)((int)(next_u32() % 128) - 64);
        const uint16_t d = f16_bits(1e-4f + 9e-4f * unit());
        memcpy(b + 208, &d, 2);
    }
}

static void fill_q80(uint8_t *W, int64_t nblk) {
    for (int64_t i = 0; i < nblk; i++) {
        uint8_t *b = W + 34 * i;
        const uint16_t d = f16_bits(1e-3f + 9e-3f * unit());
        memcpy(b, &d, 2);
        for (int k = 2; k < 34; k++) b[k] = (uint8_t)(int8_t)((int)(next_u32() % 255) - 127);
    }
}

static int failures = 0;
#define CHECK_HIP(e)                                                              \
    do {                                                                          \
        hipError_t err_ = (e);                                                    \
        if (err_ != hipSuccess) {                                                 \
            fprintf(stderr, "HIP error %d at line %d\n", (int)err_, __LINE__); \
            exit(2);                                                              \
        }                                                                         \
    } while (0)
#define CHECK_QD(s)                                                                          \
    do {                                                                                     \
        qd_status st_ = (s);                                                                 \
        if (st_ != QD_OK) {                                                                  \
            fprintf(stderr, "qdecode error %s at line %d\n", qd_status_str(st_), __LINE__); \
            exit(3);                                                                         \
        }                                                                                    \
    } while (0)

static void *to_device(const void *h, size_t n) {
    void *d = NULL;
    CHECK_HIP(hipMalloc(&d, n));
    CHECK_HIP(hipMemcpy(d, h, n, hipMemcpyHostToDevice));
    return d;
}

/* got within the bound of the oracle's (y64, S) */
static void within(const char *name, const float *got, const double *y64, const double *S, int64_t n) {
    int bad = 0;
    for (int64_t i = 0; i < n; i++)
        if (!(fabs((double)got[i] - y64[i]) <= 1e-4 * S[i] + 1e-6)) bad++;
    if (bad) {
        fprintf(stderr, "%s: %d of %lld outputs out of bound\n", name, bad, (long long)n);
        failures++;
    }
}

static void gemv_case(int fmt, int64_t N, int64_t K, int batch, hipStream_t s) {
    const int64_t rb = qd_row_bytes((qd_format)fmt, K);
    uint8_t *W = malloc((size_t)(N * rb));
    float *x = malloc(sizeof(float) * (size_t)(batch * K)), *y = malloc(sizeof(float) * (size_t)(batch * N));
    double *y64 = malloc(sizeof(double) * (size_t)(batch * N)), *S = malloc(sizeof(double) * (size_t)(batch * N));
    if (fmt == QD_Q4_K) fill_q4k(W, N * K / 256);
    else fill_q6k(W, N * K / 256);
    for (int64_t i = 0; i < batch * K; i++) x[i] = normalish();
    void *dW = to_device(W, (size_t)(N * rb));
    float *dx = to_device(x, sizeof(float) * (size_t)(batch * K)), *dy = NULL;
    CHECK_HIP(hipMalloc((void **)&dy, sizeof(float) * (size_t)(batch * N)));
    CHECK_QD(qgemv((qd_format)fmt, dW, dx, dy, N, K, batch, s));
    CHECK_HIP(hipStreamSynchronize(s));
    CHECK_HIP(hipMemcpy(y, dy, sizeof(float) * (size_t)(batch * N), hipMemcpyDeviceToHost));
    if (orc_gemv(fmt, W, x, N, K, batch, 0, N, y64, S) != 0) failures++;
    within(fmt == QD_Q4_K ? "qgemv q4_k" : "qgemv q6_k", y, y64, S, batch * N);
    CHECK_HIP(hipFree(dW)); CHECK_HIP(hipFree(dx)); CHECK_HIP(hipFree(dy));
    free(W); free(x); free(y); free(y64); free(S);
}

static void ffn_case(hipStream_t s) {
    const int64_t H = 512, F = 1024;
    const int64_t rbg = qd_row_bytes(QD_Q4_K, H), rbd = qd_row_bytes(QD_Q6_K, F);
    uint8_t *Wg = malloc((size_t)(F * rbg)), *Wu = malloc((size_t)(F * rbg)), *Wd = malloc((size_t)(H * rbd));
    fill_q4k(Wg, F * H / 256);
    fill_q4k(Wu, F * H / 256);
    fill_q6k(Wd, H * F / 256);
    float x[512], nw[512], r[512], y[512], h[1024];
    for (int i = 0; i < 512; i++) {
        x[i] = normalish();
        nw[i] = 1.0f + 0.1f * normalish();
        r[i] = normalish();
    }
    void *dWg = to_device(Wg, (size_t)(F * rbg)), *dWu = to_device(Wu, (size_t)(F * rbg));
    void *dWd = to_device(Wd, (size_t)(H * rbd));
    float *dx = to_device(x, sizeof x), *dnw = to_device(nw, sizeof nw), *dy = to_device(r, sizeof r), *dh = NULL;
    CHECK_HIP(hipMalloc((void **)&dh, sizeof h));
    /* y starts as the residual r and is updated in place: y = FFN(x) + r */
    CHECK_QD(qffn_decode_residual(QD_Q4_K, dWg, dWu, QD_Q6_K, dWd, dx, dnw, 1e-6f, QD_ACT_SILU, dy, dy, dh,
                                  F, H, 1, s));
    CHECK_HIP(hipStreamSynchronize(s));
    CHECK_HIP(hipMemcpy(y, dy, sizeof y, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(h, dh, sizeof h, hipMemcpyDeviceToHost));
    /* stage by stage: the down projection of the GPU's own h, plus r (the h
     * stage itself is checked against the oracle by the Python tests) */
    double y64[512], S[512];
    if (orc_gemv(QD_Q6_K, Wd, h, H, F, 1, 0, H, y64, S) != 0) failures++;
    for (int i = 0; i < 512; i++) {
        y64[i] += r[i];
        /* the residual add is one more fp32 rounding: 2^-23 |y| <= 1e-4 * (1.2e-3 |y|) */
        S[i] += fabs(y64[i]) * 1.2e-3;
    }
    within("qffn_decode_residual", y, y64, S, 512);
    int finite = 1;
    for (int i = 0; i < 1024; i++) finite &= isfinite(h[i]);
    if (!finite) failures++;
    CHECK_HIP(hipFree(dWg)); CHECK_HIP(hipFree(dWu)); CHECK_HIP(hipFree(dWd));
    CHECK_HIP(hipFree(dx)); CHECK_HIP(hipFree(dnw)); CHECK_HIP(hipFree(dy)); CHECK_HIP(hipFree(dh));
    free(Wg); free(Wu); free(Wd);
}

static void int8_case(hipStream_t s) {
    const int64_t N = 300, K = 2560;
    const int batch = 3;
    const int64_t rb = qd_row_bytes(QD_Q8_0, K), nq = batch * K, nd = batch * (K / 32);
    uint8_t *W = malloc((size_t)(N * rb));
    float *x = malloc(sizeof(float) * (size_t)nq), *y = malloc(sizeof(float) * (size_t)(batch * N));
    float *d = malloc(sizeof(float) * (size_t)nd), *d_ref = malloc(sizeof(float) * (size_t)nd);
    int8_t *q = malloc((size_t)nq), *q_ref = malloc((size_t)nq);
    double *y64 = malloc(sizeof(double) * (size_t)(batch * N)), *S = malloc(sizeof(double) * (size_t)(batch * N));
    fill_q80(W, N * K / 32);
    for (int64_t i = 0; i < nq; i++) x[i] = normalish();
    for (int i = 0; i < 32; i++) x[K + i] = 0.0f; /* an all-zero run */
    void *dW = to_device(W, (size_t)(N * rb));
    float *dx = to_device(x, sizeof(float) * (size_t)nq), *dd = NULL, *dy = NULL;
    int8_t *dq = NULL;
    CHECK_HIP(hipMalloc((void **)&dq, (size_t)nq));
    CHECK_HIP(hipMalloc((void **)&dd, sizeof(float) * (size_t)nd));
    CHECK_HIP(hipMalloc((void **)&dy, sizeof(float) * (size_t)(batch * N)));
    CHECK_QD(qquantize_q8_act(dx, dq, dd, K, batch, s));
    CHECK_QD(qgemv_q8_0_preq(dW, dq, dd, dy, N, K, batch, s));
    CHECK_HIP(hipStreamSynchronize(s));
    CHECK_HIP(hipMemcpy(q, dq, (size_t)nq, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(d, dd, sizeof(float) * (size_t)nd, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(y, dy, sizeof(float) * (size_t)(batch * N), hipMemcpyDeviceToHost));
    if (orc_quantize_q8_act(x, K, batch, q_ref, d_ref) != 0) failures++;
    if (memcmp(q, q_ref, (size_t)nq) != 0 || memcmp(d, d_ref, sizeof(float) * (size_t)nd) != 0) {
        fprintf(stderr, "qquantize_q8_act: codes or scales differ from the oracle\n");
        failures++;
    }
    if (orc_gemv_q8_0_q8act(W, q_ref, d_ref, N, K, batch, 0, N, y64, S) != 0) failures++;
    within("qgemv_q8_0_preq", y, y64, S, batch * N);
    CHECK_HIP(hipFree(dW)); CHECK_HIP(hipFree(dx)); CHECK_HIP(hipFree(dq));
    CHECK_HIP(hipFree(dd)); CHECK_HIP(hipFree(dy));
    free(W); free(x); free(y); free(d); free(d_ref); free(q); free(q_ref); free(y64); free(S);
}

int main(void) {
    hipStream_t s;
    CHECK_HIP(hipStreamCreate(&s));
    gemv_case(QD_Q4_K, 512, 512, 1, s);
    gemv_case(QD_Q6_K, 256, 8192, 2, s);
    ffn_case(s);
    int8_case(s);
    /* a rejected call: K not a multiple of 256 */
    if (qgemv_q4k((void *)0x10000, (const float *)0x20000, (float *)0x30000, 4, 100, 1, s) != QD_ESHAPE)
        failures++;
    CHECK_HIP(hipStreamSynchronize(s));
    CHECK_HIP(hipStreamDestroy(s));
    if (failures) {
        fprintf(stderr, "c_abi_example: %d failures\n", failures);
        return 1;
    }
    printf("c_abi_example: ok (qdecode %d)\n", qd_version());
    return 0;
}
