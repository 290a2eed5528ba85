/*
 * Host-only driver that calls every entry point of the C oracle on small
 * seeded inputs, edge shapes and rejected arguments.  tests/test_oracle_sanitizers.py
 * builds it together with oracle/oracle.c under AddressSanitizer and
 * UndefinedBehaviorSanitizer (gcc, no GPU code) and checks that it runs clean.
 * Inputs are arbitrary bytes, so decoded values may be NaN or infinite; only
 * memory safety, defined behaviour and the return codes are checked here (the
 * values are pinned by the oracle's own tests).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../oracle/oracle.h"

static uint64_t state = 0x5EEDull;

static uint32_t next_u32(void) {
    /* SplitMix64 step (test data only) */
    uint64_t z = (state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return (uint32_t)((z ^ (z >> 31)) >> 32);
}

static void fill_bytes(uint8_t *p, size_t n) {
    for (size_t i = 0; i < n; i++) p[i] = (uint8_t)next_u32();
}

static float small_float(void) { return (float)((int)(next_u32() % 2001) - 1000) / 500.0f; }

static int fails = 0;
#define CHECK(c)                                                            \
    do {                                                                    \
        if (!(c)) {                                                         \
            fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
            fails++;                                                        \
        }                                                                   \
    } while (0)

static void one_format(int fmt, int64_t N, int64_t K, int batch) {
    const int64_t rb = orc_row_bytes(fmt, K);
    CHECK(rb > 0);
    uint8_t *W = malloc((size_t)(N * rb));
    float *x = malloc(sizeof(float) * (size_t)(batch * K));
    float *deq = malloc(sizeof(float) * (size_t)(N * K));
    double *y = malloc(sizeof(double) * (size_t)(batch * N));
    double *S = malloc(sizeof(double) * (size_t)(batch * N));
    fill_bytes(W, (size_t)(N * rb));
    for (int64_t i = 0; i < batch * K; i++) x[i] = small_float();

    CHECK(orc_dequant_rows(fmt, W, K, 0, N, deq) == 0);
    CHECK(orc_dequant_rows(fmt, W, K, 1, N, deq) == 0);
    CHECK(orc_gemv(fmt, W, x, N, K, batch, 0, N, y, S) == 0);
    CHECK(orc_gemv(fmt, W, x, N, K, batch, N / 2, N, y, NULL) == 0);
    CHECK(orc_gemv(fmt, W, x, N, K, batch, 0, 1, NULL, S) == 0);
    CHECK(orc_gemv(fmt, W, x, N, K, batch, 0, 0, y, S) == 0);

    /* bf16 GEMM over a token and row sub-range */
    const int64_t M = 3;
    uint16_t *X = malloc(sizeof(uint16_t) * (size_t)(M * K));
    double *Y = malloc(sizeof(double) * (size_t)(M * N));
    for (int64_t i = 0; i < M * K; i++) X[i] = orc_f32_to_bf16(small_float());
    CHECK(orc_gemm_bf16(fmt, W, X, M, N, K, 0, M, 0, N, Y, NULL) == 0);
    CHECK(orc_gemm_bf16(fmt, W, X, M, N, K, 1, 2, N - 1, N, Y, Y) == 0);

    /* rejected shapes and formats */
    CHECK(orc_dequant_rows(9, W, K, 0, N, deq) == -1);
    CHECK(orc_gemv(9, W, x, N, K, batch, 0, N, y, S) == -1);
    CHECK(orc_gemv(fmt, W, x, N, K + 1, batch, 0, N, y, S) == -1);
    CHECK(orc_gemm_bf16(9, W, X, M, N, K, 0, M, 0, N, Y, NULL) == -1);

    free(W); free(x); free(deq); free(y); free(S); free(X); free(Y);
}

int main(void) {
    /* sizes */
    CHECK(orc_block_elems(ORC_Q4_K) == 256 && orc_block_bytes(ORC_Q4_K) == 144);
    CHECK(orc_block_elems(ORC_Q6_K) == 256 && orc_block_bytes(ORC_Q6_K) == 210);
    CHECK(orc_block_elems(ORC_Q8_0) == 32 && orc_block_bytes(ORC_Q8_0) == 34);
    CHECK(orc_block_elems(7) == 0 && orc_block_bytes(-1) == 0);
    CHECK(orc_row_bytes(ORC_Q4_K, 100) == 0 && orc_row_bytes(ORC_Q8_0, 0) == 0);

    /* every binary16 pattern, and bf16 rounding of special values */
    volatile float acc = 0.f;
    for (uint32_t h = 0; h < 65536; h++) acc += orc_f16_to_f32((uint16_t)h) * 0.f;
    const float specials[] = {0.f, -0.f, 1.f, -1.f, INFINITY, -INFINITY, NAN, 3.4028235e38f, 1e-45f};
    for (size_t i = 0; i < sizeof specials / sizeof specials[0]; i++)
        acc += orc_bf16_to_f32(orc_f32_to_bf16(specials[i])) * 0.f;

    /* single blocks of arbitrary bytes, and every Q4_K scale/min slot */
    uint8_t blk[210];
    float w[256];
    for (int r = 0; r < 64; r++) {
        fill_bytes(blk, sizeof blk);
        orc_dequant_q4k_block(blk, w);
        orc_dequant_q6k_block(blk, w);
        orc_dequant_q8_0_block(blk, w);
        for (int j = 0; j < 8; j++) {
            int sc = -1, m = -1;
            orc_q4k_scale_min(blk, j, &sc, &m);
            CHECK(sc >= 0 && sc < 64 && m >= 0 && m < 64);
        }
    }

    /* matrices: ragged row counts, several blocks per row, odd Q8_0 counts */
    one_format(ORC_Q4_K, 5, 512, 3);
    one_format(ORC_Q6_K, 7, 768, 2);
    one_format(ORC_Q8_0, 3, 96, 4);
    one_format(ORC_Q8_0, 2, 160, 1);

    /* norm and activations */
    float xs[2 * 64], nw[64];
    double out[2 * 64];
    for (int i = 0; i < 128; i++) xs[i] = small_float();
    for (int i = 0; i < 64; i++) nw[i] = 1.0f + small_float() / 10.f;
    orc_rmsnorm(xs, nw, 64, 2, 1e-6, out);
    for (int i = -40; i <= 40; i++) {
        acc += (float)orc_gelu_tanh(i * 0.5) * 0.f;
        acc += (float)orc_silu(i * 0.5) * 0.f;
        acc += (float)orc_act(ORC_ACT_GELU_TANH, i) * 0.f + (float)orc_act(ORC_ACT_SILU, -i) * 0.f;
    }
    (void)acc;
    if (fails) return 1;
    printf("oracle sanitizer driver: ok\n");
    return 0;
}
