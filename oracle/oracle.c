/*
 * oracle.c -- CPU oracle for block-quantized decode GEMV.
 *
 * TEST INFRASTRUCTURE ONLY (see oracle.h).  Plain C, one weight at a time,
 * fp64 accumulation.  Parity pins for every function live in
 * tests/test_oracle_pins.py.
 *
 * What the pages fix, and what is a reading:
 *  - larql "Architecture -> Metal shader map", dispatch predicate table: the
 *    Q4_K weights larql reads directly from llama.cpp-saved GGUF files use
 *    the 144-byte block.  Its Gemma 3 table runs Q4_K (Q, K, O, gate, up,
 *    lm_head) and Q6_K (V, down) under the ollama Q4_K_M convention.
 *  - dotLLM PR #320, commit on the Q8_0 GEMV row-stride fix: a Q8_0 block is
 *    34 bytes (blocksPerRow * 34) and rows are packed without padding; the
 *    commit on CPU Q8_0 kernels gives the 32-element block.
 *  - The field lists and value formulas (w = d*sc*q - dmin*m for Q4_K,
 *    w = d*scale*(q-32) for Q6_K, w = d*q for Q8_0) come with the workload
 *    definitions this library is measured on.
 *  - Reading: no page prints the bit placement inside a block.  The layout
 *    below is the GGUF k-quant layout the larql page names, restated field by
 *    field; little-endian throughout.
 */
#include "oracle.h"

#include <math.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>

int orc_block_elems(int fmt) {
    switch (fmt) {
    case ORC_Q4_K: return 256;
    case ORC_Q6_K: return 256;
    case ORC_Q8_0: return 32;
    default: return 0;
    }
}

int orc_block_bytes(int fmt) {
    switch (fmt) {
    case ORC_Q4_K: return 144;
    case ORC_Q6_K: return 210;
    case ORC_Q8_0: return 34;
    default: return 0;
    }
}

int64_t orc_row_bytes(int fmt, int64_t K) {
    int qk = orc_block_elems(fmt);
    if (qk == 0 || K <= 0 || K % qk != 0) return 0;
    return (K / qk) * (int64_t)orc_block_bytes(fmt);
}

static uint16_t rd_u16(const uint8_t *p) {
    return (uint16_t)(p[0] | (p[1] << 8));
}

/* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 * exponent 0 -> subnormal, value = fraction * 2^-24;
 * exponent 31 -> infinity (fraction 0) or NaN;
 * otherwise value = (1024 + fraction) * 2^(exponent - 25). */
float orc_f16_to_f32(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int f = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);
    return (float)(sign ? -v : v);
}

/* bfloat16 keeps the top 16 bits of the fp32 encoding.  Round to nearest,
 * ties to even, done on the value: find the two neighbouring bfloat16 values
 * and pick the nearer one. */
uint16_t orc_f32_to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if (isnan(f)) return (uint16_t)((u >> 16) | 0x0040); /* quiet NaN */
    if (isinf(f)) return (uint16_t)(u >> 16);
    uint32_t lo = u & 0xFFFF0000u;             /* truncation toward zero */
    uint32_t hi = lo + 0x00010000u;            /* next value away from zero */
    float flo, fhi;
    memcpy(&flo, &lo, 4);
    memcpy(&fhi, &hi, 4);
    double vlo = (double)flo;
    /* past the largest finite bf16 the next value is 2^128, i.e. overflow to
     * infinity; the distance is taken to 2^128 as IEEE rounding does */
    double vhi = isinf(fhi) ? copysign(ldexp(1.0, 128), (double)f) : (double)fhi;
    double dlo = fabs((double)f - vlo);
    double dhi = fabs(vhi - (double)f);
    if (dlo < dhi) return (uint16_t)(lo >> 16);
    if (dhi < dlo) return (uint16_t)(hi >> 16);
    /* exact tie: the even one (low bit of the bf16 fraction clear) */
    return (uint16_t)((((lo >> 16) & 1) == 0) ? (lo >> 16) : (hi >> 16));
}

float orc_bf16_to_f32(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* ---------------------------------------------------------------- Q4_K ---
 * 144 bytes:  [0,2) d (f16)   [2,4) dmin (f16)
 *             [4,16) s[0..11]: eight 6-bit scales and eight 6-bit mins
 *             [16,144) qs[0..127]: 256 four-bit quants
 * Sub-block j (0..7) covers weights 32j..32j+31.
 *  j < 4: scale = low 6 bits of s[j], min = low 6 bits of s[j+4].
 *  j >= 4: scale = low nibble of s[j+4], with the top 2 bits of s[j-4] as
 *          bits 4..5; min = high nibble of s[j+4], with the top 2 bits of
 *          s[j] as bits 4..5.
 * Quants: the 128 bytes form four runs of 32; run c holds weights
 * 64c..64c+31 in its low nibbles and 64c+32..64c+63 in its high nibbles.
 * Weight i = d*scale_j*q_i - dmin*min_j with j = i/32. */
void orc_q4k_scale_min(const uint8_t *blk, int j, int *sc, int *m) {
    const uint8_t *s = blk + 4;
    if (j < 4) {
        *sc = s[j] & 63;
        *m = s[j + 4] & 63;
    } else {
        *sc = (s[j + 4] & 15) | ((s[j - 4] >> 6) << 4);
        *m = (s[j + 4] >> 4) | ((s[j] >> 6) << 4);
    }
}

void orc_dequant_q4k_block(const uint8_t *blk, float *w) {
    double d = orc_f16_to_f32(rd_u16(blk));
    double dmin = orc_f16_to_f32(rd_u16(blk + 2));
    const uint8_t *qs = blk + 16;
    for (int i = 0; i < 256; i++) {
        int j = i / 32;
        int run = i / 64;
        int pos = i % 64;
        uint8_t byte = qs[32 * run + pos % 32];
        int q = (pos < 32) ? (byte & 15) : (byte >> 4);
        int sc, m;
        orc_q4k_scale_min(blk, j, &sc, &m);
        /* d*sc*q has at most 11+6+4 significant bits and dmin*m at most
         * 11+6, so both products are exact in fp64; the difference is exact
         * unless the exponents are more than 32 apart, and then the larger
         * term (exact in fp32) is the correctly rounded result either way.
         * The cast to float is therefore the single correct rounding of the
         * real value d*sc*q - dmin*m. */
        w[i] = (float)(d * sc * q - dmin * m);
    }
}

/* ---------------------------------------------------------------- Q6_K ---
 * 210 bytes:  [0,128) ql: low 4 bits of each quant
 *             [128,192) qh: high 2 bits of each quant
 *             [192,208) sc[0..15]: int8 scales, one per 16 weights
 *             [208,210) d (f16)
 * The block is two halves of 128 weights.  In half h, weight
 * 128h + 32g + l (g = 0..3, l = 0..31) takes
 *   low 4 bits:  byte ql[64h + 32*(g%2) + l], low nibble for g < 2,
 *                high nibble for g >= 2;
 *   high 2 bits: bits 2g..2g+1 of byte qh[32h + l].
 * q = low | high << 4 (0..63); weight i = d * sc[i/16] * (q - 32). */
void orc_dequant_q6k_block(const uint8_t *blk, float *w) {
    const uint8_t *ql = blk;
    const uint8_t *qh = blk + 128;
    const int8_t *sc = (const int8_t *)(blk + 192);
    double d = orc_f16_to_f32(rd_u16(blk + 208));
    for (int i = 0; i < 256; i++) {
        int h = i / 128;
        int g = (i % 128) / 32;
        int l = i % 32;
        uint8_t lbyte = ql[64 * h + 32 * (g % 2) + l];
        int lo = (g < 2) ? (lbyte & 15) : (lbyte >> 4);
        int hi = (qh[32 * h + l] >> (2 * g)) & 3;
        int q = lo | (hi << 4);
        /* 11 + 7 + 6 significant bits: exact in fp32 */
        w[i] = (float)(d * sc[i / 16] * (q - 32));
    }
}

/* ---------------------------------------------------------------- Q8_0 ---
 * 34 bytes:  [0,2) d (f16)   [2,34) q[0..31] (int8)
 * weight i = d * q_i. */
void orc_dequant_q8_0_block(const uint8_t *blk, float *w) {
    double d = orc_f16_to_f32(rd_u16(blk));
    const int8_t *q = (const int8_t *)(blk + 2);
    for (int i = 0; i < 32; i++) w[i] = (float)(d * q[i]);
}

static void dequant_block(int fmt, const uint8_t *blk, float *w) {
    if (fmt == ORC_Q4_K) orc_dequant_q4k_block(blk, w);
    else if (fmt == ORC_Q6_K) orc_dequant_q6k_block(blk, w);
    else orc_dequant_q8_0_block(blk, w);
}

int orc_dequant_rows(int fmt, const uint8_t *W, int64_t K, int64_t n0,
                     int64_t n1, float *out) {
    int64_t rb = orc_row_bytes(fmt, K);
    if (rb == 0 || n0 < 0 || n1 < n0) return -1;
    int qk = orc_block_elems(fmt), bb = orc_block_bytes(fmt);
    for (int64_t n = n0; n < n1; n++)
        for (int64_t b = 0; b < K / qk; b++)
            dequant_block(fmt, W + n * rb + b * bb, out + (n - n0) * K + b * qk);
    return 0;
}

/* ----------------------------------------------------------------- GEMV ---
 * The product every projection on the decode path computes: the larql
 * Gemma 3 table's q4k_matvec (lm_head), q4k_matvec_8sg (O), q6k_matvec
 * (down); dotLLM's matmul_q8_0 ("direct quantized GEMV against Q8_0-packed
 * weights").  Written as the definition: decode row n, then sum w*x. */
int orc_gemv(int fmt, const uint8_t *W, const float *x, int64_t N, int64_t K,
             int batch, int64_t n0, int64_t n1, double *y64, double *S) {
    int64_t rb = orc_row_bytes(fmt, K);
    if (rb == 0 || batch < 1 || n0 < 0 || n1 < n0 || n1 > N) return -1;
    float *w = (float *)malloc(sizeof(float) * (size_t)K);
    if (!w) return -1;
    for (int64_t n = n0; n < n1; n++) {
        orc_dequant_rows(fmt, W, K, n, n + 1, w);
        for (int b = 0; b < batch; b++) {
            double acc = 0.0, acc_abs = 0.0;
            for (int64_t k = 0; k < K; k++) {
                double p = (double)w[k] * (double)x[(int64_t)b * K + k];
                acc += p;
                acc_abs += fabs(p);
            }
            if (y64) y64[(int64_t)b * N + n] = acc;
            if (S) S[(int64_t)b * N + n] = acc_abs;
        }
    }
    free(w);
    return 0;
}

/* ----------------------------------------- int8-quantized activations ---
 * dotLLM PR #320, the CPU Q8_0 kernel work (GemmQ8_0 with pre-quantized
 * input): the activation row is itself quantized to Q8_0 form before the
 * integer dot product.  Per run of 32 activations: d = max|x| / 127 (fp32);
 * q = x / d (fp32 division) rounded to the nearest integer, halves away from
 * zero; a run of zeros has d = 0 and q = 0.  K must be a multiple of 32. */
int orc_quantize_q8_act(const float *x, int64_t K, int batch, int8_t *q, float *d) {
    if (K <= 0 || K % 32 != 0 || batch < 1) return -1;
    for (int64_t r = 0; r < (int64_t)batch * (K / 32); r++) {
        const float *xr = x + 32 * r;
        float amax = 0.0f;
        for (int i = 0; i < 32; i++) {
            float a = fabsf(xr[i]);
            if (a > amax) amax = a;
        }
        float dr = amax / 127.0f;
        d[r] = dr;
        for (int i = 0; i < 32; i++) {
            float v = dr > 0.0f ? roundf(xr[i] / dr) : 0.0f;
            q[32 * r + i] = (int8_t)v;
        }
    }
    return 0;
}

/* Q8_0 weights against int8-quantized activations (from orc_quantize_q8_act):
 * y64[b*N + n] = sum over 32-runs j of dw[n][j] * dx[b][j] * sum_i qw * qx,
 * S[b*N + n] the same with every product's absolute value, both in fp64, for
 * rows [n0, n1).  Returns 0, or -1 on a bad shape. */
int orc_gemv_q8_0_q8act(const uint8_t *W, const int8_t *qx, const float *dx, int64_t N, int64_t K,
                        int batch, int64_t n0, int64_t n1, double *y64, double *S) {
    const int64_t rb = orc_row_bytes(ORC_Q8_0, K);
    if (rb == 0 || batch < 1 || n0 < 0 || n1 < n0 || n1 > N) return -1;
    const int64_t nb = K / 32;
    for (int64_t n = n0; n < n1; n++) {
        const uint8_t *row = W + n * rb;
        for (int b = 0; b < batch; b++) {
            double acc = 0.0, acc_abs = 0.0;
            for (int64_t j = 0; j < nb; j++) {
                const uint8_t *blk = row + 34 * j;
                const double dw = (double)orc_f16_to_f32(rd_u16(blk));
                const double dxj = (double)dx[(int64_t)b * nb + j];
                const int8_t *qw = (const int8_t *)(blk + 2);
                const int8_t *qa = qx + ((int64_t)b * nb + j) * 32;
                for (int i = 0; i < 32; i++) {
                    const double p = dw * dxj * (double)qw[i] * (double)qa[i];
                    acc += p;
                    acc_abs += fabs(p);
                }
            }
            if (y64) y64[(int64_t)b * N + n] = acc;
            if (S) S[(int64_t)b * N + n] = acc_abs;
        }
    }
    return 0;
}

/* ------------------------------------------------------------- RMS-norm ---
 * larql Gemma 3 table, "Input RMS-norm": standard RMS-norm with the weight
 * offset baked into the stored weight, so the weight multiplies directly.
 * x / sqrt(mean(x^2) + eps) * w, eps inside the square root. */
void orc_rmsnorm(const float *x, const float *w, int64_t K, int batch,
                 double eps, double *out) {
    for (int b = 0; b < batch; b++) {
        const float *xb = x + (int64_t)b * K;
        double ss = 0.0;
        for (int64_t k = 0; k < K; k++) ss += (double)xb[k] * (double)xb[k];
        double inv = 1.0 / sqrt(ss / (double)K + eps);
        for (int64_t k = 0; k < K; k++)
            out[(int64_t)b * K + k] = (double)xb[k] * inv * (double)w[k];
    }
}

/* ----------------------------------------------- Post-norm residual ---
 * larql "Architecture -> Metal shader map", Gemma 3 table ("has_post_norms":
 * four norms per layer): after the O projection, post_attn_residual_norm_store
 * (the post-attention RMS-norm of the projection, the residual add, the FFN
 * input norm of the sum, both stored); after the down projection,
 * post_ffn_norm_residual_add (the post-FFN RMS-norm of the projection added
 * to the residual, the next layer's input).  Reading: the post-norm order
 * of that pipeline -- the norm applies to the projection before the
 * residual add -- with each weight multiplied directly, as in orc_rmsnorm:
 *   y[n]  = r[n] + p[n] * w1[n] / sqrt(mean(p^2) + eps)
 *   y2[n] = y[n] * w2[n] / sqrt(mean(y^2) + eps)        (when w2 and y2)
 * per batch column; p in fp64 (the exact projection), everything in fp64. */
void orc_post_norm_residual(const double *p, const float *r, const float *w1, const float *w2,
                            int64_t N, int batch, double eps, double *y, double *y2) {
    for (int b = 0; b < batch; b++) {
        const double *pb = p + (int64_t)b * N;
        const float *rb = r + (int64_t)b * N;
        double *yb = y + (int64_t)b * N;
        double ss = 0.0;
        for (int64_t n = 0; n < N; n++) ss += pb[n] * pb[n];
        const double inv = 1.0 / sqrt(ss / (double)N + eps);
        for (int64_t n = 0; n < N; n++) yb[n] = (double)rb[n] + pb[n] * inv * (double)w1[n];
        if (w2 && y2) {
            double ss2 = 0.0;
            for (int64_t n = 0; n < N; n++) ss2 += yb[n] * yb[n];
            const double inv2 = 1.0 / sqrt(ss2 / (double)N + eps);
            for (int64_t n = 0; n < N; n++) y2[(int64_t)b * N + n] = yb[n] * inv2 * (double)w2[n];
        }
    }
}

/* ---------------------------------------------------------- Activations ---
 * larql Gemma 3 table, "GEGLU activation": the GELU-tanh variant applied to
 * gate, times up.  GELU with the tanh approximation (Hendrycks & Gimpel):
 *   0.5 g (1 + tanh( sqrt(2/pi) (g + 0.044715 g^3) )).
 * larql Llama table and the gerbil guide's SwiGLU MLP: SiLU on gate, times
 * up.  SiLU(g) = g / (1 + exp(-g)). */
double orc_gelu_tanh(double g) {
    const double pi = 3.14159265358979323846;
    const double k = sqrt(2.0 / pi);
    return 0.5 * g * (1.0 + tanh(k * (g + 0.044715 * g * g * g)));
}

double orc_silu(double g) { return g / (1.0 + exp(-g)); }

double orc_act(int act, double g) {
    return act == ORC_ACT_SILU ? orc_silu(g) : orc_gelu_tanh(g);
}

/* -------------------------------------------------------- Prefill GEMM ---
 * Multi-token prefill against quantized weights (dotLLM's tiled Q8_0 GEMM
 * for prefill is the pages' instance).  Here the operands are bfloat16:
 * each fp32 dequantised weight rounded to bf16, the activations given as
 * bf16; products summed in fp64. */
int orc_gemm_bf16(int fmt, const uint8_t *W, const uint16_t *X, int64_t M,
                  int64_t N, int64_t K, int64_t m0, int64_t m1, int64_t n0,
                  int64_t n1, double *Y64, double *S) {
    int64_t rb = orc_row_bytes(fmt, K);
    if (rb == 0 || m0 < 0 || m1 < m0 || m1 > M || n0 < 0 || n1 < n0 || n1 > N)
        return -1;
    float *w = (float *)malloc(sizeof(float) * (size_t)K);
    if (!w) return -1;
    for (int64_t n = n0; n < n1; n++) {
        orc_dequant_rows(fmt, W, K, n, n + 1, w);
        for (int64_t k = 0; k < K; k++) w[k] = orc_bf16_to_f32(orc_f32_to_bf16(w[k]));
        for (int64_t m = m0; m < m1; m++) {
            double acc = 0.0, acc_abs = 0.0;
            for (int64_t k = 0; k < K; k++) {
                double p = (double)w[k] * (double)orc_bf16_to_f32(X[m * K + k]);
                acc += p;
                acc_abs += fabs(p);
            }
            if (Y64) Y64[m * N + n] = acc;
            if (S) S[m * N + n] = acc_abs;
        }
    }
    free(w);
    return 0;
}
