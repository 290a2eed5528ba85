/*
 * oracle.h -- CPU oracle for block-quantized decode GEMV.
 *
 * TEST INFRASTRUCTURE ONLY.  This is the checker that the GPU library is
 * measured against.  Only the test-suite, the smoke check and the benchmark's
 * CPU-baseline leg may load it.  It shares no source, header, table or helper
 * with the HIP library under quantized_decode_q4k_amd/, and it never calls it.
 *
 * Everything here is written for a reader to check by eye against the
 * definitions: every weight is decoded on its own, then dot products are
 * accumulated in fp64.  Nothing is blocked, fused or reordered.
 *
 * Formats (values per block / bytes per block):
 *   ORC_Q4_K  256 / 144    ORC_Q6_K  256 / 210    ORC_Q8_0  32 / 34
 * A matrix of N rows and K columns is N rows of K/QK consecutive blocks with
 * row stride (K/QK)*block_bytes and no padding (dotLLM PR #320, the commit
 * fixing the Q8_0 GEMV row stride to blocksPerRow * 34).
 */
#ifndef QDECODE_ORACLE_H
#define QDECODE_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_Q4_K = 0, ORC_Q6_K = 1, ORC_Q8_0 = 2 };
enum { ORC_ACT_GELU_TANH = 0, ORC_ACT_SILU = 1 };

/* Weights per block and bytes per block; 0 for an unknown format. */
int orc_block_elems(int fmt);
int orc_block_bytes(int fmt);
/* Bytes in one row of K weights; 0 if K is not a positive multiple of the
 * block size. */
int64_t orc_row_bytes(int fmt, int64_t K);

/* IEEE 754 binary16 -> fp32 (exact, subnormals included). */
float orc_f16_to_f32(uint16_t h);
/* fp32 -> bfloat16 with round-to-nearest-even; NaN stays NaN. */
uint16_t orc_f32_to_bf16(float f);
float orc_bf16_to_f32(uint16_t b);

/* Decode one block into fp32 weights (256, 256 or 32 of them). */
void orc_dequant_q4k_block(const uint8_t *blk, float *w);
void orc_dequant_q6k_block(const uint8_t *blk, float *w);
void orc_dequant_q8_0_block(const uint8_t *blk, float *w);

/* Q4_K: the 6-bit scale and min of sub-block j (0..7) of one block. */
void orc_q4k_scale_min(const uint8_t *blk, int j, int *sc, int *m);

/* Decode rows [n0, n1) of an N x K matrix into out[(n - n0) * K + k].
 * Returns 0, or -1 on a bad format or shape. */
int orc_dequant_rows(int fmt, const uint8_t *W, int64_t K, int64_t n0,
                     int64_t n1, float *out);

/* y64[b*N + n] = sum_k w[n][k] * x[b*K + k] and
 * S[b*N + n]   = sum_k |w[n][k] * x[b*K + k]|, both in fp64,
 * for rows n in [n0, n1) and b in [0, batch).  Either output may be NULL.
 * Returns 0, or -1 on a bad format or shape. */
int orc_gemv(int fmt, const uint8_t *W, const float *x, int64_t N, int64_t K,
             int batch, int64_t n0, int64_t n1, double *y64, double *S);

/* Activations quantized to Q8_0 form per run of 32 (dotLLM's pre-quantized
 * input for its Q8_0 GEMM): d = max|x| / 127 in fp32, q = round(x / d) with
 * halves away from zero (fp32 division), zeros for an all-zero run.
 * q: int8 [batch][K], d: fp32 [batch][K/32].  Returns 0 or -1 (K % 32). */
int orc_quantize_q8_act(const float *x, int64_t K, int batch, int8_t *q, float *d);

/* Q8_0 weights against quantized activations: y64 = sum_j dw * dx * sum q*q,
 * S = the same over |products|, fp64, rows [n0, n1).  Returns 0 or -1. */
int orc_gemv_q8_0_q8act(const uint8_t *W, const int8_t *qx, const float *dx, int64_t N, int64_t K,
                        int batch, int64_t n0, int64_t n1, double *y64, double *S);

/* RMS-norm in fp64: out[b*K + k] = x[b*K+k] * w[k] / sqrt(mean_k(x^2) + eps).
 * The weight multiplies directly (any "1 + w" offset is already in w). */
void orc_rmsnorm(const float *x, const float *w, int64_t K, int batch,
                 double eps, double *out);

/* Post-norm and residual (larql Gemma 3 table, post_attn_residual_norm_store
 * and post_ffn_norm_residual_add), fp64, per batch column of N:
 *   y  = r + p * w1 / sqrt(mean(p^2) + eps)
 *   y2 = y * w2 / sqrt(mean(y^2) + eps)     (skipped when w2 or y2 is NULL)
 * p [batch][N] fp64; r [batch][N], w1 [N], w2 [N] fp32. */
void orc_post_norm_residual(const double *p, const float *r, const float *w1, const float *w2,
                            int64_t N, int batch, double eps, double *y, double *y2);

/* Activations in fp64. */
double orc_gelu_tanh(double g);
double orc_silu(double g);
double orc_act(int act, double g);

/* Prefill GEMM with bf16 operands:
 * Y64[m*N + n] = sum_k bf16(w[n][k]) * X[m*K + k]   (X already bf16 bits)
 * S[m*N + n]   = sum_k |bf16(w[n][k]) * X[m*K + k]|
 * for n in [n0, n1), m in [m0, m1); bf16(w) is the round-to-nearest-even
 * bfloat16 of the fp32 dequantised weight.  Either output may be NULL.
 * Outputs are indexed with the full N.  Returns 0 or -1. */
int orc_gemm_bf16(int fmt, const uint8_t *W, const uint16_t *X, int64_t M,
                  int64_t N, int64_t K, int64_t m0, int64_t m1, int64_t n0,
                  int64_t n1, double *Y64, double *S);

#ifdef __cplusplus
}
#endif
#endif
