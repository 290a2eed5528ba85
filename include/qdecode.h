/*
 * qdecode.h -- block-quantized matrix-vector products for transformer decode
 * on AMD Instinct MI355X (gfx950).  C ABI.
 *
 * What is computed.  Every projection of a decoder layer in the engines the
 * source pages describe streams a block-quantized weight matrix against an
 * fp32 activation vector:
 *   - larql "Architecture -> Metal shader map", Gemma 3 table: Q4_K for the
 *     Q/K projections, O (q4k_matvec_8sg), FFN gate+up (q4k_ffn_gate_up_8sg,
 *     followed by the GELU-tanh geglu) and lm_head (q4k_matvec); Q6_K for V
 *     and FFN down (q6k_matvec).  Llama table: the same gate+up kernel with
 *     SiLU instead of GELU-tanh.
 *   - dotLLM PR #320: a direct Q8_0 GEMV (matmul_q8_0) and a tiled Q8_0 GEMM
 *     for multi-token prefill.
 * The kernel is chosen by the weight format (larql's "How dispatch happens
 * today": format predicates, no per-architecture tables); here each format
 * has its own entry point.
 *
 * Block formats (values / bytes per block):
 *   Q4_K  256 / 144: f16 d, f16 dmin, 12 bytes of packed 6-bit scales and
 *                    mins for 8 sub-blocks of 32, 128 bytes of 4-bit quants;
 *                    w = d*scale*q - dmin*min.
 *   Q6_K  256 / 210: 128 bytes low 4 bits, 64 bytes high 2 bits, 16 int8
 *                    scales (one per 16 weights), f16 d; w = d*scale*(q-32).
 *   Q8_0   32 /  34: f16 d, 32 int8 quants; w = d*q.
 * Bit placement inside a block follows the GGUF k-quant layout that the larql
 * page's dispatch table names for its 144-byte GGUF-direct Q4_K extracts.
 *
 * Matrix layout.  A weight matrix of N rows and K columns is N rows stored
 * one after another; row n holds K/QK consecutive blocks and starts at byte
 * n * qd_row_bytes(fmt, K).  There is no padding between rows (dotLLM PR
 * #320, the Q8_0 GEMV row-stride fix: the stride is blocksPerRow * 34).
 *
 * Conventions for every call below.
 *   - All array pointers are DEVICE pointers, owned by the caller, and must
 *     stay valid until the work enqueued on `stream` has finished.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *     enqueues work and returns; nothing is synchronised.  Results are ready
 *     when the stream has completed.
 *   - Outputs are overwritten, never accumulated into.  Inputs are read-only.
 *   - Arguments are checked on the host before anything is enqueued; a bad
 *     argument returns an error code and enqueues nothing.  Launch failures
 *     return QD_ELAUNCH.  A device fault surfaces at the caller's next
 *     synchronisation of the stream.
 *   - Shapes: N, M >= 1; batch in 1..QD_MAX_BATCH (1 for qmoe_ffn_decode);
 *     batches above QD_BATCH_CHUNK run as successive launches of up to
 *     QD_BATCH_CHUNK columns on the same stream (the weights are streamed
 *     once per chunk; dotLLM's batched decode reads them once per batch);
 *     K a positive multiple of
 *     256 for Q4_K and Q6_K, of 32 for Q8_0 (dotLLM's CPU Q8_0 kernels reject
 *     lengths that are not a multiple of the 32-element block).
 *   - Alignment: weight pointers 16-byte aligned; fp32 and bf16 activation
 *     pointers 16-byte aligned; output pointers 4-byte aligned.
 *   - Outputs must not overlap inputs.
 *   - Threads: calls may be made from any host thread.  Calls that keep
 *     partial sums or counters between kernels (split-K launches, h of the
 *     decode FFN, the int8 activation codes, row epilogues) use a
 *     per-(device, stream) workspace that the library allocates on first
 *     need and grows when a larger call needs more; calls on the same stream
 *     are ordered by the stream, so they never share it concurrently.
 *   - HIP graphs: a call made while its stream is being captured never
 *     allocates and never enqueues a memory set: if its workspace would
 *     have to be created or grown, it returns QD_ECAPTURE, enqueues
 *     nothing, and the capture stays valid.  Make one uncaptured call of
 *     each shape on the stream first (the workspace then has its size).  A
 *     workspace that is outgrown later stays allocated until the process
 *     ends, so graphs captured with it stay valid.  Counters in the
 *     workspace return to zero at the end of every kernel that uses them, so
 *     replays need no reset.
 */
#ifndef QDECODE_H
#define QDECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum qd_status {
    QD_OK = 0,
    QD_EINVAL = 1,       /* null pointer, unknown enum, aliasing outputs */
    QD_ESHAPE = 2,       /* N, M, K or batch out of range */
    QD_EALIGN = 3,       /* pointer not aligned as required */
    QD_ELAUNCH = 4,      /* the HIP runtime refused the launch */
    QD_EUNSUPPORTED = 5, /* valid arguments the library has no kernel for */
    QD_ENOMEM = 6,       /* workspace allocation failed */
    QD_ECAPTURE = 7,     /* the stream is capturing and the call would have to
                            create or grow its workspace (nothing enqueued) */
    QD_ETOOBIG = 8       /* the allocation-free call needs more scratch than it
                            holds (nothing enqueued) */
} qd_status;

typedef enum qd_format { QD_Q4_K = 0, QD_Q6_K = 1, QD_Q8_0 = 2 } qd_format;

/* FFN gate activation.  larql Gemma 3 table, "GEGLU activation": GELU with
 * the tanh approximation applied to gate, times up; larql Llama table and
 * the gerbil architecture guide's SwiGLU MLP: SiLU(gate) times up. */
typedef enum qd_act { QD_ACT_GELU_TANH = 0, QD_ACT_SILU = 1 } qd_act;

#define QD_MAX_BATCH 64
/* Columns of x one launch streams the weights for; larger batches run as
 * successive launches of up to this many columns each. */
#define QD_BATCH_CHUNK 8

/* Weights per block (256, 256, 32) and bytes per block (144, 210, 34);
 * 0 for an unknown format. */
int qd_block_elems(qd_format fmt);
int qd_block_bytes(qd_format fmt);

/* Bytes in one row of K weights, or 0 if K is not a positive multiple of the
 * block size. */
int64_t qd_row_bytes(qd_format fmt, int64_t K);

/* Static description of a status code (never NULL). */
const char *qd_status_str(qd_status status);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int qd_version(void);

/*
 * y = W x  (batch-1 to batch-8 GEMV with in-register dequantisation)
 *
 * The decode-path projection: larql's q4k_matvec / q4k_matvec_8sg (Q4_K:
 * Q, K, O, lm_head), q6k_matvec (Q6_K: V, down); dotLLM's matmul_q8_0 (Q8_0).
 *
 *   W      N x K quantized matrix in `fmt` blocks (layout above)
 *   x      fp32 [batch][K], row-major
 *   y      fp32 [batch][N], row-major; y[b][n] = sum_k w[n][k] * x[b][k]
 *
 * Accuracy: |y - y_exact| <= 1e-4 * sum_k |w[n][k] x[b][k]| + 1e-6, where w
 * is the exactly dequantised weight, on every block, including Q4_K blocks
 * whose scale and min terms cancel.  Batch 1-2: each run of 32 activations
 * is staged as 2^-s X with X a 31-bit integer (exact for activations within
 * 2^7 of the run's largest magnitude, else rounded at 2^-31 of it), the
 * products of integer quants and X are summed exactly (int8 dot products),
 * and the block scales are applied per sub-block (Q4_K: scale and min terms
 * combined in fp64 and rounded once; Q6_K, Q8_0: one fp32 product).  Batch
 * 3-8: every weight is formed in fp32 with one rounding (Q4_K: d*scale*q -
 * dmin*min as one fused multiply-add; Q6_K and Q8_0 products are exact)
 * before it meets its activation.  A NaN or infinite activation makes every
 * output it reaches non-finite.
 */
qd_status qgemv_q4k(const void *W, const float *x, float *y, int64_t N,
                    int64_t K, int batch, void *stream);
qd_status qgemv_q6k(const void *W, const float *x, float *y, int64_t N,
                    int64_t K, int batch, void *stream);
qd_status qgemv_q8_0(const void *W, const float *x, float *y, int64_t N,
                     int64_t K, int batch, void *stream);

/* Same as the three above with the format as an argument. */
qd_status qgemv(qd_format fmt, const void *W, const float *x, float *y,
                int64_t N, int64_t K, int batch, void *stream);

/*
 * y = Q8_0 W times x quantized to int8  (opt-in; a different result from
 * qgemv_q8_0)
 *
 * dotLLM PR #320's CPU Q8_0 GEMM runs on pre-quantized input: the activation
 * row is quantized to Q8_0 form and multiplied with integer dot products.
 * Here each run of 32 activations gets d = max|x| / 127 and
 * q = round(x / d) (fp32 division, halves away from zero; zeros for an
 * all-zero run), and
 *   y[b][n] = sum_j dw[n][j] * d[b][j] * sum_i qw[n][32j+i] * q[b][32j+i].
 *
 *   W, N, K, batch   as qgemv_q8_0 (K a multiple of 32; x finite)
 *   x                fp32 [batch][K], 16-byte aligned
 *   y                fp32 [batch][N]
 * Accuracy: within 1e-4 * sum |dw d qw q| + 1e-6 of that quantized sum
 * computed exactly; against the fp32 qgemv_q8_0 it differs by the
 * activation rounding, within 5e-2 * sum|w x| for N(0,1)-like activations.
 * The activations are quantized into the stream's workspace (as
 * qquantize_q8_act does), then multiplied as qgemv_q8_0_preq does: two
 * launches.
 * Errors: as qgemv, QD_ENOMEM; QD_EUNSUPPORTED when the codes one
 * workgroup stages for one column (its K-slice, K/ks bytes plus scales) do
 * not fit its 63 KB of LDS and K cannot be split (more than 65536 row tiles:
 * K > 57344 with N above about 262144).
 */
qd_status qgemv_q8_0_q8act(const void *W, const float *x, float *y, int64_t N, int64_t K,
                          int batch, void *stream);

/*
 * Activations quantized to int8 per run of 32, as qgemv_q8_0_q8act does
 * before its integer dots (dotLLM PR #320: the CPU Q8_0 GEMM runs on input
 * quantized once, then reused).  For run j of column b:
 *   d[b][j] = max|x[b][32j .. 32j+31]| / 127          (fp32, correctly rounded)
 *   q[b][32j+i] = round(x[b][32j+i] / d[b][j])        (fp32 quotient, halves away
 *                                                      from zero; 0 when d = 0)
 *
 *   x   fp32 [batch][K], 16-byte aligned, finite
 *   q   int8 [batch][K], 16-byte aligned (out)
 *   d   fp32 [batch][K / 32], 4-byte aligned (out)
 *   K   a multiple of 32; batch 1..QD_MAX_BATCH
 * Errors: QD_EINVAL (null or overlapping buffers), QD_ESHAPE, QD_EALIGN.
 */
qd_status qquantize_q8_act(const float *x, int8_t *q, float *d, int64_t K, int batch, void *stream);

/*
 * y = Q8_0 W times activations already quantized by qquantize_q8_act:
 *   y[b][n] = sum_j dw[n][j] * d[b][j] * sum_i qw[n][32j+i] * q[b][32j+i]
 * (dotLLM PR #320: Q8_0 GEMM on pre-quantized input).  One quantization can
 * serve every projection of the same activations.  At batch > 1 on a
 * matrix with few row tiles the sum over K is split across workgroups, with
 * partial sums in the stream's workspace (allocated on first need, as the
 * other split-K calls do); the result is deterministic either way.
 *
 *   W, N, K, batch, y  as qgemv_q8_0
 *   q, d               as qquantize_q8_act writes them (q 16-byte aligned)
 * Accuracy: within 1e-4 * sum |dw d qw q| + 1e-6 of the exact sum.
 * Errors: as qgemv_q8_0_q8act.
 */
qd_status qgemv_q8_0_preq(const void *W, const int8_t *q, const float *d, float *y, int64_t N,
                         int64_t K, int batch, void *stream);

/*
 * y = W x + r  (GEMV with the residual add fused into its epilogue)
 *
 * The decoder's residual stream: larql's Gemma 3 table follows the O
 * projection with post_attn_residual_norm_store and the down projection
 * with post_ffn_norm_residual_add; the residual add of both is folded into
 * the GEMV's store here (the norms, which need the whole output row, are not).
 *
 *   fmt, W, x, N, K, batch   as qgemv
 *   r      fp32 [batch][N] residual, 4-byte aligned; it may be y itself
 *          (y += W x in place) but must not otherwise overlap y
 *   y      fp32 [batch][N]; y[b][n] = sum_k w[n][k] x[b][k] + r[b][n]
 * Accuracy: |y - y_exact| <= 1e-4 * sum_k |w x| + 1e-6 + one fp32 rounding
 * of the sum.
 * Errors: as qgemv; QD_EINVAL for a NULL r or an r that overlaps y without
 * being y.
 */
qd_status qgemv_residual(qd_format fmt, const void *W, const float *x, const float *r, float *y,
                         int64_t N, int64_t K, int batch, void *stream);

/*
 * y = r + RMSNorm(W x; post_w),  y2 = RMSNorm(y; next_w)   (GEMV with the
 * post-norm, residual and next-norm epilogue)
 *
 * The post-norm pipeline of the larql Gemma 3 table ("has_post_norms", four
 * norms per layer): after the O projection, post_attn_residual_norm_store
 * applies the post-attention RMS-norm to the projection, adds the residual,
 * applies the FFN input norm to the sum and stores both; after the down
 * projection, post_ffn_norm_residual_add applies the post-FFN RMS-norm and
 * adds the residual (the next layer's input).  Per batch column b:
 *   p      = W x[b]                                 (the GEMV)
 *   y[b]   = r[b] + p * post_w / sqrt(mean(p^2) + eps)
 *   y2[b]  = y[b] * next_w / sqrt(mean(y[b]^2) + eps)   (only with next_w)
 * The norm of p needs the whole output row: every workgroup stores its
 * rows of p in the stream's workspace (device-coherent stores), and the
 * last workgroup to finish (a device-scope counter, counted only after its
 * stores have completed) forms y and y2 with sums in a fixed order.
 *
 *   fmt, W, x, N, K, batch   as qgemv
 *   post_w  fp32 [N] post-norm weight, multiplied directly (the page's
 *           "weight offset baked into stored weight")
 *   eps     added to the mean square inside each square root
 *   r       fp32 [batch][N] residual; may be y itself (in place), must not
 *           otherwise overlap y or y2
 *   y       fp32 [batch][N]
 *   next_w  fp32 [N] or NULL; y2 fp32 [batch][N] or NULL (both or neither)
 * Accuracy: p meets the GEMV bound; y and y2 carry that error through the
 * norm (relative error of 1/rms at most
 * sum_n (2|p_n| e_n + e_n^2) / (2 sum_n p_n^2 + 2 N eps) for per-element GEMV
 * errors e_n) plus a few fp32 roundings.
 * Errors: as qgemv; QD_EINVAL for a NULL post_w or r, next_w without y2 (or
 * the reverse), overlapping buffers; QD_ENOMEM, QD_ECAPTURE (workspace).
 */
qd_status qgemv_post_norm_residual(qd_format fmt, const void *W, const float *x, const float *post_w,
                                   float eps, const float *r, float *y, const float *next_w, float *y2,
                                   int64_t N, int64_t K, int batch, void *stream);

/*
 * q = Wq xn,  k = Wk xn,  v = Wv xn,  xn = RMSNorm(x) if norm_w != NULL else x
 *
 * The attention input projections of one decoder layer in one launch: the
 * larql Gemma 3 table fuses the input RMS-norm with the Q, K and V
 * projections (Q and K in Q4_K, V in Q6_K, "Q4_K_M" mix) into one dispatch;
 * here each matrix may have its own format.
 *
 *   fmt_q, Wq, Nq   Q projection, Nq x K
 *   fmt_k, Wk, Nk   K projection, Nk x K
 *   fmt_v, Wv, Nv   V projection, Nv x K
 *   x               fp32 [batch][K]
 *   norm_w, eps     RMS-norm as in qffn_gate_up_act (NULL = no norm)
 *   q, k, v         fp32 [batch][Nq], [batch][Nk], [batch][Nv]; they must not
 *                   overlap each other or any input
 *   K               a multiple of 256 when any matrix is Q4_K or Q6_K (of 32
 *                   when all are Q8_0)
 * Accuracy: each output meets the GEMV bound for xn.  One launch when K is
 * a multiple of 256 and every matrix's staged activations fit one
 * workgroup's LDS (at batch 1 on the streaming kernel, the CUs shared in
 * proportion to the matrices' bytes; at batch 2-8 K up to 14592 in Q4_K on
 * the register kernel); otherwise the same bound from three GEMV launches.
 * Needs no workspace.
 * Errors: as qgemv for each matrix (QD_ESHAPE, QD_EALIGN, QD_EINVAL).
 */
qd_status qqkv_proj(qd_format fmt_q, const void *Wq, int64_t Nq, qd_format fmt_k,
                    const void *Wk, int64_t Nk, qd_format fmt_v, const void *Wv, int64_t Nv,
                    const float *x, const float *norm_w, float eps, float *q, float *k,
                    float *v, int64_t K, int batch, void *stream);

/*
 * h = act(Wg xn) * (Wu xn),  xn = RMSNorm(x) if norm_w != NULL else x
 *
 * The fused FFN gate+up of larql's q4k_ffn_gate_up_8sg with the geglu
 * element-wise step folded into its epilogue, and the input RMS-norm of the
 * larql Gemma 3 table folded into the staging of x.
 *
 *   fmt     format of both Wg and Wu (Q4_K in the Gemma FFN)
 *   Wg, Wu  N_ff x K quantized matrices (gate, up)
 *   x       fp32 [batch][K]
 *   norm_w  fp32 [K] RMS-norm weight, or NULL for no norm.  The norm is
 *           xn = x * norm_w / sqrt(mean(x^2) + eps): the weight multiplies
 *           directly (larql: "weight offset baked into stored weight").
 *   eps     added to mean(x^2) inside the square root (ignored without norm)
 *   act     QD_ACT_GELU_TANH: 0.5 g (1 + tanh(sqrt(2/pi)(g + 0.044715 g^3)))
 *           QD_ACT_SILU:      g / (1 + exp(-g))
 *   h       fp32 [batch][N_ff]
 *   g_out, u_out  optional fp32 [batch][N_ff] copies of the gate and up
 *           projections (NULL = not written)
 * Accuracy: g and u each meet the GEMV bound; h = act(g) * u evaluated in
 * fp32 from them.
 */
qd_status qffn_gate_up_act(qd_format fmt, const void *Wg, const void *Wu,
                           const float *x, const float *norm_w, float eps,
                           qd_act act, float *h, float *g_out, float *u_out,
                           int64_t N_ff, int64_t K, int batch, void *stream);

/*
 * y = Wd h,  h = act(Wg xn) * (Wu xn),  xn = RMSNorm(x) if norm_w else x
 *
 * The whole decode FFN of one layer (larql Gemma 3 table: input norm ->
 * q4k_ffn_gate_up_8sg -> geglu -> q6k_matvec), as qffn_gate_up_act followed
 * by qgemv on the same stream, with h kept in the library's workspace.
 *
 *   fmt_gu, Wg, Wu   gate and up, N_ff x K
 *   fmt_down, Wd     down, K x N_ff
 *   x                fp32 [batch][K];  norm_w, eps, act as in qffn_gate_up_act
 *   y                fp32 [batch][K]
 *   h_out            optional fp32 [batch][N_ff] copy of h (NULL = kept in
 *                    the library's workspace), 16-byte aligned
 * Accuracy: h as in qffn_gate_up_act; y meets the GEMV bound for the h it
 * was computed from.
 * Errors: as qffn_gate_up_act and qgemv, QD_ENOMEM, QD_ECAPTURE.
 */
qd_status qffn_decode(qd_format fmt_gu, const void *Wg, const void *Wu, qd_format fmt_down,
                      const void *Wd, const float *x, const float *norm_w, float eps, qd_act act,
                      float *y, float *h_out, int64_t N_ff, int64_t K, int batch, void *stream);

/*
 * y = Wd h + r,  h = act(Wg xn) * (Wu xn)   (qffn_decode with the residual
 * add of larql's post_ffn_norm_residual_add folded into the down store)
 *
 * Arguments as qffn_decode, plus r: fp32 [batch][K] residual, 4-byte
 * aligned, which may be y itself (y += FFN(x) in place) but must not
 * otherwise overlap y or h_out.
 * Errors: as qffn_decode; QD_EINVAL for a NULL or overlapping r.
 */
qd_status qffn_decode_residual(qd_format fmt_gu, const void *Wg, const void *Wu,
                               qd_format fmt_down, const void *Wd, const float *x,
                               const float *norm_w, float eps, qd_act act, const float *r,
                               float *y, float *h_out, int64_t N_ff, int64_t K, int batch,
                               void *stream);

/*
 * qffn_decode without any allocation, for callers that cannot allocate
 * device memory: code running under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.
 *
 * Same arguments, results (bit for bit) and kernels as qffn_decode; h (when
 * h_out is NULL), split-K partial sums and counters live in a fixed scratch
 * array the library holds on each GPU it runs on (8 MiB of floats plus
 * 272 KB of counters, kept until the process ends), not in the stream's
 * workspace.  Nothing is allocated, ever: the scratch's address on the
 * current device is looked up once (hipGetSymbolAddress), and each call
 * that uses it first clears its counters with a small kernel on `stream`.
 * Every call on one GPU shares that GPU's scratch, whatever the stream:
 * calls that overlap on one GPU (concurrent streams, or host threads
 * without ordering) race and give wrong results.
 * Limit: batch <= QD_BATCH_CHUNK columns need h plus the larger launch's
 * partial sums within the 2^21 floats (e.g. the Gemma-4-31B FFN at batch 8
 * needs about 1.2 M); a call that needs more returns QD_ETOOBIG with
 * nothing enqueued.
 * Errors: as qffn_decode (never QD_ENOMEM or QD_ECAPTURE), QD_ETOOBIG.
 */
qd_status qffn_decode_noalloc(qd_format fmt_gu, const void *Wg, const void *Wu, qd_format fmt_down,
                              const void *Wd, const float *x, const float *norm_w, float eps, qd_act act,
                              float *y, float *h_out, int64_t N_ff, int64_t K, int batch, void *stream);

/*
 * y = r + RMSNorm(Wd h; post_w),  y2 = RMSNorm(y; next_w),
 * h = act(Wg xn) * (Wu xn)   (qffn_decode with the post_ffn_norm_residual_add
 * epilogue of the larql Gemma 3 table on the down projection)
 *
 * Arguments as qffn_decode, plus post_w, r, next_w and y2 as in
 * qgemv_post_norm_residual (r, y, y2 are [batch][K]); eps serves the input
 * norm and both post norms.  In the Gemma 3 pipeline x is already
 * normalised by the previous call's next_w, so norm_w is NULL there.
 * Errors: as qffn_decode and qgemv_post_norm_residual.
 */
qd_status qffn_decode_post_norm_residual(qd_format fmt_gu, const void *Wg, const void *Wu,
                                         qd_format fmt_down, const void *Wd, const float *x,
                                         const float *norm_w, float eps, qd_act act, const float *post_w,
                                         const float *r, float *y, const float *next_w, float *y2,
                                         float *h_out, int64_t N_ff, int64_t K, int batch, void *stream);

/*
 * y = sum_z coef[z] * Wd[e_z] h_z,  h_z = act(Wg[e_z] xn) * (Wu[e_z] xn),
 * e_z = ids[z], z < n_sel, xn = RMSNorm(x) if norm_w else x   (batch 1)
 *
 * The mixture-of-experts FFN of one decode token (larql's MoE table: each
 * routed expert's gate+up with the activation, then its down projection,
 * the expert outputs combined with the router's weights).  The expert ids
 * and weights are device arrays, read by the kernels (no host round trip),
 * so a router running on the GPU can feed this call inside a graph.
 *
 *   fmt_gu, Wg, Wu  n_experts stacked N_ff x K matrices each (expert e at
 *                   byte offset e * N_ff * qd_row_bytes(fmt_gu, K))
 *   fmt_down, Wd    n_experts stacked K x N_ff matrices (expert e at byte
 *                   offset e * K * qd_row_bytes(fmt_down, N_ff))
 *   ids             int32 [n_sel] expert per slot (repeats allowed; an id
 *                   outside [0, n_experts) makes its slot contribute zero)
 *   coef            fp32 [n_sel] routing weight per slot
 *   n_sel           1..64 selected slots
 *   x, norm_w, eps, act   as qffn_gate_up_act (one token: x is fp32 [K])
 *   y               fp32 [K], overwritten
 *   h_out           optional fp32 [n_sel][N_ff] (16-byte aligned) copy of
 *                   every slot's h (NULL = kept in the workspace)
 * Accuracy: each h_z as in qffn_gate_up_act; y within
 * sum_z |coef[z]| (1e-4 sum|w h_z| + 1e-6) plus the fp32 rounding of the
 * weighted sum, for the h it was computed from.  The slots are summed in
 * slot order (deterministic).
 * Errors: QD_ESHAPE (shapes, n_experts < 1, n_sel outside 1..64),
 * QD_EINVAL (NULL pointers, bad act, outputs overlapping inputs),
 * QD_EALIGN, QD_EUNSUPPORTED when K or N_ff does not fit one workgroup's
 * LDS (rows of whole 256-weight superunits: the streaming kernel's staged
 * digits and ring; other rows: K or N_ff up to 14592 in Q4_K).  Calls that
 * overlap on one stream's workspace race.
 */
qd_status qmoe_ffn_decode(qd_format fmt_gu, const void *Wg, const void *Wu, qd_format fmt_down,
                          const void *Wd, int n_experts, const int32_t *ids, const float *coef,
                          int n_sel, const float *x, const float *norm_w, float eps, qd_act act,
                          float *y, float *h_out, int64_t N_ff, int64_t K, void *stream);

/*
 * Y = X W^T for a multi-token prefill: the weights are dequantised to bf16
 * and contracted on the bf16 matrix cores with fp32 accumulation.  dotLLM
 * PR #320 (Vulkan backend section) adds a tiled Q8_0 GEMM for multi-token
 * prefill, which is the pages' instance; here any of the three formats.
 *
 *   W   N x K quantized matrix (rows of qd_row_bytes(fmt, K) bytes), device,
 *       16-byte aligned
 *   X   bf16 bits [M][K], row-major, device, 16-byte aligned
 *   Y   fp32 [M][N], row-major, device, 4-byte aligned; written, never read
 *       Y[m][n] = sum_k bf16(w[n][k]) * X[m][k], where bf16(w) is the
 *       round-to-nearest-even bfloat16 of the exact fp32 dequantised weight
 *   M   tokens, 1 <= M and M * K < 2^31
 * Accuracy: |Y - Y_exact| <= 1e-4 * sum_k |bf16(w) X| + 1e-6.
 * Errors: QD_ESHAPE (M, N or K out of range, K not a multiple of the block),
 * QD_EINVAL (null pointer, Y overlapping W or X), QD_EALIGN, QD_ENOMEM
 * (split-K workspace), QD_ELAUNCH.  Shapes with few output tiles split K
 * across workgroups through the per-stream workspace; partial sums are
 * added in a fixed order, so results are deterministic.
 */
qd_status qgemm_prefill(qd_format fmt, const void *W, const uint16_t *X,
                        float *Y, int64_t M, int64_t N, int64_t K,
                        void *stream);

/*
 * H = bf16( act(X Wg^T) * (X Wu^T) ) for a prefill FFN: the two prefill
 * GEMMs share X and the activation product is taken in fp32 in the
 * epilogue (GELU-tanh geglu of the larql Gemma 3 table, or SiLU), then
 * rounded to bf16 (nearest even) so that H feeds qgemm_prefill for the down
 * projection.
 *
 *   Wg, Wu  N_ff x K quantized matrices, device, 16-byte aligned
 *   X       bf16 bits [M][K], device, 16-byte aligned
 *   H       bf16 bits [M][N_ff], device, 2-byte aligned
 *   g_out, u_out  optional fp32 [M][N_ff] gate and up products (NULL = no)
 * Errors as qgemm_prefill, plus QD_EINVAL for an unknown act.
 */
qd_status qgemm_prefill_gate_up_act(qd_format fmt, const void *Wg,
                                    const void *Wu, const uint16_t *X,
                                    qd_act act, uint16_t *H, float *g_out,
                                    float *u_out, int64_t M, int64_t N_ff,
                                    int64_t K, void *stream);

/*
 * out = dequantised W, fp32 [N][K] (exact: the single rounding of the real
 * value of each weight), or its round-to-nearest-even bf16 bits.  dotLLM PR
 * #320's CPU kernels have the same operation for one row
 * (DequantizeRowToF32); here it serves the tests, which check the
 * in-kernel decoders bit for bit against the oracle.
 *   W    N x K quantized matrix, device, 16-byte aligned
 *   out  fp32 [N][K] (4-byte aligned) or bf16 bits [N][K] (2-byte aligned),
 *        device, must not overlap W
 * Errors: QD_ESHAPE, QD_EINVAL (null pointer, unknown format, overlap),
 * QD_EALIGN, QD_ELAUNCH.
 */
qd_status qdequant(qd_format fmt, const void *W, float *out, int64_t N,
                   int64_t K, void *stream);
qd_status qdequant_bf16(qd_format fmt, const void *W, uint16_t *out,
                        int64_t N, int64_t K, void *stream);

/*
 * Launch-shape override for tuning sweeps (process-wide; 0 = automatic).
 *   p_in   K-slices interleaved inside one workgroup (1, 2, 4, 8, 16; also
 *          the lane groups per row of qgemv_q8_0_preq / qgemv_q8_0_q8act)
 *   p_out  K-slices across workgroups (>= 1; > 1 uses the split-K workspace)
 *   nr     rows per lane group for plain GEMV (1 or 2)
 * Returns QD_EINVAL for values outside these sets.
 */
qd_status qd_set_launch_override(int p_in, int p_out, int nr);

/*
 * Batch path of qgemv*, qffn_gate_up_act and qffn_decode* at batch 3..64
 * (process-wide; tuning and comparisons):
 *   0  automatic: the matrix-core kernels, which stream the weights once
 *      per call for every batch row (integer products of the quants with
 *      the activations' digits, the same result class as batch 1..2)
 *   1  the fp32 register kernel, in launches of up to 8 batch rows
 * k_slices: K-slices across workgroups of the matrix-core kernels (0 =
 * automatic; else 1..1024, capped at the row's superunits of 256 weights).
 * Returns QD_EINVAL for other values.
 */
qd_status qd_set_batch_override(int mode, int k_slices);

/*
 * Row slots each lane group of the register-streaming GEMV walks one after
 * another (process-wide; 0 = automatic, else 1..64).  Larger values give
 * each workgroup more rows for the one staging of its activation slice.
 * Returns QD_EINVAL outside 0..64.
 */
qd_status qd_set_walk_override(int rows_per_group);

/*
 * Tile override of the prefill GEMMs (0 = automatic): tm = 2 or 4 (tokens
 * per workgroup / 32), splits = K-splits across workgroups (1..1024; more
 * than the K-tiles of 128 weights is clamped).
 */
qd_status qd_set_gemm_override(int tm, int splits);

/*
 * Stream-K scheduling of the prefill GEMMs (process-wide tuning knob).
 * units_per_wg: 0 = off (whole tiles, or the planned K-split), > 0 = each
 * workgroup takes that many consecutive (tile, K-tile of 128 weights) units
 * in tile-major order.  A tile shared by several workgroups is summed by the
 * last to arrive in workgroup order, so results do not depend on timing
 * (they differ from the unsplit sums by the order of fp32 additions).
 * Returns QD_EINVAL below 0.
 */
qd_status qd_set_gemm_streamk(int units_per_wg);

/*
 * Shape override of the streaming GEMV path (process-wide; 0 = automatic).
 *   wg_per_cu  workgroups per CU (1..8; LDS is divided between them)
 *   depth      steps of 16 superunits in flight per copying wave (1..32,
 *              capped by what the ring and the wait counter allow)
 *   consumers  decoding waves beside the copying waves (4 or 8; 0 = 8)
 *   producers  copying waves (1, 2 or 4; 0 = automatic)
 * A non-zero wg_per_cu forces the streaming path where the shape allows it.
 * Returns QD_EINVAL for values outside these sets.
 */
qd_status qd_set_stream_override(int wg_per_cu, int depth, int consumers, int producers);

/*
 * Launch plan qgemv_q8_0_preq / qgemv_q8_0_q8act would use for this shape,
 * computed on the host without any HIP call (tests and tuning):
 *   out[0] lane groups per row, out[1] K-slices across workgroups,
 *   out[2] superunits (256 weights) per slice, out[3] columns per launch
 *   (0 = the shape is not supported: QD_EUNSUPPORTED from those calls).
 * Errors: QD_ESHAPE / QD_EINVAL as qgemv_q8_0 (out must not be NULL).
 */
qd_status qd_plan_q8act(int64_t N, int64_t K, int batch, int32_t *out);

#ifdef __cplusplus
}
#endif
#endif /* QDECODE_H */
