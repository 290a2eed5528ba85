// qd_internal.h -- declarations shared by the HIP translation units of the
// library (launchers and argument blocks).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qd {

enum Fmt : int { kQ4K = 0, kQ6K = 1, kQ80 = 2 };

// Every format is processed in "superunits" of 256 weights: one Q4_K or Q6_K
// block, or eight Q8_0 blocks.  Four lanes share a superunit, 64 weights each.
constexpr int kSuper = 256;
constexpr int kThreads = 256;            // threads per workgroup (4 waves)
constexpr int kGroups = kThreads / 4;    // lane groups per workgroup
constexpr int kLdsBudgetBytes = 65536 - 1024;  // dynamic LDS per workgroup (two fit on a CU)

// Row epilogue of a GEMV (qd_epilogue.h): y = r + RMSNorm(p; w1) and
// optionally y2 = RMSNorm(y; w2), formed by the last workgroup to finish.
struct PostNorm {
    const float *w1 = nullptr;  // post-norm weight [N]; nullptr = no epilogue
    const float *w2 = nullptr;  // next-norm weight [N] or nullptr
    const float *r = nullptr;   // residual [batch][N] (may be the output)
    float *y2 = nullptr;        // [batch][N] when w2 is given
    float *p = nullptr;         // workspace [batch][N]: the projection
    unsigned *ctr = nullptr;    // completed row tiles (zero between launches)
    unsigned tiles = 0;         // row tiles of the launch
    float eps = 0.f;
};

// Arguments of the GEMV / fused gate-up kernels.
struct MvArgs {
    const uint8_t *W0;      // row stream 0: the matrix (GEMV) or gate (FFN)
    const uint8_t *W1;      // row stream 1: up (FFN); unused for GEMV
    const float *x;         // [batch][K]
    const float *norm_w;    // [K] or nullptr
    float *y;               // GEMV: [batch][N]; FFN: h [batch][N]
    const float *res;       // GEMV: optional [batch][N] added to y (may equal y)
    float *g_out;           // FFN optional [batch][N]
    float *u_out;           // FFN optional [batch][N]
    float *partials;        // split-K: [p_out][batch][nr][N]
    unsigned *counters;     // split-K: one per row tile, zero between calls
    int64_t N;              // output rows
    int64_t K;              // columns
    int64_t row_bytes;      // bytes per weight row
    int nb;                 // superunits per row, ceil(K / 256)
    int nblk;               // format blocks per row (Q8_0: K / 32)
    int nk;                 // superunits per K-slice (split across workgroups)
    int p_in;               // K-interleave inside a workgroup
    int p_out;              // K-slices across workgroups (gridDim.y)
    int rpg;                // row slots each lane group walks (0 or 1: one)
    int act;                // qd_act
    float eps;
    // Mixture-of-experts decode (moe_kernel): slot z of the launch uses
    // expert ids[z] of n_experts stacked matrices (w_estride bytes apart).
    // Gate/up: slot z writes y + z * y_sstride.  Down: slot z reads
    // x + z * x_sstride over the whole row and is split-K slice z, and the
    // slices are summed with weights coef[z].
    const int32_t *ids;
    const float *coef;
    int64_t w_estride, x_sstride, y_sstride;
    int n_experts;
    PostNorm pn;            // GEMV row epilogue (pn.w1 = nullptr: none)
};

struct Shape {
    int p_in;
    int p_out;
    int nr;   // row streams per lane group: 2 for FFN (gate, up); 1 or 2 for GEMV
    int rpg = 1;  // row slots walked by each lane group
};

// Launchers (qd_gemv.hip).
// LDS bytes the GEMV kernel needs for `nk` staged superunits of `batch` rows.
size_t mv_lds_bytes(int fmt, int batch, int nk);
hipError_t launch_gemv(int fmt, int batch, bool ffn, MvArgs a, Shape s, hipStream_t st);
// Mixture-of-experts decode GEMVs (qd_gemv.hip), batch 1, n_sel slots:
// gate/up (ffn) on a (tiles, 1, n_sel) grid, down on (tiles, n_sel).
hipError_t launch_moe(int fmt, bool ffn, const MvArgs &a, int64_t tiles, int n_sel, hipStream_t st);

// Q8_0 GEMV on int8-quantized activations (qd_gemv_i8.hip), and the
// quantizer (x [runs][32] -> q int8 codes, d fp32 scale per run).
struct Q8ActArgs {
    const uint8_t *W;       // N x K Q8_0
    const int8_t *q;        // [batch][K] codes, 16-byte aligned
    const float *d;         // [batch][K / 32] scales
    float *y;               // [batch][N]
    int64_t N, K, row_bytes;
    int p;                  // lane groups per row (1, 2, 4, 8, 16)
    int off_scales;         // LDS byte offset of the activation scales
    int ks, su_per;         // K-slices across workgroups (grid.y) and superunits per slice
    float *partials;        // ks > 1: [ks][batch][N] partial sums
    unsigned *counters;     // ks > 1: one per row tile, zero between launches
};
size_t q8act_lds_bytes(int batch, int64_t K);
hipError_t launch_q8act(const Q8ActArgs &a, int batch, unsigned grid, hipStream_t st);
hipError_t launch_q8quant(const float *x, int8_t *q, float *d, int64_t runs, hipStream_t st);

// Fused Q/K/V projection (qd_gemv.hip): three GEMVs over the same activation
// rows in one launch.  Workgroups [0, tiles[0]) are row tiles of matrix 0,
// the next tiles[1] of matrix 1, then tiles[2] of matrix 2; each runs the
// GEMV tile of its own format with no split across workgroups (a[i].p_out
// must be 1 and a[i].nk == a[i].nb).
struct QkvArgs {
    MvArgs a[3];
    int fmt[3];
    int tiles[3];
};
hipError_t launch_qkv(const QkvArgs &q, int batch, size_t lds, hipStream_t st);

// Dequantisers (qd_dequant.hip).
hipError_t launch_dequant(int fmt, const uint8_t *W, float *out, uint16_t *out_bf16,
                          int64_t N, int64_t K, hipStream_t st);

// Streaming GEMV (qd_gemv_stream.hip): one workgroup per row range, weights
// copied through an LDS ring.
struct StreamArgs {
    const uint8_t *W0;      // weights (gate for the fused FFN)
    const uint8_t *W1;      // up (fused FFN) or nullptr
    const float *x;         // [batch][K], 16-byte aligned
    const float *norm_w;    // optional RMS-norm weight [K]
    float *y, *g_out, *u_out;
    const float *res;       // GEMV: optional [batch][N] added to y (may equal y)
    int64_t N, K;
    int64_t row_bytes;
    int64_t mat_bytes;      // N * row_bytes, a multiple of 16
    int nb;                 // superunits per row (K / 256)
    int rows_base, rows_extra;  // workgroup i owns rows_base + (i < rows_extra) rows
    int units_max;          // (rows_base + (rows_extra > 0)) * nb
    int consumers;          // decoding waves (4 or 8)
    int producers;          // copying waves (1, 2 or 4)
    int slots;              // ring slots (steps)
    int lag;                // steps in flight per copying wave
    int off_x, off_part, off_red;  // LDS layout (bytes): staged digits, row partials, flags
    int act;
    float eps;
    PostNorm pn;            // GEMV row epilogue (pn.w1 = nullptr: none)
    // routed experts of the MoE decode FFN (launch_stream_moe): n_sel * wps
    // workgroups, wps per slot; expert e's matrices at W + e * w_estride
    const int32_t *ids;
    const float *coef;
    int n_experts, n_sel, wps;
    int64_t w_estride;
    int64_t x_sstride, y_sstride;  // down: h_z at x + z * x_sstride; gate/up: h_z at y + z * y_sstride
    float *part;                   // down: [n_sel][N] slot rows
    unsigned *counters;            // down: [wps], zero between launches
};
size_t stream_pc_layout(int fmt, int batch, bool ffn, int nb, int units_max, int slots,
                        StreamArgs *a);
int stream_copies_per_step(int fmt, bool ffn);
hipError_t launch_stream(int fmt, int batch, bool ffn, const StreamArgs &a, unsigned grid,
                         size_t lds, hipStream_t st);
hipError_t launch_stream_moe(int fmt, bool ffn, const StreamArgs &a, unsigned grid, size_t lds,
                             hipStream_t st);
// Q/K/V in one streaming launch (batch 1): wgs[i] workgroups for matrix i
// (format fmt[i], plain GEMV arguments a[i], each with 8 decoding waves).
struct StreamQkvArgs {
    StreamArgs a[3];
    int fmt[3];
    int wgs[3];
};
hipError_t launch_stream_qkv(const StreamQkvArgs &q, size_t lds, hipStream_t st);

// Batch 3..64 GEMVs on the matrix cores (qd_gemv_mfma.hip).  xdig_kernel
// writes the activation digits of up to 64 batch rows in groups of 8: per
// (group, superunit) the A-operand fragments of its 8 runs (1 KB each) and
// a record per run and batch row ({scale, scale * sum X} as two doubles for
// Q4_K, the scale as a float otherwise).  mq_kernel streams 128 weight rows
// per workgroup over a K-slice of nk superunits (gridDim.y slices, split-K
// partials summed by the last workgroup of a row tile).
constexpr int kFragRun = 1024;        // bytes of one run's A operand (8 batch rows)
// Weight rows per workgroup (4 waves of 32 rows): 128 of one matrix, or 64
// rows of both gate and up for the fused FFN.
__host__ __device__ constexpr int mq_tile_rows(bool ffn) { return ffn ? 64 : 128; }
struct XdArgs {
    const float *x;         // [batch][K], 16-byte aligned
    const float *norm_w;    // [K] or nullptr
    float eps;
    uint8_t *dig;           // [ng][nb] superunits of digits (mq_su_bytes_host each)
    int64_t K;
    int R;                  // runs of activations (K / 32)
    int nb;                 // superunits (ceil(K / 256))
    int batch;
};
struct MqArgs {
    const uint8_t *W0;      // the matrix (GEMV) or gate (FFN)
    const uint8_t *W1;      // up (FFN)
    const uint8_t *dig;     // xdig_kernel's output
    float *y, *g_out, *u_out;
    const float *res;       // GEMV: optional [batch][N] added to y (may equal y)
    float *partials;        // split-K: [p_out][batch][1 or 2][N]
    unsigned *counters;     // split-K: one per row tile, zero between calls
    int64_t N, K, row_bytes;
    int nb;                 // superunits per row
    int nblk;               // format blocks per row
    int nk;                 // superunits per K-slice
    int batch;
    int act;
    PostNorm pn;            // GEMV row epilogue (pn.w1 = nullptr: none)
    // FFN: h also written as the activation digits of the down projection
    // (its K is this launch's N), in xdig_kernel's layout; y may then be
    // nullptr (h not kept in fp32)
    uint8_t *hdig;          // nullptr: none
    int hd_nb;              // down superunits per row (N / 256)
    int hd_sx;              // the down format takes run sums (Q4_K)
};
size_t mq_su_bytes_host(int fmt);      // digits bytes per (group, superunit)
size_t mq_lds_bytes(int fmt, int ng);
int xdig_max_k();                      // longest row xdig_kernel takes
int mq_wg_per_cu(int fmt, int ng, bool ffn);  // resident workgroups per CU
hipError_t launch_xdig(const XdArgs &a, int ng, bool sx, hipStream_t st);
hipError_t launch_mq(int fmt, int ng, bool ffn, const MqArgs &a, unsigned tiles, unsigned p_out,
                     hipStream_t st);

// Prefill GEMM (qd_prefill.hip).  A workgroup owns 32*tm tokens by 256
// output columns (plain: 256 weight rows; FFN: 128 rows of gate and of up)
// over K-tiles [kt_per_split*ks, ...) of 128 weights.
constexpr int kGemmKT = 128;          // weights per K-tile
constexpr int kGemmCols = 256;        // accumulator columns per workgroup
struct GemmArgs {
    const uint8_t *Wg;      // weights (or gate for the FFN variant)
    const uint8_t *Wu;      // up (FFN variant) or nullptr
    const uint16_t *X;      // bf16 [M][K]
    float *Y;               // fp32 [M][N] (plain GEMM)
    uint16_t *H;            // bf16 [M][N] (FFN variant)
    float *g_out;           // optional fp32 [M][N] (FFN variant)
    float *u_out;
    float *partials;        // split-K: tiles * splits, stream-K: 2 * grid partial tiles of 32*tm * kGemmCols floats
    unsigned *counters;     // split-K: one per output tile, zero between calls
    int64_t M, N, K;
    int64_t row_bytes;
    int nblk;               // quant blocks per row
    int kt_total;           // ceil(K / kGemmKT)
    int kt_per_split;
    int splits;
    int m_tiles, n_tiles;
    int act;
    int sk_per;             // stream-K: (tile, K-tile) units per workgroup; 0 = split-K
};
hipError_t launch_gemm(int fmt, bool ffn, int tm, const GemmArgs &a, hipStream_t st);

}  // namespace qd
