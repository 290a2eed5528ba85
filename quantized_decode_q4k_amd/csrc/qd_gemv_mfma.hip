// qd_gemv_mfma.hip -- batch 3..64 GEMVs and fused gate/up on the matrix
// cores, the weights streamed once per call.
//
// What is computed is the same y = sum_k w_k x_k as everywhere in this
// library (larql "Architecture -> Metal shader map": the Q4_K / Q6_K
// matvec and gate/up rows of the Gemma 3 and Gemma 4 tables; dotLLM PR #320:
// matmul_q8_0 and the batched ForwardBatch GEMM that streams each weight
// once for all the tokens of a step).  The arithmetic is the integer form of
// qd_digits.h, spread over the matrix cores:
//
//  * Activations (normalised first when an RMS-norm weight is given) are
//    written once per call by xdig_kernel as the 31-bit integers X of each
//    run of 32 (one exponent per run and batch row), split into four signed
//    byte planes.  The planes of 8 batch rows form the A operand of one
//    v_mfma_i32_32x32x32_i8: 32 A rows = (batch row bb, plane p) at row
//    bb + 8p, 32 k = the run's activations.  One 1 KB "fragment" per (group
//    of 8 batch rows, run), laid out exactly as the 64 lanes read it
//    (lane l: row l % 32, k = 16 (l / 32) .. +15).
//  * A wave owns 32 weight rows; its 64 lanes hold the integer quants of
//    one sub-block of those rows as the B operand (lane l: row l % 32, the
//    16 quants k = 16 (l / 32) .. +15).  The product is, for every (batch
//    row, plane, weight row), the exact integer sum of quant x digit over
//    the sub-block.  The output registers of lane l hold all four planes of
//    the batch rows 4 (l / 32) .. +3 for its weight row, so the planes are
//    recombined and the block scales applied in the lane: Q4_K in fp64
//    (d sc 2^-s I - dmin m 2^-s sum X, no cancellation), Q6_K and Q8_0 in
//    fp32, as in the batch-1..2 kernels.
//  * Q6_K sub-blocks hold 16 weights: one instruction takes the two
//    sub-blocks of a run, A rows 0..15 (4 batch rows x 4 planes) seeing only
//    k < 16 and rows 16..31 only k >= 16 (the other half of A is zero), so
//    each lane still loads 16 consecutive quant bytes.
//
// A workgroup is 4 waves, 128 weight rows, over a K-slice of superunits.
// While one superunit is multiplied the next one's weight tile (32 rows of
// the wave, whole 16-byte pieces of each row's contiguous block; Q6_K
// blocks are 2-byte aligned, which the copies read unaligned) is copied
// straight into the wave's second LDS tile slot by global_load_lds, and its
// digit fragments and run records into the second digit buffer the same
// way (or, where only one digit buffer fits beside two resident
// workgroups, into registers, stored after the multiply); every copy has
// landed at the end of the iteration (vmcnt 0, then a barrier).  No weight
// byte passes through vector registers before the B-layout read out of
// LDS, which keeps a wave at about 110 registers.  Split-K slices end in
// the deterministic last-arriver sum of qd_epilogue.h.
#include <type_traits>

#include "qd_digits.h"
#include "qd_epilogue.h"
#include "qd_lds.h"

namespace qd {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

// ------------------------------------------------------ activation digits ---
// Bytes of one superunit (8 runs) of one group of 8 batch rows: the 8 runs'
// fragments, then their records (RR bytes per run: 8 records).  The
// digits of a call are [group][superunit] of these, the layout the matrix
// kernel copies to LDS as it is.
__host__ __device__ constexpr int mq_su_bytes(int rr) { return 8 * kFragRun + 8 * rr; }

// A workgroup of four waves per (batch row, four superunits) of ng * 8 rows
// by ceil(nb / 4) (rows past `batch`, and runs past K / 32, are written as
// zeros): wave w takes superunit 4 blockIdx.y + w, lane l its float4 l (8
// consecutive lanes = one run).  With an RMS-norm weight every workgroup
// first forms its row's mean square itself (each thread's float4 of the
// row, all loaded before the first is used, then a fixed-order workgroup
// sum), so the digit pass is one launch over many CUs with no hand-off.
constexpr int kXdThreads = 256;
constexpr int kXdMaxK = 32768;  // longest row the matrix kernel takes
constexpr int kXdF = kXdMaxK / 4 / kXdThreads;  // float4 of the row per thread
template <bool NORM, bool SX>
__global__ __launch_bounds__(kXdThreads) void xdig_kernel(XdArgs a) {
    __shared__ float red[kXdThreads / 64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int b = blockIdx.x;
    const int t = 4 * blockIdx.y + wave;  // this wave's superunit (uniform)
    const bool live = b < a.batch;
    const int F = a.R * 8;  // float4 of the row
    const float *xb = a.x + (int64_t)b * a.K;
    const int f = 64 * t + lane;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    float4 w = make_float4(1.f, 1.f, 1.f, 1.f);
    if (live && t < a.nb && f < F) {
        v = *reinterpret_cast<const float4 *>(xb + 4 * (int64_t)f);
        if (NORM) w = *reinterpret_cast<const float4 *>(a.norm_w + 4 * (int64_t)f);
    }
    if (NORM) {
        // the row's sum of squares: thread tid adds float4 tid, tid + 256, ...
        // in order (loaded together, up to kXdF), then the workgroup's fixed
        // cross-lane and cross-wave order
        float ss = 0.f;
        if (live) {
            float4 r[kXdF];
#pragma unroll
            for (int i = 0; i < kXdF; i++) {
                const int ff = tid + kXdThreads * i;
                r[i] = make_float4(0.f, 0.f, 0.f, 0.f);
                if (ff < F) r[i] = *reinterpret_cast<const float4 *>(xb + 4 * (int64_t)ff);
            }
#pragma unroll
            for (int i = 0; i < kXdF; i++) {
                ss = fmaf(r[i].x, r[i].x, ss);
                ss = fmaf(r[i].y, r[i].y, ss);
                ss = fmaf(r[i].z, r[i].z, ss);
                ss = fmaf(r[i].w, r[i].w, ss);
            }
        }
        ss = block_total<kXdThreads>(ss, red);
        const float ir = 1.0f / sqrtf(ss / (float)a.K + a.eps);
        v.x = v.x * ir * w.x;
        v.y = v.y * ir * w.y;
        v.z = v.z * ir * w.z;
        v.w = v.w * ir * w.w;
    }
    if (t >= a.nb) return;  // uniform per wave, after the workgroup's barriers
    constexpr int RR = SX ? 128 : 32;
    const int g = b >> 3, bb = b & 7, q = lane & 7;
    uint32_t pl[4];
    double sc, sxs;
    digitize_run<SX>(v, pl, sc, sxs);  // all 8 lanes of every run take part
    const int run = f >> 3;
    uint8_t *su = a.dig + ((int64_t)g * a.nb + t) * mq_su_bytes(RR);
    uint8_t *fr = su + (run & 7) * kFragRun;
#pragma unroll
    for (int p = 0; p < 4; p++)
        *reinterpret_cast<uint32_t *>(fr + 16 * (bb + 8 * p + 32 * (q >> 2)) + 4 * (q & 3)) = pl[p];
    if (q == 0) {
        uint8_t *rec = su + 8 * kFragRun + (run & 7) * RR;
        if constexpr (SX) {
            double2 rr;
            rr.x = sc;
            rr.y = sxs;
            reinterpret_cast<double2 *>(rec)[bb] = rr;
        } else {
            reinterpret_cast<float *>(rec)[bb] = (float)sc;
        }
    }
}

// The same digits from a run held by the 32 lanes of a half-wave (lane & 31
// = the activation's index in the run, one value each; all 64 lanes of the
// wave take part): the run's largest magnitude and plane sums by cross-lane
// reductions, then each lane writes its four digit bytes, and lane 0 of the
// half the run's record.  su: the run's superunit of its group; bb: the
// batch row within the group; r8: the run within the superunit.
template <typename T>
QD_DEV T half_max(T m) {
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) m = max(m, (T)__shfl_xor((int)m, o));
    return m;
}
QD_DEV int half_sum(int v) {
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) v += __shfl_xor(v, o);
    return v;
}
template <bool SX>
QD_DEV void digitize_half(float v, uint8_t *su, int bb, int r8) {
    const int k = threadIdx.x & 31;
    const uint32_t m = half_max<uint32_t>(fbits(v) & 0x7FFFFFFFu);
    const bool bad = m >= 0x7F800000u;
    const int E = (int)(m >> 23) - 126;
    const int s = 30 - E;
    const int X = (int)rintf(ldexpf(v, s));
    const uint32_t y = (uint32_t)X + 0x80808080u;
    uint8_t *fr = su + r8 * kFragRun + 16 * (bb + 32 * (k >> 4)) + (k & 15);
    int ds[4];
#pragma unroll
    for (int p = 0; p < 4; p++) {
        const int dp = (int)((y >> (8 * p)) & 0xFFu) - 128;  // digit p, balanced
        fr[16 * 8 * p] = (uint8_t)dp;
        ds[p] = dp;
    }
    double sxs = 0.0;
    const double sc = bad ? __builtin_nan("") : ldexp(1.0, -s);
    if constexpr (SX) {
        const int s0 = half_sum(ds[0]), s1 = half_sum(ds[1]), s2 = half_sum(ds[2]), s3 = half_sum(ds[3]);
        sxs = fma((double)(s3 * 256 + s2), 65536.0, (double)(s1 * 256 + s0)) * sc;
    }
    if (k == 0) {
        uint8_t *rec = su + 8 * kFragRun + r8 * (SX ? 128 : 32);
        if constexpr (SX) {
            double2 r;
            r.x = sc;
            r.y = sxs;
            reinterpret_cast<double2 *>(rec)[bb] = r;
        } else {
            reinterpret_cast<float *>(rec)[bb] = (float)sc;
        }
    }
}
// h of gate/up row `row` (the down's activation index) for batch slot b.
QD_DEV void emit_h_digit(const MqArgs &a, float hv, int b, int64_t row) {
    const int run = (int)(row >> 5);
    const int g = b >> 3, bb = b & 7;
    uint8_t *su = a.hdig + ((int64_t)g * a.hd_nb + (run >> 3)) * mq_su_bytes(a.hd_sx ? 128 : 32);
    if (a.hd_sx) digitize_half<true>(hv, su, bb, run & 7);
    else digitize_half<false>(hv, su, bb, run & 7);
}

// --------------------------------------------------- per-lane weight bytes ---
// One lane's bytes of one superunit of its row: lane half h = lane / 32.
template <int FMT>
struct MqW;
// Q4_K: the header, and bytes 16h..16h+15 of each 32-byte quant run c
// (sub-block 2c in the low nibbles, 2c+1 in the high ones).
template <>
struct MqW<kQ4K> {
    uint4 hd;
    uint4 q[4];
};
// Q6_K: for each half H of the block, ql bytes 64H + 16h .. +15 (A) and
// 64H + 32 + 16h .. +15 (B), qh bytes 32H + 16h .. +15; the 16 scales and d.
template <>
struct MqW<kQ6K> {
    uint4 ql[2][2];
    uint4 qh[2];
    uint4 sc;
    uint32_t d;
};
// Q8_0: quants 16h..16h+15 of each of the 8 blocks, and each block's d.
template <>
struct MqW<kQ80> {
    uint4 q[8];
    uint32_t d[8];
};

typedef uint32_t u4_a2 __attribute__((ext_vector_type(4), aligned(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
QD_DEV uint4 ld128u(const uint8_t *p) {  // 16 bytes at a 2-byte-aligned address
    const u4_a2 v = *reinterpret_cast<const u4_a2 *>(p);
    return make_uint4(v.x, v.y, v.z, v.w);
}
QD_DEV uint32_t ld16(const uint8_t *p) { return *reinterpret_cast<const uint16_t *>(p); }

// ---- a wave's weight tile: 32 rows x one superunit.  Each row's unit is
// contiguous in memory, so the tile is read as 16-byte pieces with the lanes
// walking the rows' bytes in order (one instruction covers several whole
// rows, few cache lines), then written row-major to the wave's own LDS area
// and read back in the matrix core's B layout.
//   UB     bytes of one superunit of a row
//   NPC    16-byte pieces read per row (Q6_K: the last one starts 14 bytes
//          early, so no piece reads past the unit)
//   PITCH  LDS bytes per row (Q6_K padded so the 32 rows' reads fall in
//          distinct banks)
template <int FMT>
struct MqGeo;
template <> struct MqGeo<kQ4K> { static constexpr int UB = 144, NPC = 9, PITCH = 144; };
template <> struct MqGeo<kQ6K> { static constexpr int UB = 210, NPC = 14, PITCH = 224; };
template <> struct MqGeo<kQ80> { static constexpr int UB = 272, NPC = 17, PITCH = 272; };
template <int FMT>
QD_DEV constexpr int piece_src(int q) { return (FMT == kQ6K && q == 13) ? 194 : 16 * q; }
template <int FMT>
QD_DEV constexpr int piece_dst(int q) { return 16 * q; }
template <int FMT>
__host__ __device__ constexpr int mq_ni() { return (32 * MqGeo<FMT>::NPC + 63) / 64; }
// A wave's weight tile: 32 rows of PITCH = 16 NPC bytes, piece p of the
// tile (row p / NPC, piece p % NPC) at byte 16 p, so that one LDS copy of
// the 64 lanes fills 1 KB contiguously.  One per wave: the wave reads its
// whole tile into registers before it multiplies, and the next superunit's
// tile is copied into the same slot from then on.
template <int FMT>
__host__ __device__ constexpr int mq_slot() { return 32 * MqGeo<FMT>::PITCH; }
static_assert(MqGeo<kQ4K>::PITCH == 16 * MqGeo<kQ4K>::NPC && MqGeo<kQ6K>::PITCH == 16 * MqGeo<kQ6K>::NPC &&
                  MqGeo<kQ80>::PITCH == 16 * MqGeo<kQ80>::NPC,
              "tiles are filled 16 bytes per piece");
// Digit buffers in LDS: two (the next superunit's are copied in while the
// current one is read) where two workgroups still fit on a CU with them, or
// where not even one buffer lets two fit; else one (two workgroups per CU
// with one buffer measured faster than one with two: lm_head Q8_0 at batch
// 8, 193 -> 157 us).
template <int FMT, int NG>
__host__ __device__ constexpr int mq_nbuf() {
    constexpr int buf = NG * mq_su_bytes(FMT == kQ4K ? 128 : 32), rest = 16 + 4 * mq_slot<FMT>();
    constexpr int cu = 160 * 1024;
    if (2 * (2 * buf + rest) <= cu) return 2;
    if (2 * (buf + rest) <= cu) return 1;
    return 2 * buf + rest <= cu ? 2 : 1;
}
template <int FMT, int NG>
__host__ __device__ constexpr int mq_lds() {
    return mq_nbuf<FMT, NG>() * NG * mq_su_bytes(FMT == kQ4K ? 128 : 32) + 16 + 4 * mq_slot<FMT>();
}

// This lane's bytes of the tile in the B layout (row l % 32, half h = l / 32),
// read back from the wave's LDS area `scr` (row-major, PITCH per row).
template <int FMT>
QD_DEV void mq_read_tile(MqW<FMT> &w, const uint8_t *scr, int j, int h) {
    const uint8_t *rowp = scr + j * MqGeo<FMT>::PITCH;
    if constexpr (FMT == kQ4K) {
        w.hd = ld128(rowp);
#pragma unroll
        for (int c = 0; c < 4; c++) w.q[c] = ld128(rowp + 16 + 32 * c + 16 * h);
    } else if constexpr (FMT == kQ6K) {
#pragma unroll
        for (int H = 0; H < 2; H++) {
            w.ql[H][0] = ld128(rowp + 64 * H + 16 * h);
            w.ql[H][1] = ld128(rowp + 64 * H + 32 + 16 * h);
            w.qh[H] = ld128(rowp + 128 + 32 * H + 16 * h);
        }
        w.sc = ld128(rowp + 192);
        w.d = ld16(rowp + 208 + (208 - piece_src<kQ6K>(13)));  // d sits at 208..209 of the unit
    } else {
#pragma unroll
        for (int r = 0; r < 8; r++) {
            w.q[r] = ld128u(rowp + 34 * r + 2 + 16 * h);
            w.d[r] = ld16(rowp + 34 * r);
        }
    }
}

QD_DEV uint4 u4and(uint4 v, uint32_t m) { return make_uint4(v.x & m, v.y & m, v.z & m, v.w & m); }
QD_DEV uint4 u4shr(uint4 v, int s) { return make_uint4(v.x >> s, v.y >> s, v.z >> s, v.w >> s); }
QD_DEV v4i as_v4i(uint4 v) {
    v4i r;
    r[0] = (int)v.x;
    r[1] = (int)v.y;
    r[2] = (int)v.z;
    r[3] = (int)v.w;
    return r;
}
QD_DEV v16i mfma8(v4i a, v4i b) {
    const v16i z = {};
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, z, 0, 0, 0);
}
// Planes p = 0..3 of one batch row sit at output registers base + stride p.
template <int BASE, int STRIDE>
QD_DEV double undig64(const v16i &d) {
    return fma((double)(d[BASE + 3 * STRIDE] * 256 + d[BASE + 2 * STRIDE]), 65536.0,
               (double)(d[BASE + STRIDE] * 256 + d[BASE]));
}
template <int BASE, int STRIDE>
QD_DEV float undig32(const v16i &d) {
    return fmaf((float)(d[BASE + 3 * STRIDE] * 256 + d[BASE + 2 * STRIDE]), 65536.f,
                (float)(d[BASE + STRIDE] * 256 + d[BASE]));
}

// The accumulators are complete here: an empty asm that reads and writes
// them, so the compiler cannot sink a sub-block's products past the next
// one (which would keep every product's registers alive at once).
template <typename T, int A, int B, int C>
QD_DEV void pin_acc(T (&acc)[A][B][C]) {
#pragma unroll
    for (int i = 0; i < A; i++)
#pragma unroll
        for (int j = 0; j < B; j++)
#pragma unroll
            for (int k = 0; k < C; k++) asm volatile("" : "+v"(acc[i][j][k]));
}

// Copy of one superunit's digits (every group, BUF bytes of GB per group)
// through registers: thread tid moves the 16-byte pieces tid + 256 v.
// (native vectors, not the uint4 struct, whose copies between address
// spaces would go through private memory)
template <int SV, int BUF, int GB>
QD_DEV void mq_stage_load(u32x4 (&stg)[SV], const uint8_t *dig, int nb, int t, int tid) {
#pragma unroll
    for (int v = 0; v < SV; v++) {
        const int e = min(tid + 256 * v, BUF / 16 - 1);  // repeats past the end are not stored
        const int g = e / (GB / 16), o = e - g * (GB / 16);
        stg[v] = reinterpret_cast<const u32x4 *>(dig + ((int64_t)g * nb + t) * GB)[o];
    }
}
template <int SV, int BUF>
QD_DEV void mq_stage_store(uint8_t *dst, const u32x4 (&stg)[SV], int tid) {
#pragma unroll
    for (int v = 0; v < SV; v++)
        if (v < SV - 1 || tid + 256 * v < BUF / 16) *reinterpret_cast<u32x4 *>(dst + 16 * (tid + 256 * v)) = stg[v];
}

// ------------------------------------------------------------ the kernel ---
template <int FMT, int NG, bool FFN>
__global__ __launch_bounds__(256) void mq_kernel(MqArgs a) {
    constexpr int NR = 1;                       // one matrix per wave
    constexpr int TILE = mq_tile_rows(FFN);     // rows per workgroup (of each matrix)
    constexpr int RR = FMT == kQ4K ? 128 : 32;  // record bytes per run (8 batch rows)
    constexpr int GB = mq_su_bytes(RR);         // bytes per superunit per group
    constexpr int BUF = NG * GB;
    constexpr int SV = (BUF / 16 + 255) / 256;  // staged uint4 per thread
    using Acc = typename std::conditional<FMT == kQ4K, double, float>::type;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];  // [NBUF][BUF], 16 zero bytes, 4 tiles
    __shared__ float red[4];
    __shared__ int flag;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int h = lane >> 5;
    const int bx = blockIdx.x, ks = blockIdx.y, p_out = gridDim.y;
    const int t_beg = ks * a.nk, t_end = min(a.nb, t_beg + a.nk);
    const int64_t N = a.N;
    // FFN: waves 0-1 take 64 rows of gate, waves 2-3 the same rows of up
    const int mi = FFN ? wave >> 1 : 0;
    const int rloc = (FFN ? (wave & 1) : wave) * 32 + (lane & 31);
    const int64_t row = (int64_t)bx * TILE + rloc;
    const bool row_ok = row < N;
    const int64_t rowc = row_ok ? row : N - 1;
    (void)rowc;

    // ---- digits of superunit t (every group) into a digit buffer: by LDS
    // copies where there are two buffers, else through registers (loaded
    // before the current superunit is multiplied, stored after)
    constexpr int NBUF = mq_nbuf<FMT, NG>();
    u32x4 stg[NBUF == 1 ? SV : 1];
    auto stage_load = [&](int t) {
        if constexpr (NBUF == 1) mq_stage_load<SV, BUF, GB>(stg, a.dig, a.nb, t, tid);
    };
    auto stage_store = [&](int bi) {
        if constexpr (NBUF == 1) mq_stage_store<SV, BUF>(lds + bi * BUF, stg, tid);
    };
    auto stage_copy = [&](int t, int bi) {  // thread tid copies pieces tid + 256 v
#pragma unroll
        for (int v = 0; v < SV; v++) {
            const int e = tid + 256 * v;
            if (v == SV - 1 && 256 * v + 64 * wave >= BUF / 16) break;  // no piece of this wave
            const int ec = min(e, BUF / 16 - 1);
            const int g = ec / (GB / 16), o = ec - g * (GB / 16);
            if (e < BUF / 16)
                lds_copy16(a.dig + ((int64_t)g * a.nb + t) * GB + 16 * o,
                           lds_addr(lds + bi * BUF + 16 * (256 * v + 64 * wave)));
        }
    };

    // ---- weight tiles by LDS copies, one superunit ahead: lane piece p =
    // 64 i + lane of copy i is piece p % NPC of the wave's row p / NPC
    constexpr int NI = mq_ni<FMT>(), NPC = MqGeo<FMT>::NPC, UB = MqGeo<FMT>::UB;
    uint32_t voff[NI];
    bool pv[NI];
    {
        const int64_t row0w = (int64_t)bx * TILE + (FFN ? (wave & 1) : wave) * 32;
#pragma unroll
        for (int i = 0; i < NI; i++) {
            const int p = 64 * i + lane;
            const int r = p / NPC, q = p - (p / NPC) * NPC;
            pv[i] = p < 32 * NPC;
            const int64_t rr = min(row0w + r, N - 1);
            voff[i] = (uint32_t)(rr * a.row_bytes + piece_src<FMT>(q));
        }
    }
    const uint8_t *wbase = mi ? a.W1 : a.W0;
    uint8_t *scr = lds + NBUF * BUF + 16 + wave * mq_slot<FMT>();  // [32 rows][PITCH]
    auto wcopy = [&](int t) {
        t = min(t, t_end - 1);
        // the copy's base address and LDS destination in scalar registers
        const uint64_t b64 = reinterpret_cast<uint64_t>(wbase + (int64_t)UB * t);
        // (readfirstlane returns int: widen through uint32_t, not by sign)
        const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b64);
        const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b64 >> 32));
        const uint64_t bu = ((uint64_t)hi << 32) | (uint64_t)lo;
        const uint8_t *base = reinterpret_cast<const uint8_t *>(bu);
        const uint32_t dst = __builtin_amdgcn_readfirstlane(lds_addr(scr));
#pragma unroll
        for (int i = 0; i < NI; i++)
            if (i < NI - 1 || pv[i]) lds_copy16_s(base, voff[i], dst + 1024 * i);
    };

    Acc acc[NR][NG][4];
#pragma unroll
    for (int i = 0; i < NR; i++)
#pragma unroll
        for (int g = 0; g < NG; g++)
#pragma unroll
            for (int jj = 0; jj < 4; jj++) acc[i][g][jj] = (Acc)0;

    // Q6_K: A operand offsets of the two half-zero instructions of a run;
    // lanes whose A row and k half disagree read 16 zero bytes past the
    // digit buffers instead
    const int ai = lane & 31;
    const bool a_live = (ai < 16) == (h == 0);
    int aoff[2];
#pragma unroll
    for (int u = 0; u < 2; u++) {
        const int i16 = ai & 15;
        const int bb = 4 * ((i16 & 7) >> 2) + 2 * u + (i16 >> 3);
        aoff[u] = 16 * (bb + 8 * (i16 & 3) + 32 * h);
    }
    const uint8_t *zero16 = lds + mq_nbuf<FMT, NG>() * BUF;

    // ---- one superunit, software-pipelined over its steps (sub-block and
    // group): step n's fragment is read two steps ahead and its product
    // issued one step ahead, so the matrix core and LDS latencies run under
    // the previous step's scaling; the accumulators are pinned after each
    // step so the compiler keeps that order
    // Four or more groups: one step at a time (the pipelined form's
    // registers and code do not fit at that size)
    auto compute_wide = [&](const MqW<FMT> &wv, const uint8_t *buf) {
        if constexpr (FMT == kQ4K) {
            const double dd = (double)f16_lo(wv.hd.x), dm = (double)f16_hi(wv.hd.x);
            const uint32_t s03 = wv.hd.y, s47 = wv.hd.z, s811 = wv.hd.w;
            const uint32_t scp[2] = {s03 & 0x3F3F3F3Fu, (s811 & 0x0F0F0F0Fu) | ((s03 >> 2) & 0x30303030u)};
            const uint32_t mnp[2] = {s47 & 0x3F3F3F3Fu, ((s811 >> 4) & 0x0F0F0F0Fu) | ((s47 >> 2) & 0x30303030u)};
#pragma unroll
            for (int sb = 0; sb < 8; sb++) {
                const v4i B = as_v4i(u4and((sb & 1) ? u4shr(wv.q[sb >> 1], 4) : wv.q[sb >> 1], 0x0F0F0F0Fu));
                const double ae = dd * (double)((scp[sb >> 2] >> (8 * (sb & 3))) & 0xFFu);
                const double be = dm * (double)((mnp[sb >> 2] >> (8 * (sb & 3))) & 0xFFu);
#pragma unroll
                for (int g = 0; g < NG; g++) {
                    const uint8_t *gb = buf + g * GB;
                    const v4i A = *reinterpret_cast<const v4i *>(gb + sb * kFragRun + 16 * lane);
                    const double2 *rc = reinterpret_cast<const double2 *>(gb + 8 * kFragRun + sb * RR + 64 * h);
                    const v16i d = mfma8(A, B);
#pragma unroll
                    for (int jj = 0; jj < 4; jj++) {
                        const double2 r = rc[jj];
                        const double I = jj == 0 ? undig64<0, 4>(d) : jj == 1 ? undig64<1, 4>(d)
                                         : jj == 2 ? undig64<2, 4>(d) : undig64<3, 4>(d);
                        acc[0][g][jj] = fma(ae * r.x, I, fma(-be, r.y, acc[0][g][jj]));
                    }
                    pin_acc(acc);
                }
            }
        } else if constexpr (FMT == kQ6K) {
            const float d6 = f16_lo(wv.d);
            const uint32_t sw[4] = {wv.sc.x, wv.sc.y, wv.sc.z, wv.sc.w};
#pragma unroll
            for (int r = 0; r < 8; r++) {
                const int H = r >> 2, g4 = r & 3;
                const uint4 ql = wv.ql[H][g4 & 1];
                const uint4 nib = u4and(g4 >= 2 ? u4shr(ql, 4) : ql, 0x0F0F0F0Fu);
                const uint4 hb = u4and(u4shr(wv.qh[H], 2 * g4), 0x03030303u);
                v4i B;
                B[0] = (int)(nib.x | byte_lut(kQ6HiTable, hb.x));
                B[1] = (int)(nib.y | byte_lut(kQ6HiTable, hb.y));
                B[2] = (int)(nib.z | byte_lut(kQ6HiTable, hb.z));
                B[3] = (int)(nib.w | byte_lut(kQ6HiTable, hb.w));
                const float ds0 = d6 * sbyte(sw[r >> 1], 2 * (r & 1)), ds1 = d6 * sbyte(sw[r >> 1], 2 * (r & 1) + 1);
#pragma unroll
                for (int g = 0; g < NG; g++) {
                    const uint8_t *gb = buf + g * GB;
                    const float4 S = *reinterpret_cast<const float4 *>(gb + 8 * kFragRun + r * RR + 16 * h);
#pragma unroll
                    for (int u = 0; u < 2; u++) {
                        const v4i A = *reinterpret_cast<const v4i *>(a_live ? gb + r * kFragRun + aoff[u] : zero16);
                        const v16i d = mfma8(A, B);
                        const float s0 = u ? S.z : S.x, s1 = u ? S.w : S.y;
                        Acc &a0 = acc[0][g][2 * u], &a1 = acc[0][g][2 * u + 1];
                        a0 = fmaf(ds0 * s0, undig32<0, 1>(d), a0);
                        a0 = fmaf(ds1 * s0, undig32<8, 1>(d), a0);
                        a1 = fmaf(ds0 * s1, undig32<4, 1>(d), a1);
                        a1 = fmaf(ds1 * s1, undig32<12, 1>(d), a1);
                        pin_acc(acc);
                    }
                }
            }
        } else {
#pragma unroll
            for (int r = 0; r < 8; r++) {
                const v4i B = as_v4i(wv.q[r]);
                const float dq = f16_lo(wv.d[r]);
#pragma unroll
                for (int g = 0; g < NG; g++) {
                    const uint8_t *gb = buf + g * GB;
                    const v4i A = *reinterpret_cast<const v4i *>(gb + r * kFragRun + 16 * lane);
                    const float4 S = *reinterpret_cast<const float4 *>(gb + 8 * kFragRun + r * RR + 16 * h);
                    const v16i d = mfma8(A, B);
                    acc[0][g][0] = fmaf(dq * S.x, undig32<0, 4>(d), acc[0][g][0]);
                    acc[0][g][1] = fmaf(dq * S.y, undig32<1, 4>(d), acc[0][g][1]);
                    acc[0][g][2] = fmaf(dq * S.z, undig32<2, 4>(d), acc[0][g][2]);
                    acc[0][g][3] = fmaf(dq * S.w, undig32<3, 4>(d), acc[0][g][3]);
                    pin_acc(acc);
                }
            }
        }
    };
    auto compute = [&](const MqW<FMT> &wv, const uint8_t *buf) {
        if constexpr (NG >= 4) {
            compute_wide(wv, buf);
        } else if constexpr (FMT == kQ4K) {
            const double dd = (double)f16_lo(wv.hd.x), dm = (double)f16_hi(wv.hd.x);
            const uint32_t s03 = wv.hd.y, s47 = wv.hd.z, s811 = wv.hd.w;
            // 6-bit scales / mins of sub-blocks 0..3 and 4..7, a byte each
            const uint32_t scp[2] = {s03 & 0x3F3F3F3Fu, (s811 & 0x0F0F0F0Fu) | ((s03 >> 2) & 0x30303030u)};
            const uint32_t mnp[2] = {s47 & 0x3F3F3F3Fu, ((s811 >> 4) & 0x0F0F0F0Fu) | ((s47 >> 2) & 0x30303030u)};
            constexpr int NS = 8 * NG;  // step n: sub-block n / NG, group n % NG
            auto bop = [&](int sb) {
                return as_v4i(u4and((sb & 1) ? u4shr(wv.q[sb >> 1], 4) : wv.q[sb >> 1], 0x0F0F0F0Fu));
            };
            auto aload = [&](int n) {
                return *reinterpret_cast<const v4i *>(buf + (n % NG) * GB + (n / NG) * kFragRun + 16 * lane);
            };
            auto rload = [&](int n, double2 (&r)[4]) {
                const double2 *rc =
                    reinterpret_cast<const double2 *>(buf + (n % NG) * GB + 8 * kFragRun + (n / NG) * RR + 64 * h);
#pragma unroll
                for (int jj = 0; jj < 4; jj++) r[jj] = rc[jj];
            };
            v4i Aq[3];
            v16i Dq[2];
            double2 Rq[2][4];
            Aq[0] = aload(0);
            if (NS > 1) Aq[1] = aload(1);
            rload(0, Rq[0]);
            Dq[0] = mfma8(Aq[0], bop(0));
#pragma unroll
            for (int n = 0; n < NS; n++) {
                const int sb = n / NG, g = n % NG;
                if (n + 2 < NS) Aq[(n + 2) % 3] = aload(n + 2);
                if (n + 1 < NS) {
                    rload(n + 1, Rq[(n + 1) & 1]);
                    Dq[(n + 1) & 1] = mfma8(Aq[(n + 1) % 3], bop((n + 1) / NG));
                }
                const double ae = dd * (double)((scp[sb >> 2] >> (8 * (sb & 3))) & 0xFFu);
                const double be = dm * (double)((mnp[sb >> 2] >> (8 * (sb & 3))) & 0xFFu);
                const v16i &d = Dq[n & 1];
                const double2(&r)[4] = Rq[n & 1];
                acc[0][g][0] = fma(ae * r[0].x, undig64<0, 4>(d), fma(-be, r[0].y, acc[0][g][0]));
                acc[0][g][1] = fma(ae * r[1].x, undig64<1, 4>(d), fma(-be, r[1].y, acc[0][g][1]));
                acc[0][g][2] = fma(ae * r[2].x, undig64<2, 4>(d), fma(-be, r[2].y, acc[0][g][2]));
                acc[0][g][3] = fma(ae * r[3].x, undig64<3, 4>(d), fma(-be, r[3].y, acc[0][g][3]));
                pin_acc(acc);
            }
        } else if constexpr (FMT == kQ6K) {
            const float d6 = f16_lo(wv.d);
            const uint32_t sw[4] = {wv.sc.x, wv.sc.y, wv.sc.z, wv.sc.w};
            // step n: run n / (2 NG), group (n / 2) % NG, half-zero instruction n % 2
            constexpr int NS = 16 * NG;
            auto bop = [&](int r) {  // quants q - 32 of sub-blocks 2r (k < 16) and 2r + 1
                const int H = r >> 2, g4 = r & 3;
                const uint4 ql = wv.ql[H][g4 & 1];
                const uint4 nib = u4and(g4 >= 2 ? u4shr(ql, 4) : ql, 0x0F0F0F0Fu);
                const uint4 hb = u4and(u4shr(wv.qh[H], 2 * g4), 0x03030303u);
                v4i B;
                B[0] = (int)(nib.x | byte_lut(kQ6HiTable, hb.x));
                B[1] = (int)(nib.y | byte_lut(kQ6HiTable, hb.y));
                B[2] = (int)(nib.z | byte_lut(kQ6HiTable, hb.z));
                B[3] = (int)(nib.w | byte_lut(kQ6HiTable, hb.w));
                return B;
            };
            auto aload = [&](int n) {
                const int r = n / (2 * NG), g = (n >> 1) % NG, u = n & 1;
                const uint8_t *p = a_live ? buf + g * GB + r * kFragRun + aoff[u] : zero16;
                return *reinterpret_cast<const v4i *>(p);
            };
            auto sload = [&](int n) {
                const int r = n / (2 * NG), g = (n >> 1) % NG;
                return *reinterpret_cast<const float4 *>(buf + g * GB + 8 * kFragRun + r * RR + 16 * h);
            };
            v4i Aq[3];
            v16i Dq[2];
            float4 Sq[2];
            Aq[0] = aload(0);
            Aq[1] = aload(1);
            Sq[0] = sload(0);
            Dq[0] = mfma8(Aq[0], bop(0));
#pragma unroll
            for (int n = 0; n < NS; n++) {
                const int r = n / (2 * NG), g = (n >> 1) % NG, u = n & 1;
                if (n + 2 < NS) Aq[(n + 2) % 3] = aload(n + 2);
                if (n + 1 < NS) {
                    Sq[(n + 1) & 1] = sload(n + 1);
                    Dq[(n + 1) & 1] = mfma8(Aq[(n + 1) % 3], bop((n + 1) / (2 * NG)));
                }
                const v16i &d = Dq[n & 1];
                const float4 S = Sq[n & 1];
                const float ds0 = d6 * sbyte(sw[r >> 1], 2 * (r & 1));      // sub-block 2r
                const float ds1 = d6 * sbyte(sw[r >> 1], 2 * (r & 1) + 1);  // sub-block 2r + 1
                // registers 4a + p (sub-block 2r) and 8 + 4a + p (2r + 1) hold
                // batch row 4h + 2u + a
                const float s0 = u ? S.z : S.x, s1 = u ? S.w : S.y;
                Acc &a0 = acc[0][g][2 * u], &a1 = acc[0][g][2 * u + 1];
                a0 = fmaf(ds0 * s0, undig32<0, 1>(d), a0);
                a0 = fmaf(ds1 * s0, undig32<8, 1>(d), a0);
                a1 = fmaf(ds0 * s1, undig32<4, 1>(d), a1);
                a1 = fmaf(ds1 * s1, undig32<12, 1>(d), a1);
                pin_acc(acc);
            }
        } else {
            constexpr int NS = 8 * NG;  // step n: block n / NG, group n % NG
            auto aload = [&](int n) {
                return *reinterpret_cast<const v4i *>(buf + (n % NG) * GB + (n / NG) * kFragRun + 16 * lane);
            };
            auto sload = [&](int n) {
                return *reinterpret_cast<const float4 *>(buf + (n % NG) * GB + 8 * kFragRun + (n / NG) * RR + 16 * h);
            };
            v4i Aq[3];
            v16i Dq[2];
            float4 Sq[2];
            Aq[0] = aload(0);
            if (NS > 1) Aq[1] = aload(1);
            Sq[0] = sload(0);
            Dq[0] = mfma8(Aq[0], as_v4i(wv.q[0]));
#pragma unroll
            for (int n = 0; n < NS; n++) {
                const int r = n / NG, g = n % NG;
                if (n + 2 < NS) Aq[(n + 2) % 3] = aload(n + 2);
                if (n + 1 < NS) {
                    Sq[(n + 1) & 1] = sload(n + 1);
                    Dq[(n + 1) & 1] = mfma8(Aq[(n + 1) % 3], as_v4i(wv.q[(n + 1) / NG]));
                }
                const v16i &d = Dq[n & 1];
                const float4 S = Sq[n & 1];
                const float dq = f16_lo(wv.d[r]);
                acc[0][g][0] = fmaf(dq * S.x, undig32<0, 4>(d), acc[0][g][0]);
                acc[0][g][1] = fmaf(dq * S.y, undig32<1, 4>(d), acc[0][g][1]);
                acc[0][g][2] = fmaf(dq * S.z, undig32<2, 4>(d), acc[0][g][2]);
                acc[0][g][3] = fmaf(dq * S.w, undig32<3, 4>(d), acc[0][g][3]);
                pin_acc(acc);
            }
        }
    };

    // ---- main loop: superunit t multiplied from LDS half (t - t_beg) & 1
    // while superunit t + 1's fragments are loaded for the other half
    if (FMT == kQ6K && tid == 0) *reinterpret_cast<uint4 *>(const_cast<uint8_t *>(zero16)) = make_uint4(0u, 0u, 0u, 0u);
    // ---- main loop: superunit t's tile read out of the wave's slot into
    // registers, then superunit t + 1's tile copied into the slot and its
    // digits into the other digit buffer (or loaded into registers, where
    // there is one buffer) while t is multiplied; every copy of an iteration
    // has landed at its end (vmcnt 0, then the barrier makes the digits of
    // every wave visible)
    if (t_beg < t_end) {
        wcopy(t_beg);
        if constexpr (NBUF == 2) stage_copy(t_beg, 0);
        else stage_load(t_beg);
        stage_store(0);
        vm_wait<0>();
        block_sync();
        for (int t = t_beg; t < t_end; t++) {
            const int bi = NBUF == 2 ? (t - t_beg) & 1 : 0;
            const bool more = t + 1 < t_end;
            MqW<FMT> wv;
            mq_read_tile<FMT>(wv, scr, lane & 31, h);
            lgkm_wait();  // the tile is in registers: the slot may be refilled
            if (more) {
                wcopy(t + 1);
                if constexpr (NBUF == 2) stage_copy(t + 1, bi ^ 1);
                else stage_load(t + 1);
            }
            compute(wv, lds + bi * BUF);
            if (more && NBUF == 1) {
                block_sync();  // every wave is done with the buffer
                stage_store(0);
            }
            vm_wait<0>();
            block_sync();
        }
    }

    // ---- outputs: lane (row, batch rows 8g + 4h + jj)
    constexpr int NP = FFN ? 2 : 1;
    const int B = a.batch;
    if (p_out == 1) {
        if constexpr (FFN) {
            // up (waves 2-3) hands its rows to gate (waves 0-1) through LDS
            float *ub = reinterpret_cast<float *>(lds);  // [64 rows][8 NG]; the digit buffers are done
            if (mi == 1) {
#pragma unroll
                for (int g = 0; g < NG; g++)
#pragma unroll
                    for (int jj = 0; jj < 4; jj++) ub[rloc * 8 * NG + 8 * g + 4 * h + jj] = (float)acc[0][g][jj];
            }
            block_sync();
            if (mi == 0) {  // uniform per wave; the rows of an FFN tile are all in the matrix
#pragma unroll
                for (int g = 0; g < NG; g++)
#pragma unroll
                    for (int jj = 0; jj < 4; jj++) {
                        const int b = 8 * g + 4 * h + jj;  // the same slot for the 32 lanes of a half
                        const float gv = (float)acc[0][g][jj], uv = ub[rloc * 8 * NG + 8 * g + 4 * h + jj];
                        const float hv = act_apply(a.act, gv) * uv;  // 0 for the zero digits of slots past B
                        if (a.hdig) emit_h_digit(a, hv, b, row);
                        if (b >= B || !row_ok) continue;
                        const int64_t o = (int64_t)b * N + row;
                        if (a.y) a.y[o] = hv;
                        if (a.g_out) a.g_out[o] = gv;
                        if (a.u_out) a.u_out[o] = uv;
                    }
            }
        } else {
            if (row_ok) {
#pragma unroll
                for (int g = 0; g < NG; g++)
#pragma unroll
                    for (int jj = 0; jj < 4; jj++) {
                        const int b = 8 * g + 4 * h + jj;
                        if (b >= B) continue;
                        const int64_t o = (int64_t)b * N + row;
                        const float vv = (float)acc[0][g][jj];
                        if (a.pn.w1) xstore(a.pn.p + o, vv);  // the row epilogue forms y
                        else a.y[o] = a.res ? vv + a.res[o] : vv;
                    }
            }
            if (a.pn.w1) post_norm_tail<256>(a.pn, a.y, B, N, red, &flag);
        }
        return;
    }
    if (row_ok) {
#pragma unroll
        for (int g = 0; g < NG; g++)
#pragma unroll
            for (int jj = 0; jj < 4; jj++) {
                const int b = 8 * g + 4 * h + jj;
                if (b >= B) continue;
                xstore(a.partials + (((int64_t)ks * B + b) * NP + mi) * N + row, (float)acc[0][g][jj]);
            }
    }
    // ---- split-K: the last workgroup of this row tile sums the partials in
    // slice order (the hand-off of qd_epilogue.h on the tile's counter)
    if (!arrive_last<256>(a.counters + bx, (unsigned)p_out, &flag)) return;
    // each thread sums the slices of up to EPT outputs of the tile, with
    // KC slices per output loaded at once (independent loads in flight,
    // added in slice order afterwards)
    constexpr int EPT = TILE * 8 * NG / 256;
    constexpr int KC = EPT * NP >= 32 ? 1 : 32 / (EPT * NP);
    const int64_t tile0 = (int64_t)bx * TILE;
    float s[EPT][NP];
#pragma unroll
    for (int m = 0; m < EPT; m++)
#pragma unroll
        for (int i = 0; i < NP; i++) s[m][i] = 0.f;
    for (int k0 = 0; k0 < p_out; k0 += KC) {
        float v[EPT][NP][KC];
#pragma unroll
        for (int m = 0; m < EPT; m++) {
            const int e = tid + 256 * m;
            const int b = e / TILE;
            const int64_t r = tile0 + (e - b * TILE);
            const bool ok = b < B && r < N;
#pragma unroll
            for (int u = 0; u < KC; u++) {
                const int k = min(k0 + u, p_out - 1);
                const float *p = a.partials + (((int64_t)k * B + b) * NP) * N + r;
#pragma unroll
                for (int i = 0; i < NP; i++) v[m][i][u] = ok ? xload(p + i * N) : 0.f;
            }
        }
#pragma unroll
        for (int m = 0; m < EPT; m++)
#pragma unroll
            for (int u = 0; u < KC; u++)
                if (k0 + u < p_out)
#pragma unroll
                    for (int i = 0; i < NP; i++) s[m][i] += v[m][i][u];
    }
#pragma unroll
    for (int m = 0; m < EPT; m++) {
        const int e = tid + 256 * m;
        const int b = e / TILE;
        const int64_t r = tile0 + (e - b * TILE);
        const float s0 = s[m][0];
        if constexpr (FFN) {
            // a wave holds one batch slot's 64 rows: a run in each half
            const float s1 = s[m][NP - 1];
            const float hv = act_apply(a.act, s0) * s1;  // 0 for slots past B
            if (a.hdig) emit_h_digit(a, hv, b, r);
            if (b >= B || r >= N) continue;
            const int64_t o = (int64_t)b * N + r;
            if (a.y) a.y[o] = hv;
            if (a.g_out) a.g_out[o] = s0;
            if (a.u_out) a.u_out[o] = s1;
        } else {
            if (b >= B || r >= N) continue;
            const int64_t o = (int64_t)b * N + r;
            if (a.pn.w1) xstore(a.pn.p + o, s0);
            else a.y[o] = a.res ? s0 + a.res[o] : s0;
        }
    }
    if (tid == 0)  // ready for the next call
        __hip_atomic_store(a.counters + bx, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (!FFN && a.pn.w1) post_norm_tail<256>(a.pn, a.y, B, N, red, &flag);
}

// ------------------------------------------------------------- launchers ---
size_t mq_su_bytes_host(int fmt) { return (size_t)mq_su_bytes(fmt == kQ4K ? 128 : 32); }
template <int FMT>
static size_t mq_lds_f(int ng) {
    switch (ng) {
    case 1: return mq_lds<FMT, 1>();
    case 2: return mq_lds<FMT, 2>();
    case 4: return mq_lds<FMT, 4>();
    default: return mq_lds<FMT, 8>();
    }
}
size_t mq_lds_bytes(int fmt, int ng) {
    return fmt == kQ4K ? mq_lds_f<kQ4K>(ng) : fmt == kQ6K ? mq_lds_f<kQ6K>(ng) : mq_lds_f<kQ80>(ng);
}

// Allow each kernel the dynamic LDS it uses (once per kernel; the static
// words of the kernel come on top).
template <auto Kern>
static hipError_t allow_lds_mq(size_t bytes) {
    static const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(Kern),
                                                    hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    return e;
}

int xdig_max_k() { return kXdMaxK; }

hipError_t launch_xdig(const XdArgs &a, int ng, bool sx, hipStream_t st) {
    if (a.K > xdig_max_k() || a.nb < 1 || 256 * (int64_t)a.nb < a.K) return hipErrorInvalidValue;
    const dim3 grid((unsigned)(ng * 8), (unsigned)((a.nb + 3) / 4));
    const bool norm = a.norm_w != nullptr;
    const dim3 blk(kXdThreads);
    if (norm && sx) hipLaunchKernelGGL((xdig_kernel<true, true>), grid, blk, 0, st, a);
    else if (norm) hipLaunchKernelGGL((xdig_kernel<true, false>), grid, blk, 0, st, a);
    else if (sx) hipLaunchKernelGGL((xdig_kernel<false, true>), grid, blk, 0, st, a);
    else hipLaunchKernelGGL((xdig_kernel<false, false>), grid, blk, 0, st, a);
    return hipGetLastError();
}

template <int FMT, int NG, bool FFN>
static hipError_t launch_mq_one(const MqArgs &a, dim3 grid, hipStream_t st) {
    const size_t lds = mq_lds_bytes(FMT, NG);
    if (allow_lds_mq<mq_kernel<FMT, NG, FFN>>(lds) != hipSuccess) return hipErrorInvalidValue;
    hipLaunchKernelGGL((mq_kernel<FMT, NG, FFN>), grid, dim3(256), lds, st, a);
    return hipGetLastError();
}

template <int FMT>
static hipError_t launch_mq_f(const MqArgs &a, int ng, bool ffn, dim3 grid, hipStream_t st) {
    switch (ng) {
    case 1: return ffn ? launch_mq_one<FMT, 1, true>(a, grid, st) : launch_mq_one<FMT, 1, false>(a, grid, st);
    case 2: return ffn ? launch_mq_one<FMT, 2, true>(a, grid, st) : launch_mq_one<FMT, 2, false>(a, grid, st);
    case 4: return ffn ? launch_mq_one<FMT, 4, true>(a, grid, st) : launch_mq_one<FMT, 4, false>(a, grid, st);
    case 8: return ffn ? launch_mq_one<FMT, 8, true>(a, grid, st) : launch_mq_one<FMT, 8, false>(a, grid, st);
    default: return hipErrorInvalidValue;
    }
}

// Workgroups of a matrix kernel resident per CU (registers and LDS).
template <int FMT, int NG, bool FFN>
static int mq_occ() {
    static const int n = [] {
        const size_t lds = mq_lds_bytes(FMT, NG);
        if (allow_lds_mq<mq_kernel<FMT, NG, FFN>>(lds) != hipSuccess) return 1;
        int wg = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&wg, reinterpret_cast<const void *>(mq_kernel<FMT, NG, FFN>),
                                                         256, lds) != hipSuccess)
            return 1;
        return wg > 0 ? wg : 1;
    }();
    return n;
}
template <int FMT>
static int mq_occ_f(int ng, bool ffn) {
    switch (ng) {
    case 1: return ffn ? mq_occ<FMT, 1, true>() : mq_occ<FMT, 1, false>();
    case 2: return ffn ? mq_occ<FMT, 2, true>() : mq_occ<FMT, 2, false>();
    case 4: return ffn ? mq_occ<FMT, 4, true>() : mq_occ<FMT, 4, false>();
    default: return ffn ? mq_occ<FMT, 8, true>() : mq_occ<FMT, 8, false>();
    }
}
int mq_wg_per_cu(int fmt, int ng, bool ffn) {
    switch (fmt) {
    case kQ4K: return mq_occ_f<kQ4K>(ng, ffn);
    case kQ6K: return mq_occ_f<kQ6K>(ng, ffn);
    default: return mq_occ_f<kQ80>(ng, ffn);
    }
}

hipError_t launch_mq(int fmt, int ng, bool ffn, const MqArgs &a, unsigned tiles, unsigned p_out,
                     hipStream_t st) {
    const dim3 grid(tiles, p_out);
    switch (fmt) {
    case kQ4K: return launch_mq_f<kQ4K>(a, ng, ffn, grid, st);
    case kQ6K: return launch_mq_f<kQ6K>(a, ng, ffn, grid, st);
    case kQ80: return launch_mq_f<kQ80>(a, ng, ffn, grid, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace qd
