// qd_gemv_stream.hip -- decode GEMV and fused gate/up with the weights
// streamed through LDS (the default path for batch 1 and 2).
//
// Same products as qd_gemv.hip (y[b][n] = sum_k w[n][k] x[b][k], or the
// fused act(Wg x) * (Wu x) of the larql Gemma 3 table), organised for the
// small matrices of a decode step, whose time is set by how fast the whole
// weight stream can be put in flight:
//
//  * One workgroup per CU, each owning a contiguous range of rows (row
//    counts differ by at most one).  A row range is one contiguous byte
//    range of the matrix, so the workgroup's weights are a single stream.
//  * The stream is cut into steps of 16 superunits (256 weights each: one
//    Q4_K or Q6_K block, eight Q8_0 blocks).  Wave w takes steps w, w+4, ...
//    and copies each into a ring of its own in LDS with
//    global_load_lds_dwordx4: 1 KB of consecutive bytes per instruction, no
//    registers, several steps in flight while it decodes an earlier one.
//  * Decoding reads a lane group's block (4 lanes per superunit, the lane
//    split of the GEMV kernels) and its activations from LDS, and writes the
//    superunit's partial sum to LDS.  After the stream, each row's partials
//    are added in superunit order, so a result does not depend on the launch
//    shape.
//  * x is copied into LDS the same way (16-byte skew every 64 floats), then
//    RMS-normalised in place; Q4_K also keeps the sum of every 32-run of x.
// The copies are ordered by explicit waits (qd_lds.h).
#include "qd_decode.h"
#include "qd_lds.h"

namespace qd {
namespace {

constexpr int kStepUnits = 16;  // superunits per step (one per lane group of a wave)
constexpr int kWaves = kThreads / 64;

template <int FMT>
struct StreamFmt;
template <>
struct StreamFmt<kQ4K> {
    static constexpr int UB = 144;   // bytes per superunit
    static constexpr int NCH = 144;  // 16-byte chunks per step (steps start 16-byte aligned)
};
template <>
struct StreamFmt<kQ6K> {
    static constexpr int UB = 210;
    static constexpr int NCH = 211;  // a step may start up to 14 bytes past a 16-byte boundary
};
template <>
struct StreamFmt<kQ80> {
    static constexpr int UB = 272;
    static constexpr int NCH = 272;
};

template <int FMT>
constexpr int copies_per_step() {
    return (StreamFmt<FMT>::NCH + 63) / 64;
}

// Wait until at most n copies / loads of this wave are outstanding (n is
// uniform; the immediate is chosen by a scalar branch).
QD_DEV void vm_wait_n(int n) {
    switch (n) {
#define QD_VMW(i) case i: vm_wait<i>(); break;
        QD_VMW(0) QD_VMW(1) QD_VMW(2) QD_VMW(3) QD_VMW(4) QD_VMW(5) QD_VMW(6) QD_VMW(7)
        QD_VMW(8) QD_VMW(9) QD_VMW(10) QD_VMW(11) QD_VMW(12) QD_VMW(13) QD_VMW(14) QD_VMW(15)
        QD_VMW(16) QD_VMW(17) QD_VMW(18) QD_VMW(19) QD_VMW(20) QD_VMW(21) QD_VMW(22) QD_VMW(23)
        QD_VMW(24) QD_VMW(25) QD_VMW(26) QD_VMW(27) QD_VMW(28) QD_VMW(29) QD_VMW(30) QD_VMW(31)
        QD_VMW(32) QD_VMW(33) QD_VMW(34) QD_VMW(35) QD_VMW(36) QD_VMW(37) QD_VMW(38) QD_VMW(39)
        QD_VMW(40) QD_VMW(41) QD_VMW(42) QD_VMW(43) QD_VMW(44) QD_VMW(45) QD_VMW(46) QD_VMW(47)
        QD_VMW(48) QD_VMW(49) QD_VMW(50) QD_VMW(51) QD_VMW(52) QD_VMW(53) QD_VMW(54) QD_VMW(55)
        QD_VMW(56) QD_VMW(57) QD_VMW(58) QD_VMW(59) QD_VMW(60) QD_VMW(61) QD_VMW(62) QD_VMW(63)
#undef QD_VMW
    default: vm_wait<0>(); break;
    }
}

// Logical activation index k -> LDS float index (16-byte skew every 64).
QD_DEV int xphys(int k) { return k + ((k >> 6) << 2); }
constexpr int kSuperPhys = kSuper + kSuper / 16;  // 272 floats per superunit

// --------------------------------------------------------- block loads ---
// One lane's share of a superunit from LDS (blk: the superunit's first byte
// in the ring), into the register layouts of qd_decode.h.
QD_DEV uint32_t lds32(const uint8_t *p) { return *reinterpret_cast<const uint32_t *>(p); }

QD_DEV void lds_q4k(RawQ4K &r, const uint8_t *blk, int c) {
    const uint4 h = *reinterpret_cast<const uint4 *>(blk);
    const uint4 a = *reinterpret_cast<const uint4 *>(blk + 16 + 32 * c);
    const uint4 b = *reinterpret_cast<const uint4 *>(blk + 32 + 32 * c);
    r.h[0] = h.x; r.h[1] = h.y; r.h[2] = h.z; r.h[3] = h.w;
    r.q[0] = a.x; r.q[1] = a.y; r.q[2] = a.z; r.q[3] = a.w;
    r.q[4] = b.x; r.q[5] = b.y; r.q[6] = b.z; r.q[7] = b.w;
}

// Q6_K blocks start on 2-byte boundaries: whole dwords from the 4-byte
// aligned address at or below each field, re-aligned by sh in decoding.
QD_DEV void lds_q6k(RawQ6K &r, const uint8_t *blk, int h, int j) {
    r.sh = (uint32_t)(lds_addr(blk) & 3u);
    const uint8_t *bp = blk - r.sh;
    const uint8_t *pa = bp + 64 * h + 16 * j;
    const uint8_t *ph = bp + 128 + 32 * h + 16 * j;
    const uint8_t *ps = bp + 192 + 8 * h;
#pragma unroll
    for (int k = 0; k < 5; k++) {
        r.a[k] = lds32(pa + 4 * k);
        r.b[k] = lds32(pa + 32 + 4 * k);
        r.h[k] = lds32(ph + 4 * k);
    }
#pragma unroll
    for (int k = 0; k < 3; k++) r.s[k] = lds32(ps + 4 * k);
    r.d = lds32(bp + 208);
}

// Q8_0 superunits are 16-byte aligned in the ring (272-byte units, rows of
// whole superunits), so lane c's two blocks start on a dword: block A (d,
// then quants 2 bytes in) is the "Q" case of load_q80 and block B (quants on
// a dword, d in the high half of the dword before) the "P" case.
QD_DEV void lds_q80(RawQ80 &r, const uint8_t *blk, int c) {
    const uint8_t *g = blk + 68 * c;
#pragma unroll
    for (int k = 0; k < 9; k++) r.q[k] = lds32(g + 4 * k);
    r.pd = r.q[8];
#pragma unroll
    for (int k = 0; k < 8; k++) r.p[k] = lds32(g + 36 + 4 * k);
    r.a_is_p = 0u;
}

// ------------------------------------------------- per-superunit dots ---
// xv: this lane's 64 activations (in the lane's own order, see each format)
// for each batch row; result: this lane's share of w . x per row stream.

// Q4_K: xv[0..7] low run (64c + 0..31), xv[8..15] high run; X: sums of x
// over sub-blocks 2c and 2c+1.
template <int NR, int B>
QD_DEV void dot_q4k(const RawQ4K (&r)[NR], const float4 (&xv)[B][16], const float2 (&X)[B],
                    const Q4Lane &L, float (&out)[NR][B]) {
    const float inv_unit = fp8_inv_unit();  // exact power of two
#pragma unroll
    for (int i = 0; i < NR; i++) {
        float alo[B], ahi[B];
#pragma unroll
        for (int b = 0; b < B; b++) { alo[b] = 0.f; ahi[b] = 0.f; }
#pragma unroll
        for (int dw = 0; dw < 8; dw++) {
            const Q4Nibbles n = q4k_nibbles(r[i].q[dw]);
#pragma unroll
            for (int b = 0; b < B; b++) {
                const float4 xl = xv[b][dw], xh = xv[b][8 + dw];
                float s = alo[b];
                s = fmaf(n.lo01.x, xl.x, s);
                s = fmaf(n.lo01.y, xl.y, s);
                s = fmaf(n.lo23.x, xl.z, s);
                s = fmaf(n.lo23.y, xl.w, s);
                alo[b] = s;
                float u = ahi[b];
                u = fmaf(n.hi01.x, xh.x, u);
                u = fmaf(n.hi01.y, xh.y, u);
                u = fmaf(n.hi23.x, xh.z, u);
                u = fmaf(n.hi23.y, xh.w, u);
                ahi[b] = u;
            }
        }
        const Q4Scales s = q4k_scales(r[i], L);
#pragma unroll
        for (int b = 0; b < B; b++) {
            const float q = s.d * fmaf(s.sc1, ahi[b], s.sc0 * alo[b]);
            const float m = s.dmin * fmaf(s.m1, X[b].y, s.m0 * X[b].x);
            out[i][b] = fmaf(q, inv_unit, -m);
        }
    }
}

// Q6_K: xv[4g + i] = activations of group g (16 per group).
template <int NR, int B>
QD_DEV void dot_q6k(const RawQ6K (&r)[NR], const float4 (&xv)[B][16], int j, float (&out)[NR][B]) {
#pragma unroll
    for (int i = 0; i < NR; i++) {
        float acc[B][4];
#pragma unroll
        for (int b = 0; b < B; b++)
#pragma unroll
            for (int g = 0; g < 4; g++) acc[b][g] = 0.f;
#pragma unroll
        for (int k = 0; k < 4; k++) {
            uint32_t q[4];
            q6k_qbytes(r[i], k, q);
#pragma unroll
            for (int g = 0; g < 4; g++) {
                const float w0 = sbyte(q[g], 0), w1 = sbyte(q[g], 1);
                const float w2 = sbyte(q[g], 2), w3 = sbyte(q[g], 3);
#pragma unroll
                for (int b = 0; b < B; b++) {
                    const float4 xx = xv[b][4 * g + k];
                    float s = acc[b][g];
                    s = fmaf(w0, xx.x, s);
                    s = fmaf(w1, xx.y, s);
                    s = fmaf(w2, xx.z, s);
                    s = fmaf(w3, xx.w, s);
                    acc[b][g] = s;
                }
            }
        }
        const Q6Scales s = q6k_scales(r[i], j);
#pragma unroll
        for (int b = 0; b < B; b++) {
            float u = s.sc[0] * acc[b][0];
            u = fmaf(s.sc[1], acc[b][1], u);
            u = fmaf(s.sc[2], acc[b][2], u);
            u = fmaf(s.sc[3], acc[b][3], u);
            out[i][b] = s.d * u;
        }
    }
}

// Q8_0: xv[0..7] block A (64c + 0..31), xv[8..15] block B.
template <int NR, int B>
QD_DEV void dot_q80(const RawQ80 (&r)[NR], const float4 (&xv)[B][16], float (&out)[NR][B]) {
#pragma unroll
    for (int i = 0; i < NR; i++) {
        const float2 d = q80_d(r[i]);
        float accA[B], accB[B];
#pragma unroll
        for (int b = 0; b < B; b++) { accA[b] = 0.f; accB[b] = 0.f; }
#pragma unroll
        for (int k = 0; k < 8; k++) {
            const uint2 v = q80_qdwords(r[i], k);
#pragma unroll
            for (int b = 0; b < B; b++) {
                const float4 xa = xv[b][k], xb = xv[b][8 + k];
                float s = accA[b];
                s = fmaf(sbyte(v.x, 0), xa.x, s);
                s = fmaf(sbyte(v.x, 1), xa.y, s);
                s = fmaf(sbyte(v.x, 2), xa.z, s);
                s = fmaf(sbyte(v.x, 3), xa.w, s);
                accA[b] = s;
                float u = accB[b];
                u = fmaf(sbyte(v.y, 0), xb.x, u);
                u = fmaf(sbyte(v.y, 1), xb.y, u);
                u = fmaf(sbyte(v.y, 2), xb.z, u);
                u = fmaf(sbyte(v.y, 3), xb.w, u);
                accB[b] = u;
            }
        }
#pragma unroll
        for (int b = 0; b < B; b++) out[i][b] = fmaf(d.y, accB[b], d.x * accA[b]);
    }
}

// ------------------------------------------------------ one step ---
// A lane's operands for one superunit: its share of the block (per row
// stream) and its 64 activations (per batch row) from LDS.
template <int FMT, int B, int NR>
struct StepRegs {
    typename RawOf<FMT>::T raw[NR];
    float4 xv[B][16];
    float2 X[B];  // Q4_K: sums of x over the lane's two sub-blocks
};

// blk0: the lane group's superunit in row stream 0 (stream m is m * mstride
// bytes further); su: its superunit index within the row.
template <int FMT, int B, int NR>
QD_DEV void read_step(StepRegs<FMT, B, NR> &st, const uint8_t *blk0, int mstride, const float *xl,
                      const float *xs, int xstride, int nb, int su, int c) {
#pragma unroll
    for (int m = 0; m < NR; m++) {
        const uint8_t *blk = blk0 + m * mstride;
        if constexpr (FMT == kQ4K) lds_q4k(st.raw[m], blk, c);
        else if constexpr (FMT == kQ6K) lds_q6k(st.raw[m], blk, c >> 1, c & 1);
        else lds_q80(st.raw[m], blk, c);
    }
#pragma unroll
    for (int b = 0; b < B; b++) {
        const float *xb = xl + b * xstride;
        if constexpr (FMT == kQ6K) {
            const int base = su * kSuper + 128 * (c >> 1) + 16 * (c & 1);
#pragma unroll
            for (int gg = 0; gg < 4; gg++) {
                const float4 *xg = reinterpret_cast<const float4 *>(xb + xphys(base + 32 * gg));
#pragma unroll
                for (int n = 0; n < 4; n++) st.xv[b][4 * gg + n] = xg[n];
            }
        } else {
            const float4 *xp = reinterpret_cast<const float4 *>(xb + xphys(su * kSuper + 64 * c));
#pragma unroll
            for (int n = 0; n < 16; n++) st.xv[b][n] = xp[n];
        }
        if constexpr (FMT == kQ4K)
            st.X[b] = *reinterpret_cast<const float2 *>(xs + b * nb * 8 + 8 * su + 2 * c);
        else
            st.X[b] = make_float2(0.f, 0.f);
    }
}

template <int FMT, int B, int NR>
QD_DEV void dot_step(const StepRegs<FMT, B, NR> &st, const Q4Lane &L4, int c, float (&v)[NR][B]) {
    if constexpr (FMT == kQ4K) dot_q4k<NR, B>(st.raw, st.xv, st.X, L4, v);
    else if constexpr (FMT == kQ6K) dot_q6k<NR, B>(st.raw, st.xv, c & 1, v);
    else dot_q80<NR, B>(st.raw, st.xv, v);
}

// ------------------------------------------------------------ kernel ---
template <int FMT, int B, int NR, bool FFN>
__global__ __launch_bounds__(kThreads) void stream_kernel(StreamArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    constexpr int UB = StreamFmt<FMT>::UB;
    constexpr int NCH = StreamFmt<FMT>::NCH;
    constexpr int NI = copies_per_step<FMT>();
    constexpr int SLOTM = NCH * 16;  // bytes of one matrix's step in a slot

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = lane & 3, g = lane >> 2;
    const int64_t N = a.N, K = a.K;
    const int nb = a.nb;
    const int PD = a.pd;

    // rows of this workgroup
    const int wg = blockIdx.x;
    const int64_t r0 = (int64_t)wg * a.rows_base + min(wg, a.rows_extra);
    const int cnt = a.rows_base + (wg < a.rows_extra ? 1 : 0);
    const int U = cnt * nb;                                   // superunits per matrix
    const int S = (U + kStepUnits - 1) / kStepUnits;          // steps
    const int nw = S > w ? (S - w + kWaves - 1) / kWaves : 0; // steps of this wave

    // LDS layout
    uint8_t *ring = smem + w * PD * NR * SLOTM;
    float *xl = reinterpret_cast<float *>(smem + a.off_x);
    float *xs = reinterpret_cast<float *>(smem + a.off_xsum);
    const float *nwl = reinterpret_cast<const float *>(smem + a.off_nw);
    float *part = reinterpret_cast<float *>(smem + a.off_part);
    float *red = reinterpret_cast<float *>(smem + a.off_red);
    const int xstride = nb * kSuperPhys;  // floats per staged batch row

    // byte stream of this workgroup's rows, per matrix; a step is copied
    // from the 16-byte boundary at or below its first byte
    const int64_t wbeg = r0 * a.row_bytes;
    const int off0 = (int)(wbeg & 15);
    const uint8_t *mats[NR];
    mats[0] = a.W0;
    if constexpr (NR == 2) mats[1] = a.W1;
    const int64_t last16 = a.mat_bytes - 16;  // last 16-byte chunk of a matrix

    auto issue = [&](int i, int slot) {
        // copies of this wave's i-th step (step w + 4 i) into ring slot `slot`
        const int step = w + kWaves * i;
        const int64_t a0 = ((wbeg + (int64_t)step * kStepUnits * UB) & ~(int64_t)15);
#pragma unroll
        for (int m = 0; m < NR; m++) {
            const uint32_t dst = lds_addr(ring + (slot * NR + m) * SLOTM);
#pragma unroll
            for (int j = 0; j < NI; j++) {
                const int64_t off = min(a0 + 16 * (int64_t)(64 * j + lane), last16);
                if (j < NI - 1 || lane < NCH - 64 * (NI - 1))
                    lds_copy16(mats[m] + off, dst + 1024 * j);
            }
        }
    };

    // ---- x into LDS: physical float p of batch row b holds logical
    // k = unskew(p); pad floats receive a harmless copy of x[0]
    const int xf4 = B * nb * (kSuperPhys / 4);  // float4 slots
    for (int f0 = w * 64; f0 < xf4; f0 += kThreads) {
        const int f = f0 + lane;
        const int b = f / (nb * (kSuperPhys / 4));
        const int p = 4 * (f - b * (nb * (kSuperPhys / 4)));  // physical float in the row
        const int t = p / kSuperPhys, q = p - t * kSuperPhys;
        const int run = q / 68, e = q - run * 68;
        const int64_t k = (int64_t)t * kSuper + run * 64 + e;
        const int64_t so = (e < 64 && k < K && f < xf4) ? (int64_t)b * K + k : 0;
        if (f0 + 64 <= xf4 || lane < xf4 - f0) lds_copy16(a.x + so, lds_addr(xl + 4 * f0));
    }
    // ---- the norm weight (K floats, unskewed) the same way
    const bool norm = a.norm_w != nullptr;
    if (norm) {
        const int nf4 = (int)(K / 4);
        for (int f0 = w * 64; f0 < nf4; f0 += kThreads)
            if (f0 + 64 <= nf4 || lane < nf4 - f0)
                lds_copy16(a.norm_w + 4 * (int64_t)(f0 + lane), lds_addr(nwl + 4 * f0));
    }

    // ---- the first steps of the weight stream (at most PD in flight)
    const int pro = min(PD, nw);
    for (int i = 0; i < pro; i++) issue(i, i);

    // ---- x (and the norm weight) landed: this wave's copies, then every wave's
    vm_wait_n(pro * NR * NI);
    block_sync();

    // ---- RMS-normalise in place; Q4_K: sums of every 32-run
    const int F = nb * (kSuper / 4);  // logical float4 per batch row
    if (norm) {
        float ss[B];
#pragma unroll
        for (int b = 0; b < B; b++) ss[b] = 0.f;
        for (int f = tid; f < B * F; f += kThreads) {
            const int b = f / F;
            const int k = 4 * (f - b * F);
            const float4 v = *reinterpret_cast<const float4 *>(xl + b * xstride + xphys(k));
            float sq = fmaf(v.x, v.x, 0.f);
            sq = fmaf(v.y, v.y, sq);
            sq = fmaf(v.z, v.z, sq);
            sq = fmaf(v.w, v.w, sq);
#pragma unroll
            for (int bb = 0; bb < B; bb++)
                if (bb == b) ss[bb] += sq;
        }
#pragma unroll
        for (int b = 0; b < B; b++) {
            const float t = wave_total(ss[b]);
            if (lane == 0) red[w * B + b] = t;
        }
        block_sync();
        float inv_rms[B];
#pragma unroll
        for (int b = 0; b < B; b++) {
            const float sq = (red[b] + red[B + b]) + (red[2 * B + b] + red[3 * B + b]);
            inv_rms[b] = 1.0f / sqrtf(sq / (float)K + a.eps);
        }
        for (int f = tid; f < B * F; f += kThreads) {
            const int b = f / F;
            const int k = 4 * (f - b * F);
            float4 *ad = reinterpret_cast<float4 *>(xl + b * xstride + xphys(k));
            float4 v = *ad;
            const float4 nw4 = *reinterpret_cast<const float4 *>(nwl + k);
            float ir = inv_rms[0];
#pragma unroll
            for (int bb = 1; bb < B; bb++)
                if (bb == b) ir = inv_rms[bb];
            v.x = v.x * ir * nw4.x;
            v.y = v.y * ir * nw4.y;
            v.z = v.z * ir * nw4.z;
            v.w = v.w * ir * nw4.w;
            *ad = v;
        }
        block_sync();
    }
    if constexpr (FMT == kQ4K) {
        // lanes 8m..8m+7 hold the 8 float4 of one 32-run: F is a multiple of 64
        for (int f = tid; f < B * F; f += kThreads) {
            const int b = f / F;
            const int k = 4 * (f - b * F);
            const float4 v = *reinterpret_cast<const float4 *>(xl + b * xstride + xphys(k));
            const float sm = oct_sum((v.x + v.y) + (v.z + v.w));
            if ((lane & 7) == 0) xs[b * nb * 8 + (k >> 5)] = sm;
        }
        block_sync();
    }

    // ---- the stream
    const int Umax = a.units_max;
    Q4Lane L4;
    if constexpr (FMT == kQ4K) L4 = q4k_lane(c);
    for (int i = 0; i < nw; i++) {
        const int slot = i % PD;
        // step i's copies are in LDS: the steps issued after it (at most
        // PD - 1, fewer at the end of the stream) may still be in flight
        vm_wait_n(min(PD - 1, nw - 1 - i) * NR * NI);
        const int step = w + kWaves * i;
        const int u = step * kStepUnits + g;  // this group's superunit
        const bool live = u < U;
        const int uu = live ? u : U - 1;
        const int lr = uu / nb;
        const int su = uu - lr * nb;
        const uint8_t *blk0 = ring + slot * NR * SLOTM + off0 + g * UB;

        StepRegs<FMT, B, NR> st;
        read_step<FMT, B, NR>(st, blk0, SLOTM, xl, xs, xstride, nb, su, c);
        // every read of this slot is complete before the slot is refilled
        // with step i + PD, which streams in while this one is decoded
        lgkm_wait();
        if (i + PD < nw) issue(i + PD, slot);

        float v[NR][B];
        dot_step<FMT, B, NR>(st, L4, c, v);
#pragma unroll
        for (int m = 0; m < NR; m++)
#pragma unroll
            for (int b = 0; b < B; b++) {
                const float t = quad_sum(v[m][b]);
                if (c == 0 && live) part[(m * B + b) * Umax + u] = t;
            }
    }
    vm_wait<0>();
    block_sync();

    // ---- rows: partials in superunit order
    for (int e = tid; e < cnt * B; e += kThreads) {
        const int b = e / cnt;
        const int lr = e - b * cnt;
        const int64_t row = r0 + lr;
        float sr[NR];
#pragma unroll
        for (int m = 0; m < NR; m++) {
            const float *pp = part + (m * B + b) * Umax + lr * nb;
            float acc = 0.f;
            for (int t = 0; t < nb; t++) acc += pp[t];
            sr[m] = acc;
        }
        if constexpr (FFN) {
            a.y[(int64_t)b * N + row] = act_apply(a.act, sr[0]) * sr[1];
            if (a.g_out) a.g_out[(int64_t)b * N + row] = sr[0];
            if (a.u_out) a.u_out[(int64_t)b * N + row] = sr[1];
        } else {
            const int64_t o = (int64_t)b * N + row;
            a.y[o] = a.res ? sr[0] + a.res[o] : sr[0];
        }
    }
}

// ------------------------------------------------ producer / consumer ---
// The same products with the two jobs given to different waves, which never
// wait on a workgroup barrier inside the stream.  A wave that issues copies
// stalls at issue whenever the memory pipeline backs up, so the copying waves
// do little else, and their copies are issued from scalar registers:
//   * waves 0 .. NC-1 decode (consumers).  First they copy x (and the norm
//     weight) into LDS, each a share of the 1 KB copies, and count
//     themselves on `landed` once theirs have landed.  Then they stage x
//     together, a 64-float4 slice at a time: x * w_norm in place, each
//     wave's sum of squares of x (added in wave order, so the inverse RMS
//     does not depend on timing), and for Q4_K the sum of every 32-run;
//     they meet on `staged`.  Then consumer c takes steps c, c + NC, ...
//     and, after reading a step out of its slot, stores the number of its
//     steps read so far in done[c];
//   * waves NC .. NC + 3 copy the weights (producers; as many as the launch
//     asks for, 1, 2 or 4, and the others idle).  They issue nothing before x has landed, so
//     x does not queue behind the weight stream.  Producer p takes the
//     steps j = p (mod producers), each into ring slot j % slots, keeping up
//     to `lag` of its steps in flight; once one of its steps has landed (its
//     own vmcnt) it stores the step number in ready[slot].
// Slot reuse: producer p may refill the slot of step j once step j - slots
// has been read, which it knows from the smallest done[] of its own
// consumers (consumers c = p mod producers take only producer p's steps).
// The host keeps slots a multiple of the producer count and, when slots are
// reused, slots >= NC + producers * (lag - 1): then every step such a wait
// depends on has been published, so the wait ends.  The RMS factor is
// applied to each row's sum at the end (every product is linear in the
// staged activations).
constexpr int kPcMaxProducers = 4;

template <int FMT, int B, int NR, bool FFN, int NC>
__global__ __launch_bounds__(64 * (NC + kPcMaxProducers)) void stream_pc_kernel(StreamArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    constexpr int UB = StreamFmt<FMT>::UB;
    constexpr int NCH = StreamFmt<FMT>::NCH;
    constexpr int NI = copies_per_step<FMT>();
    constexpr int SLOTM = NCH * 16;
    constexpr int CPS = NR * NI;  // copies per step
    constexpr int NT = 64 * (NC + kPcMaxProducers);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = lane & 3, g = lane >> 2;
    const int64_t N = a.N, K = a.K;
    const int nb = a.nb;
    const int R = a.slots;
    const int NP = a.producers;

    const int wg = blockIdx.x;
    const int64_t r0 = (int64_t)wg * a.rows_base + min(wg, a.rows_extra);
    const int cnt = a.rows_base + (wg < a.rows_extra ? 1 : 0);
    const int U = cnt * nb;
    const int S = (U + kStepUnits - 1) / kStepUnits;

    uint8_t *ring = smem;
    float *xl = reinterpret_cast<float *>(smem + a.off_x);
    float *xs = reinterpret_cast<float *>(smem + a.off_xsum);
    float *nwl = reinterpret_cast<float *>(smem + a.off_nw);
    float *part = reinterpret_cast<float *>(smem + a.off_part);
    int *ready = reinterpret_cast<int *>(smem + a.off_red);
    int *done = ready + R;     // [NC]
    int *landed = done + NC;
    int *staged = landed + 1;
    float *rinv = reinterpret_cast<float *>(staged + 1);  // [B]
    float *ssq = rinv + B;                                // [NC][B]
    const int xstride = nb * kSuperPhys;
    const int64_t wbeg = r0 * a.row_bytes;
    const int off0 = (int)(wbeg & 15);
    const bool norm = a.norm_w != nullptr;

    for (int i = tid; i < R + NC + 2; i += NT) ready[i] = i < R ? -1 : 0;
    block_sync();

    if (wv >= NC) {
        // ---------------------------------------------------- producer ---
        const int p = wv - NC;
        if (p < NP) {
            __builtin_amdgcn_s_setprio(3);
            lds_wait_eq(landed, NC);
            // weight steps j = p + NP * k
            constexpr int SB = kStepUnits * UB;  // bytes per step and matrix
            const int64_t base = wbeg & ~(int64_t)15;
            uint32_t voff[NI];  // lane offset of each of a step's copies
#pragma unroll
            for (int q = 0; q < NI; q++) voff[q] = 16u * (uint32_t)lane + 1024u * (uint32_t)q;
            const bool tail_lane = lane < NCH - 64 * (NI - 1);  // lanes of the last copy
            const int64_t safe = a.mat_bytes - (int64_t)NCH * 16;  // steps starting at or below copy whole
            const int lag = a.lag;
            const int nk = S > p ? (S - p + NP - 1) / NP : 0;
            int k = 0, kp = 0;            // next step to issue / to publish (own numbering)
            int slot = p, pslot = p;      // their slots
            int freed = 0;                // own steps below NC * freed have been read
            while (kp < nk) {
                while (k < nk && k - kp < lag) {
                    const int j = p + NP * k;
                    if (j >= R && j - R >= NC * freed) {
                        // smallest done[] of this producer's consumers
                        for (;;) {
                            int m = 0x7fffffff;
                            for (int cc = p; cc < NC; cc += NP) m = min(m, lds_poll(&done[cc]));
                            freed = m;
                            if (j - R < NC * freed) break;
                            __builtin_amdgcn_s_sleep(1);
                        }
                        asm volatile("" ::: "memory");
                    }
                    const uint32_t dst = lds_addr(ring + slot * NR * SLOTM);
                    const int64_t a0 = base + (int64_t)j * SB;
                    if (a0 <= safe) {
#pragma unroll
                        for (int m = 0; m < NR; m++) {
                            const uint8_t *sp = (m == 0 ? a.W0 : a.W1) + a0;
#pragma unroll
                            for (int q = 0; q < NI; q++)
                                if (q < NI - 1 || tail_lane)
                                    lds_copy16_s(sp, voff[q], dst + m * SLOTM + 1024 * q);
                        }
                    } else {
                        // only a step reaching past the end of the matrix: clamp
                        // its sources (per lane) to the matrix's last 16 bytes
                        const int64_t last16 = a.mat_bytes - 16;
#pragma unroll
                        for (int m = 0; m < NR; m++)
#pragma unroll
                            for (int q = 0; q < NI; q++) {
                                const int64_t off = min(a0 + 16 * (int64_t)(64 * q + lane), last16);
                                if (q < NI - 1 || tail_lane)
                                    lds_copy16((m == 0 ? a.W0 : a.W1) + off, dst + m * SLOTM + 1024 * q);
                            }
                    }
                    k++;
                    slot += NP;
                    if (slot >= R) slot -= R;
                }
                // own step kp has landed once at most (k - kp - 1) are in flight
                vm_wait_n((k - kp - 1) * CPS);
                if (lane == 0) lds_flag(&ready[pslot], p + NP * kp);
                kp++;
                pslot += NP;
                if (pslot >= R) pslot -= R;
            }
        }
    } else {
        // -------------------------------------------------- consumers ---
        // copy x: batch row b, physical float4 q of the row (17 per 64-float
        // run, the last a pad that receives a copy of x[0]) holds logical
        // float4 16 * (q / 17) + q % 17; then the norm weight.  Copy i of
        // the workgroup (64 float4 each) is issued by wave i % NC.
        {
            const int nq = nb * (kSuperPhys / 4);
            const int xc = (nq + 63) / 64;               // copies per batch row of x
            const int nf4 = norm ? (int)(K / 4) : 0;
            const int total = B * xc + (nf4 + 63) / 64;
            int n = 0;
            for (int i = wv; i < total; i += NC) {
                if (i < B * xc) {
                    const int b = i / xc;
                    const int q0 = 64 * (i - b * xc);
                    const int q = q0 + lane;
                    const int run = q / 17, e = q - 17 * run;
                    const float *xb = a.x + (int64_t)b * K;
                    const float *srcp = (e < 16 && q < nq) ? xb + 4 * (16 * run + e) : xb;
                    if (q0 + 64 <= nq || lane < nq - q0)
                        lds_copy16(srcp, lds_addr(xl + b * xstride + 4 * q0));
                } else {
                    const int f0 = 64 * (i - B * xc);
                    if (f0 + 64 <= nf4 || lane < nf4 - f0)
                        lds_copy16(a.norm_w + 4 * (int64_t)(f0 + lane), lds_addr(nwl + 4 * f0));
                }
                if (++n == 48) { vm_wait<16>(); n = 16; }
            }
            vm_wait<0>();
            if (lane == 0) lds_add(landed, 1);
        }
        // stage x: slice it (64 float4 of one batch row) goes to wave it % NC
        lds_wait_eq(landed, NC);
        const int F = nb * (kSuper / 4);  // logical float4 per batch row (a multiple of 64)
        const int nit = F / 64;
        float ss[B];
#pragma unroll
        for (int b = 0; b < B; b++) ss[b] = 0.f;
        for (int it = wv; it < B * nit; it += NC) {
            const int b = it / nit;
            const int k = 4 * (64 * (it - b * nit) + lane);
            float4 *ad = reinterpret_cast<float4 *>(xl + b * xstride + xphys(k));
            float4 v = *ad;
            if (norm) {
                float sq = fmaf(v.x, v.x, 0.f);
                sq = fmaf(v.y, v.y, sq);
                sq = fmaf(v.z, v.z, sq);
                sq = fmaf(v.w, v.w, sq);
#pragma unroll
                for (int bb = 0; bb < B; bb++)
                    if (bb == b) ss[bb] += sq;
                const float4 nw4 = *reinterpret_cast<const float4 *>(nwl + k);
                v.x *= nw4.x;
                v.y *= nw4.y;
                v.z *= nw4.z;
                v.w *= nw4.w;
                *ad = v;
            }
            if constexpr (FMT == kQ4K) {
                // lanes 8m .. 8m+7 hold the 8 float4 of one 32-run
                const float sm = oct_sum((v.x + v.y) + (v.z + v.w));
                if ((lane & 7) == 0) xs[b * nb * 8 + (k >> 5)] = sm;
            }
        }
        if (norm) {
#pragma unroll
            for (int b = 0; b < B; b++) {
                const float t = wave_total(ss[b]);
                if (lane == 0) ssq[wv * B + b] = t;
            }
        }
        lgkm_wait();
        if (lane == 0) lds_add(staged, 1);
        lds_wait_eq(staged, NC);
        if (wv == 0 && lane == 0) {
#pragma unroll
            for (int b = 0; b < B; b++) {
                float t = 0.f;
                for (int w = 0; w < NC; w++) t += norm ? ssq[w * B + b] : 0.f;
                rinv[b] = norm ? 1.0f / sqrtf(t / (float)K + a.eps) : 1.0f;
            }
        }
        const int Umax = a.units_max;
        Q4Lane L4;
        if constexpr (FMT == kQ4K) L4 = q4k_lane(c);
        int slot = wv % R, nread = 0;
        const int sstep = NC % R;
        for (int j = wv; j < S; j += NC) {
            const int u = j * kStepUnits + g;
            const bool live = u < U;
            const int uu = live ? u : U - 1;
            const int lr = uu / nb;
            const int su = uu - lr * nb;
            lds_wait_eq(&ready[slot], j);
            StepRegs<FMT, B, NR> st;
            read_step<FMT, B, NR>(st, ring + slot * NR * SLOTM + off0 + g * UB, SLOTM, xl, xs, xstride,
                                  nb, su, c);
            lgkm_wait();  // the slot may be refilled from here on
            if (lane == 0) lds_flag(&done[wv], ++nread);
            float v[NR][B];
            dot_step<FMT, B, NR>(st, L4, c, v);
#pragma unroll
            for (int m = 0; m < NR; m++)
#pragma unroll
                for (int b = 0; b < B; b++) {
                    const float t = quad_sum(v[m][b]);
                    if (c == 0 && live) part[(m * B + b) * Umax + u] = t;
                }
            slot += sstep;
            if (slot >= R) slot -= R;
        }
    }
    block_sync();

    // ---- rows: partials in superunit order, times the inverse RMS
    const int Umax = a.units_max;
    for (int e = tid; e < cnt * B; e += NT) {
        const int b = e / cnt;
        const int lr = e - b * cnt;
        const int64_t row = r0 + lr;
        float sr[NR];
#pragma unroll
        for (int m = 0; m < NR; m++) {
            const float *pp = part + (m * B + b) * Umax + lr * nb;
            float acc = 0.f;
            for (int t = 0; t < nb; t++) acc += pp[t];
            sr[m] = acc * rinv[b];
        }
        if constexpr (FFN) {
            a.y[(int64_t)b * N + row] = act_apply(a.act, sr[0]) * sr[1];
            if (a.g_out) a.g_out[(int64_t)b * N + row] = sr[0];
            if (a.u_out) a.u_out[(int64_t)b * N + row] = sr[1];
        } else {
            const int64_t o = (int64_t)b * N + row;
            a.y[o] = a.res ? sr[0] + a.res[o] : sr[0];
        }
    }
}

// ------------------------------------------------ shared stream pieces ---
// Copies of one step (16 superunits of each of NR row streams) into LDS at
// dst (stream m at dst + m * SLOTM), from the 16-byte boundary a0 of the
// workgroup's byte stream.  `whole`: the step lies inside the matrix, so the
// copies are issued from a scalar base and a per-lane offset; otherwise each
// lane's source is clamped to the matrix's last 16 bytes.
template <int NI, int NCH, int SLOTM, int NR>
QD_DEV void issue_step(const uint8_t *W0, const uint8_t *W1, int64_t a0, bool whole, int64_t mat_bytes,
                       uint32_t dst, int lane, bool tail_lane) {
    if (whole) {
#pragma unroll
        for (int m = 0; m < NR; m++) {
            const uint8_t *sp = (m == 0 ? W0 : W1) + a0;
#pragma unroll
            for (int q = 0; q < NI; q++)
                if (q < NI - 1 || tail_lane)
                    lds_copy16_s(sp, 16u * (uint32_t)lane + 1024u * (uint32_t)q, dst + m * SLOTM + 1024 * q);
        }
    } else {
        const int64_t last16 = mat_bytes - 16;
#pragma unroll
        for (int m = 0; m < NR; m++)
#pragma unroll
            for (int q = 0; q < NI; q++) {
                const int64_t off = min(a0 + 16 * (int64_t)(64 * q + lane), last16);
                if (q < NI - 1 || tail_lane) lds_copy16((m == 0 ? W0 : W1) + off, dst + m * SLOTM + 1024 * q);
            }
    }
}

// This wave's share (copies wv, wv + NC, ...) of copying one activation row
// of K floats into the skewed LDS layout (physical float4 q of the row holds
// logical float4 16 * (q / 17) + q % 17; pad float4 receive a copy of x[0]),
// and of the norm weight (K floats, unskewed) when nwsrc is not null.  COH:
// device-scope loads.  Returns when this wave's copies have landed.
template <int NC, bool COH>
QD_DEV void copy_x_share(const float *x, int64_t K, int nb, float *xl, const float *nwsrc, float *nwl, int wv,
                         int lane) {
    const int nq = nb * (kSuperPhys / 4);
    const int xc = (nq + 63) / 64;
    const int nf4 = nwsrc ? (int)(K / 4) : 0;
    const int total = xc + (nf4 + 63) / 64;
    int n = 0;
    for (int i = wv; i < total; i += NC) {
        if (i < xc) {
            const int q0 = 64 * i;
            const int q = q0 + lane;
            const int run = q / 17, e = q - 17 * run;
            const float *srcp = (e < 16 && q < nq) ? x + 4 * (16 * run + e) : x;
            if (q0 + 64 <= nq || lane < nq - q0) {
                if constexpr (COH) lds_copy16_coh(srcp, lds_addr(xl + 4 * q0));
                else lds_copy16(srcp, lds_addr(xl + 4 * q0));
            }
        } else {
            const int f0 = 64 * (i - xc);
            if (f0 + 64 <= nf4 || lane < nf4 - f0) lds_copy16(nwsrc + 4 * (int64_t)(f0 + lane), lds_addr(nwl + 4 * f0));
        }
        if (++n == 48) {
            vm_wait<16>();
            n = 16;
        }
    }
    vm_wait<0>();
}

// This wave's share (64-float4 slices wv, wv + NC, ...) of staging one
// activation row in place: x * w_norm when nwl is not null, and for Q4_K
// the sum of every 32-run into xs.  Returns the wave's sum of squares of x
// (0 without a norm weight); every lane takes part.
template <int FMT, int NC>
QD_DEV float stage_x_share(float *xl, float *xs, const float *nwl, int nb, int wv, int lane) {
    float ss = 0.f;
    for (int it = wv; it < nb; it += NC) {  // nb slices of 64 float4 per row
        const int k = 4 * (64 * it + lane);
        float4 *ad = reinterpret_cast<float4 *>(xl + xphys(k));
        float4 v = *ad;
        if (nwl) {
            float sq = fmaf(v.x, v.x, 0.f);
            sq = fmaf(v.y, v.y, sq);
            sq = fmaf(v.z, v.z, sq);
            sq = fmaf(v.w, v.w, sq);
            ss += sq;
            const float4 nw4 = *reinterpret_cast<const float4 *>(nwl + k);
            v.x *= nw4.x;
            v.y *= nw4.y;
            v.z *= nw4.z;
            v.w *= nw4.w;
            *ad = v;
        }
        if constexpr (FMT == kQ4K) {
            const float sm = oct_sum((v.x + v.y) + (v.z + v.w));
            if ((lane & 7) == 0) xs[k >> 5] = sm;
        }
    }
    return nwl ? wave_total(ss) : 0.f;
}

// ------------------------------------------------- one-launch decode FFN ---
// h = act(Wg x') * (Wu x') with x' = RMS-norm(x), then y = Wd h, batch 1, in
// one launch of one workgroup per CU, built from the producer / consumer
// kernel above.  Phase A (gate/up) and phase B (down) each own a ring; the
// copying waves stream phase A's steps and then phase B's without a break,
// so the down weights stream in while gate/up is still being decoded.
// Between the phases:
//   * the decoding waves of a workgroup sum their gate/up rows, apply the
//     activation and store their h rows with device-scope stores;
//   * the workgroup then arrives at a grid barrier (a device-scope counter
//     that the last arriver resets, and a generation word it advances); the
//     wait is bounded (about 50 ms), so a grid that is not all resident at
//     once ends with wrong numbers instead of hanging;
//   * the decoding waves copy h (device-scope loads) into the LDS that
//     phase A's ring and x used, and decode phase B's steps.
// A copying wave never waits for a free slot while one of its issued steps
// is still unpublished (it publishes instead), so it cannot hold up the
// steps the decoding waves need; phase A's steps come first in its order,
// so every workgroup finishes phase A whatever phase B's ring holds.
constexpr int kFfnSpinLimit = 1 << 20;

template <int FA, int FB, int NC>
__global__ __launch_bounds__(64 * (NC + 2)) void ffn_pc_kernel(FfnStreamArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    constexpr int UBA = StreamFmt<FA>::UB, NCHA = StreamFmt<FA>::NCH;
    constexpr int NIA = copies_per_step<FA>(), SLOTA = NCHA * 16, CPSA = 2 * NIA;
    constexpr int UBB = StreamFmt<FB>::UB, NCHB = StreamFmt<FB>::NCH;
    constexpr int NIB = copies_per_step<FB>(), SLOTB = NCHB * 16, CPSB = NIB;
    constexpr int NP = 2;  // copying waves

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = lane & 3, g = lane >> 2;
    const int wg = blockIdx.x;
    const int G = gridDim.x;

    // rows of this workgroup in each phase
    const int64_t rA0 = (int64_t)wg * a.rowsA_base + min(wg, a.rowsA_extra);
    const int cntA = a.rowsA_base + (wg < a.rowsA_extra ? 1 : 0);
    const int UA = cntA * a.nbA;
    const int SA = (UA + kStepUnits - 1) / kStepUnits;
    const int64_t rB0 = (int64_t)wg * a.rowsB_base + min(wg, a.rowsB_extra);
    const int cntB = a.rowsB_base + (wg < a.rowsB_extra ? 1 : 0);
    const int UB_ = cntB * a.nbB;
    const int SB = (UB_ + kStepUnits - 1) / kStepUnits;
    const int RA = a.slotsA, RB = a.slotsB;

    uint8_t *ringA = smem + a.off_ringA;
    uint8_t *ringB = smem + a.off_ringB;
    float *xA = reinterpret_cast<float *>(smem + a.off_xA);
    float *xsA = reinterpret_cast<float *>(smem + a.off_xsA);
    float *nwA = reinterpret_cast<float *>(smem + a.off_nwA);
    float *xB = reinterpret_cast<float *>(smem + a.off_xB);
    float *xsB = reinterpret_cast<float *>(smem + a.off_xsB);
    float *partA = reinterpret_cast<float *>(smem + a.off_partA);
    float *partB = reinterpret_cast<float *>(smem + a.off_partB);
    int *readyA = reinterpret_cast<int *>(smem + a.off_flags);
    int *readyB = readyA + RA;
    int *doneA = readyB + RB;     // [NC]
    int *doneB = doneA + NC;      // [NC]
    int *cnt = doneB + NC;        // counters below
    int *landed = cnt + 0, *staged = cnt + 1, *adone = cnt + 2, *hdone = cnt + 3;
    int *hready = cnt + 4, *bland = cnt + 5, *bstaged = cnt + 6, *bdone = cnt + 7;
    float *ssq = reinterpret_cast<float *>(cnt + 8);  // [NC]
    const int nflags = RA + RB + 2 * NC + 8;
    const int xstrideA = a.nbA * kSuperPhys, xstrideB = a.nbB * kSuperPhys;
    const int64_t wbegA = rA0 * a.row_bytesA, wbegB = rB0 * a.row_bytesB;
    const bool norm = a.norm_w != nullptr;

    for (int i = tid; i < nflags; i += 64 * (NC + 2)) readyA[i] = i < RA + RB ? -1 : 0;
    block_sync();

    if (wv >= NC) {
        // ---------------------------------------------------- producers ---
        const int p = wv - NC;
        __builtin_amdgcn_s_setprio(3);
        lds_wait_eq(landed, NC);
        const int nkA = SA > p ? (SA - p + NP - 1) / NP : 0;
        const int nkB = SB > p ? (SB - p + NP - 1) / NP : 0;
        const int nk = nkA + nkB;
        const int64_t baseA = wbegA & ~(int64_t)15, baseB = wbegB & ~(int64_t)15;
        const int64_t safeA = a.mat_bytesA - (int64_t)NCHA * 16, safeB = a.mat_bytesB - (int64_t)NCHB * 16;
        const bool tailA = lane < NCHA - 64 * (NIA - 1), tailB = lane < NCHB - 64 * (NIB - 1);
        int k = 0, kp = 0;
        int slotA = p, pslotA = p, slotB = p, pslotB = p;
        int freedA = 0, freedB = 0;
        auto smallest = [&](const int *done) {
            int m = 0x7fffffff;
            for (int cc = p; cc < NC; cc += NP) m = min(m, lds_poll(&done[cc]));
            return m;
        };
        while (kp < nk) {
            bool issued = false;
            if (k < nk && k - kp < a.lag) {
                const bool isA = k < nkA;
                const int j = isA ? p + NP * k : p + NP * (k - nkA);
                const int R = isA ? RA : RB;
                int &freed = isA ? freedA : freedB;
                bool wait = j >= R && j - R >= NC * freed;
                if (wait) {
                    freed = smallest(isA ? doneA : doneB);
                    wait = j - R >= NC * freed;
                }
                if (wait && k == kp) {
                    // nothing unpublished: wait for the slot
                    while (wait) {
                        __builtin_amdgcn_s_sleep(1);
                        freed = smallest(isA ? doneA : doneB);
                        wait = j - R >= NC * freed;
                    }
                }
                if (!wait) {
                    asm volatile("" ::: "memory");
                    if (isA) {
                        const uint32_t dst = lds_addr(ringA + slotA * 2 * SLOTA);
                        const int64_t a0 = baseA + (int64_t)j * kStepUnits * UBA;
                        issue_step<NIA, NCHA, SLOTA, 2>(a.Wg, a.Wu, a0, a0 <= safeA, a.mat_bytesA, dst, lane, tailA);
                        slotA += NP;
                        if (slotA >= RA) slotA -= RA;
                    } else {
                        const uint32_t dst = lds_addr(ringB + slotB * SLOTB);
                        const int64_t a0 = baseB + (int64_t)j * kStepUnits * UBB;
                        issue_step<NIB, NCHB, SLOTB, 1>(a.Wd, nullptr, a0, a0 <= safeB, a.mat_bytesB, dst, lane, tailB);
                        slotB += NP;
                        if (slotB >= RB) slotB -= RB;
                    }
                    k++;
                    issued = true;
                }
            }
            if (!issued) {
                // publish own step kp: it has landed once the copies of the
                // steps issued after it are all that is outstanding
                const int nA = max(0, min(k, nkA) - (kp + 1));
                const int nB = max(0, k - max(kp + 1, nkA));
                vm_wait_n(nA * CPSA + nB * CPSB);
                if (kp < nkA) {
                    if (lane == 0) lds_flag(&readyA[pslotA], p + NP * kp);
                    pslotA += NP;
                    if (pslotA >= RA) pslotA -= RA;
                } else {
                    if (lane == 0) lds_flag(&readyB[pslotB], p + NP * (kp - nkA));
                    pslotB += NP;
                    if (pslotB >= RB) pslotB -= RB;
                }
                kp++;
            }
        }
        return;
    }

    // -------------------------------------------------------- consumers ---
    Q4Lane L4;
    L4 = q4k_lane(c);
    // phase A: x and the norm weight
    copy_x_share<NC, false>(a.x, a.KA, a.nbA, xA, norm ? a.norm_w : nullptr, nwA, wv, lane);
    if (lane == 0) lds_add(landed, 1);
    lds_wait_eq(landed, NC);
    {
        const float ss = stage_x_share<FA, NC>(xA, xsA, norm ? nwA : nullptr, a.nbA, wv, lane);
        if (lane == 0) ssq[wv] = ss;
        lgkm_wait();
        if (lane == 0) lds_add(staged, 1);
        lds_wait_eq(staged, NC);
    }
    float rinv = 1.0f;
    if (norm) {
        float t = 0.f;
        for (int w = 0; w < NC; w++) t += ssq[w];
        rinv = 1.0f / sqrtf(t / (float)a.KA + a.eps);
    }
    {
        const int off0 = (int)(wbegA & 15);
        int slot = wv % RA, nread = 0;
        const int sstep = NC % RA;
        for (int j = wv; j < SA; j += NC) {
            const int u = j * kStepUnits + g;
            const bool live = u < UA;
            const int uu = live ? u : UA - 1;
            const int su = uu - (uu / a.nbA) * a.nbA;
            lds_wait_eq(&readyA[slot], j);
            StepRegs<FA, 1, 2> st;
            read_step<FA, 1, 2>(st, ringA + slot * 2 * SLOTA + off0 + g * UBA, SLOTA, xA, xsA, xstrideA, a.nbA,
                                su, c);
            lgkm_wait();
            if (lane == 0) lds_flag(&doneA[wv], ++nread);
            float v[2][1];
            dot_step<FA, 1, 2>(st, L4, c, v);
#pragma unroll
            for (int m = 0; m < 2; m++) {
                const float t = quad_sum(v[m][0]);
                if (c == 0 && live) partA[m * a.unitsA_max + u] = t;
            }
            slot += sstep;
            if (slot >= RA) slot -= RA;
        }
    }
    lgkm_wait();
    if (lane == 0) lds_add(adone, 1);
    lds_wait_eq(adone, NC);
    // h rows of this workgroup (device-scope stores, then counted)
    for (int lr = wv * 64 + lane; lr < cntA; lr += NC * 64) {
        const float *pg = partA + lr * a.nbA, *pu = partA + a.unitsA_max + lr * a.nbA;
        float sg = 0.f, su_ = 0.f;
        for (int t = 0; t < a.nbA; t++) {
            sg += pg[t];
            su_ += pu[t];
        }
        sg *= rinv;
        su_ *= rinv;
        __hip_atomic_store(a.h + rA0 + lr, act_apply(a.act, sg) * su_, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
    vm_wait<0>();
    if (lane == 0) lds_add(hdone, 1);
    if (wv == 0) {
        lds_wait_eq(hdone, NC);
        if (lane == 0) {
            // h is already at device scope (device-scope stores, waited for),
            // so the barrier's own accesses are relaxed device-scope atomics:
            // a fence per poll would write back and invalidate caches on
            // every one of them
            unsigned *arrived = a.bar, *gen = a.bar + 32;
            const unsigned g0 = __hip_atomic_load(gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // g0 read before arriving
            const unsigned n = __hip_atomic_fetch_add(arrived, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (n == (unsigned)G - 1) {
                __hip_atomic_store(arrived, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // reset before the generation moves
                __hip_atomic_fetch_add(gen, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            } else {
                for (int it = 0; it < kFfnSpinLimit; it++) {
                    if (__hip_atomic_load(gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != g0) break;
                    __builtin_amdgcn_s_sleep(2);
                }
            }
            lds_flag(hready, 1);
        }
    }
    lds_wait_eq(hready, 1);
    // phase B: h into the LDS that phase A's ring and x used
    copy_x_share<NC, true>(a.h, a.KB, a.nbB, xB, nullptr, nullptr, wv, lane);
    if (lane == 0) lds_add(bland, 1);
    lds_wait_eq(bland, NC);
    if constexpr (FB == kQ4K) {
        (void)stage_x_share<FB, NC>(xB, xsB, nullptr, a.nbB, wv, lane);
        lgkm_wait();
        if (lane == 0) lds_add(bstaged, 1);
        lds_wait_eq(bstaged, NC);
    }
    {
        const int off0 = (int)(wbegB & 15);
        int slot = wv % RB, nread = 0;
        const int sstep = NC % RB;
        for (int j = wv; j < SB; j += NC) {
            const int u = j * kStepUnits + g;
            const bool live = u < UB_;
            const int uu = live ? u : UB_ - 1;
            const int su = uu - (uu / a.nbB) * a.nbB;
            lds_wait_eq(&readyB[slot], j);
            StepRegs<FB, 1, 1> st;
            read_step<FB, 1, 1>(st, ringB + slot * SLOTB + off0 + g * UBB, SLOTB, xB, xsB, xstrideB, a.nbB, su, c);
            lgkm_wait();
            if (lane == 0) lds_flag(&doneB[wv], ++nread);
            float v[1][1];
            dot_step<FB, 1, 1>(st, L4, c, v);
            const float t = quad_sum(v[0][0]);
            if (c == 0 && live) partB[u] = t;
            slot += sstep;
            if (slot >= RB) slot -= RB;
        }
    }
    lgkm_wait();
    if (lane == 0) lds_add(bdone, 1);
    lds_wait_eq(bdone, NC);
    for (int lr = wv * 64 + lane; lr < cntB; lr += NC * 64) {
        const float *pp = partB + lr * a.nbB;
        float acc = 0.f;
        for (int t = 0; t < a.nbB; t++) acc += pp[t];
        a.y[rB0 + lr] = a.res ? acc + a.res[rB0 + lr] : acc;
    }
}

}  // namespace

// LDS bytes and layout of one workgroup; 0 if it does not fit.
size_t stream_layout(int fmt, int batch, bool ffn, int nb, int units_max, int pd, StreamArgs *a) {
    const int NR = ffn ? 2 : 1;
    int nch = fmt == kQ4K ? StreamFmt<kQ4K>::NCH : fmt == kQ6K ? StreamFmt<kQ6K>::NCH
                                                                : StreamFmt<kQ80>::NCH;
    size_t off = (size_t)kWaves * pd * NR * nch * 16;
    a->off_x = (int)off;
    off += (size_t)batch * nb * kSuperPhys * 4;
    a->off_xsum = (int)off;
    if (fmt == kQ4K) off += (size_t)batch * nb * 8 * 4;
    a->off_nw = (int)off;
    if (a->norm_w) off += (size_t)nb * kSuper * 4;
    a->off_part = (int)off;
    off += (size_t)NR * batch * units_max * 4;
    a->off_red = (int)off;
    off += 16 * 4;
    return off;
}

// LDS layout of the producer / consumer kernel with `slots` ring slots; returns
// the bytes used.
size_t stream_pc_layout(int fmt, int batch, bool ffn, int nb, int units_max, int slots,
                        StreamArgs *a) {
    const int NR = ffn ? 2 : 1;
    int nch = fmt == kQ4K ? StreamFmt<kQ4K>::NCH : fmt == kQ6K ? StreamFmt<kQ6K>::NCH
                                                                : StreamFmt<kQ80>::NCH;
    size_t off = (size_t)slots * NR * nch * 16;
    a->off_x = (int)off;
    off += (size_t)batch * nb * kSuperPhys * 4;
    a->off_xsum = (int)off;
    if (fmt == kQ4K) off += (size_t)batch * nb * 8 * 4;
    a->off_nw = (int)off;
    if (a->norm_w) off += (size_t)nb * kSuper * 4;
    a->off_part = (int)off;
    off += (size_t)NR * batch * units_max * 4;
    a->off_red = (int)off;  // ready[slots], done[consumers], landed, staged, rinv[batch], ssq[consumers][batch]
    off += (size_t)(slots + a->consumers + 2 + batch + a->consumers * batch) * 4;
    return (off + 15) & ~(size_t)15;
}

int stream_copies_per_step(int fmt, bool ffn) {
    const int NR = ffn ? 2 : 1;
    switch (fmt) {
    case kQ4K: return NR * copies_per_step<kQ4K>();
    case kQ6K: return NR * copies_per_step<kQ6K>();
    case kQ80: return NR * copies_per_step<kQ80>();
    default: return 0;
    }
}

// Allow each kernel the whole LDS of a CU (once per kernel).
template <auto Kern>
static hipError_t allow_lds() {
    static const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(Kern),
                                                    hipFuncAttributeMaxDynamicSharedMemorySize,
                                                    160 * 1024);
    return e;
}

template <int FMT, int B, bool FFN, int NC>
static hipError_t launch_pc(const StreamArgs &a, unsigned grid, size_t lds, hipStream_t st) {
    constexpr int NR = FFN ? 2 : 1;
    if (allow_lds<stream_pc_kernel<FMT, B, NR, FFN, NC>>() != hipSuccess) return hipErrorInvalidValue;
    hipLaunchKernelGGL((stream_pc_kernel<FMT, B, NR, FFN, NC>), dim3(grid), dim3(64 * (NC + kPcMaxProducers)), lds,
                       st, a);
    return hipGetLastError();
}

template <int FMT, int B>
static hipError_t launch_sb(const StreamArgs &a, bool ffn, unsigned grid, size_t lds, hipStream_t st) {
    if (a.consumers == 4)
        return ffn ? launch_pc<FMT, B, true, 4>(a, grid, lds, st) : launch_pc<FMT, B, false, 4>(a, grid, lds, st);
    if (a.consumers == 8)
        return ffn ? launch_pc<FMT, B, true, 8>(a, grid, lds, st) : launch_pc<FMT, B, false, 8>(a, grid, lds, st);
    if (a.consumers != 0) return hipErrorInvalidValue;
    if (ffn) {
        if (allow_lds<stream_kernel<FMT, B, 2, true>>() != hipSuccess) return hipErrorInvalidValue;
        hipLaunchKernelGGL((stream_kernel<FMT, B, 2, true>), dim3(grid), dim3(kThreads), lds, st, a);
    } else {
        if (allow_lds<stream_kernel<FMT, B, 1, false>>() != hipSuccess) return hipErrorInvalidValue;
        hipLaunchKernelGGL((stream_kernel<FMT, B, 1, false>), dim3(grid), dim3(kThreads), lds, st, a);
    }
    return hipGetLastError();
}

template <int FMT>
static hipError_t launch_sf(const StreamArgs &a, int batch, bool ffn, unsigned grid, size_t lds,
                            hipStream_t st) {
    switch (batch) {
    case 1: return launch_sb<FMT, 1>(a, ffn, grid, lds, st);
    case 2: return launch_sb<FMT, 2>(a, ffn, grid, lds, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_stream(int fmt, int batch, bool ffn, const StreamArgs &a, unsigned grid,
                         size_t lds, hipStream_t st) {
    switch (fmt) {
    case kQ4K: return launch_sf<kQ4K>(a, batch, ffn, grid, lds, st);
    case kQ6K: return launch_sf<kQ6K>(a, batch, ffn, grid, lds, st);
    case kQ80: return launch_sf<kQ80>(a, batch, ffn, grid, lds, st);
    default: return hipErrorInvalidValue;
    }
}


// ------------------------------------------------ one-launch decode FFN ---
template <int FA, int FB>
static hipError_t launch_ffn_pc_fb(const FfnStreamArgs &a, unsigned grid, size_t lds, hipStream_t st) {
    if (allow_lds<ffn_pc_kernel<FA, FB, 8>>() != hipSuccess) return hipErrorInvalidValue;
    hipLaunchKernelGGL((ffn_pc_kernel<FA, FB, 8>), dim3(grid), dim3(64 * (8 + 2)), lds, st, a);
    return hipGetLastError();
}

template <int FA>
static hipError_t launch_ffn_pc_fa(int fmt_b, const FfnStreamArgs &a, unsigned grid, size_t lds, hipStream_t st) {
    switch (fmt_b) {
    case kQ4K: return launch_ffn_pc_fb<FA, kQ4K>(a, grid, lds, st);
    case kQ6K: return launch_ffn_pc_fb<FA, kQ6K>(a, grid, lds, st);
    case kQ80: return launch_ffn_pc_fb<FA, kQ80>(a, grid, lds, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_ffn_stream(int fmt_a, int fmt_b, const FfnStreamArgs &a, unsigned grid, size_t lds,
                             hipStream_t st) {
    switch (fmt_a) {
    case kQ4K: return launch_ffn_pc_fa<kQ4K>(fmt_b, a, grid, lds, st);
    case kQ6K: return launch_ffn_pc_fa<kQ6K>(fmt_b, a, grid, lds, st);
    case kQ80: return launch_ffn_pc_fa<kQ80>(fmt_b, a, grid, lds, st);
    default: return hipErrorInvalidValue;
    }
}

static int nch_of(int fmt) {
    return fmt == kQ4K ? StreamFmt<kQ4K>::NCH : fmt == kQ6K ? StreamFmt<kQ6K>::NCH : StreamFmt<kQ80>::NCH;
}

// LDS layout of the one-launch FFN (8 decoding waves): phase B's ring, then
// the region phase A's ring, x, run sums and norm weight share with phase
// B's h and run sums, then the partials and the flags.  Returns the bytes
// used.
size_t ffn_stream_layout(int fmt_a, int fmt_b, bool norm, int slotsA, int slotsB, FfnStreamArgs *a) {
    constexpr int NC = 8;
    size_t off = 0;
    a->off_ringB = 0;
    off += (size_t)slotsB * nch_of(fmt_b) * 16;
    const size_t region = off;
    a->off_ringA = (int)off;
    size_t ra = (size_t)slotsA * 2 * nch_of(fmt_a) * 16;
    a->off_xA = (int)(region + ra);
    ra += (size_t)a->nbA * kSuperPhys * 4;
    a->off_xsA = (int)(region + ra);
    ra += (size_t)a->nbA * 8 * 4;
    a->off_nwA = (int)(region + ra);
    if (norm) ra += (size_t)a->nbA * kSuper * 4;
    size_t rb = 0;
    a->off_xB = (int)region;
    rb += (size_t)a->nbB * kSuperPhys * 4;
    a->off_xsB = (int)(region + rb);
    rb += (size_t)a->nbB * 8 * 4;
    off = region + std::max(ra, rb);
    a->off_partA = (int)off;
    off += (size_t)2 * a->unitsA_max * 4;
    a->off_partB = (int)off;
    off += (size_t)a->unitsB_max * 4;
    off = (off + 15) & ~(size_t)15;
    a->off_flags = (int)off;
    off += (size_t)(slotsA + slotsB + 2 * NC + 8 + NC) * 4;
    return (off + 15) & ~(size_t)15;
}

int ffn_stream_copies(int fmt_a, int fmt_b) {
    const int cpa = 2 * ((nch_of(fmt_a) + 63) / 64), cpb = (nch_of(fmt_b) + 63) / 64;
    return cpa > cpb ? cpa : cpb;
}

}  // namespace qd
