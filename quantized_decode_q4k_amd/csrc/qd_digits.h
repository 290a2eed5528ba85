// qd_digits.h -- activation digits for the batch-1..2 GEMV paths: exact
// integer dot products against the quantised weights.
//
// What is computed is unchanged: y = sum_k w_k x_k with w the dequantised
// weights of the larql "Architecture -> Metal shader map" page's k-quant
// blocks (Q4_K, Q6_K) and dotLLM PR #320's Q8_0.  How it is computed at
// batch 1-2 differs from a chain of fp32 fused multiply-adds:
//
//  * Each run of 32 activations (aligned to 32; a Q4_K sub-block, a Q8_0
//    block, two Q6_K sub-blocks) is written as 2^-s X_i, with one exponent
//    s per run chosen so that |X_i| <= 2^30, X_i = rint(x_i 2^s).  This is
//    the only rounding of x: none at all for the elements within a factor
//    2^7 of the run's largest magnitude (their x 2^s is already an integer),
//    at most 2^-31 of that magnitude for the others.
//  * X_i is split into four signed bytes, X = d0 + 2^8 d1 + 2^16 d2 +
//    2^24 d3 (balanced digits, each in -128..127), stored as four byte
//    planes so that one dword of a plane holds the digits of four
//    consecutive activations.
//  * A sub-block's sum I = sum_i q_i X_i over its integer quants q_i (Q4_K
//    q in 0..15, Q6_K q - 32 in -32..31, Q8_0 q in -128..127) is formed
//    exactly with v_dot4_i32_i8: four 4-way byte dot products per four
//    weights, one per digit plane (each plane's sum stays below 2^20), then
//    I = (a3 2^8 + a2) 2^16 + (a1 2^8 + a0).
//  * The block scales are applied per sub-block.  Q6_K and Q8_0 in fp32:
//    (d sc 2^-s) I, a product of an exact factor and I rounded once.  Q4_K
//    in fp64: d sc 2^-s I - dmin m 2^-s sum_i X_i, with I exact in fp64, so
//    a sub-block whose scale and min terms cancel is as accurate as any
//    other.
//
// Per weight this is one dot instruction plus the nibble or byte assembly,
// against one fused multiply-add plus the per-weight scale-and-min formation
// (Q4_K) or convert (Q6_K, Q8_0) of the fp32 form.
//
// A run holding a NaN or an infinity gets a NaN scale, so every output it
// touches is NaN, as the fp32 form would give.
#pragma once

#include "qd_decode.h"

namespace qd {

// Bytes of one staged superunit (256 activations) of one batch row: 16
// chunks of 16 activations, each holding the four digit planes' 16 bytes,
// then 8 run records.  Within chunk t the plane k bytes sit at 16 ((k +
// t / 4) mod 4): the four lanes of a group (64 activations apart) read each
// plane from different LDS banks.
constexpr int kDigRuns = 1024;           // offset of the run records
constexpr int kDigSU = kDigRuns + 8 * 16;
// Byte offset of plane k's byte for activation p (0..255) of a superunit.
QD_DEV constexpr int dig_at(int p, int k) { return 64 * (p >> 4) + 16 * ((k + (p >> 6)) & 3) + (p & 15); }

// Per-run record: the run's scale 2^-s (fp32: exact, or a subnormal or zero
// for runs whose activations are all below about 2^-119, whose products are
// then far below the absolute part of the output bound) and, for Q4_K, the
// run's sum of X times 2^-s (fp64, exact; 0 for the other formats).
struct RunRec {
    float scale;
    int pad;
    double sxs;
};

QD_DEV uint32_t fbits(float f) { return __builtin_bit_cast(uint32_t, f); }

// Value of the lane given by a DPP control within each group of 8 lanes:
// 0xB1 = quad [1,0,3,2], 0x4E = quad [2,3,0,1], 0x141 = half-row mirror.
template <int CTRL>
QD_DEV int dpp8(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
// Maximum / sum over the 8 lanes of a run (cross-lane moves, no LDS).
QD_DEV uint32_t max8(uint32_t m) {
    m = max(m, (uint32_t)dpp8<0xB1>((int)m));
    m = max(m, (uint32_t)dpp8<0x4E>((int)m));
    return max(m, (uint32_t)dpp8<0x141>((int)m));
}
QD_DEV int sum8(int s) {
    s += dpp8<0xB1>(s);
    s += dpp8<0x4E>(s);
    return s + dpp8<0x141>(s);
}

// Exact 4-way byte dot product, accumulated: acc + sum_j a.byte[j] * b.byte[j]
// (both signed).
QD_DEV int dot4(uint32_t a, uint32_t b, int acc) {
    return __builtin_amdgcn_sdot4((int)a, (int)b, acc, false);
}
// The same with a zero accumulator as one instruction: the three-operand
// form takes the constant 0, where the builtin becomes a move of 0 and the
// accumulating two-operand form (measured: Gemma-3 decode FFN 21.3-21.5 ->
// 20.9-21.1 us, lm_head Q4_K 88.5 -> 87.2 us).  A vector-ALU instruction
// only: no memory access in the asm.
QD_DEV int dot4z(uint32_t a, uint32_t b) {
    int r;
    asm("v_dot4_i32_i8 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

// Digit plane K of four activations: byte K of each Y = X + 0x80808080 (its
// bytes are the balanced digits plus 128, for |X| <= 2^30), minus 128.
template <int K>
QD_DEV uint32_t digit_plane(uint32_t y0, uint32_t y1, uint32_t y2, uint32_t y3) {
    const uint32_t lo = __builtin_amdgcn_perm(y1, y0, 0x0C0C0000u | ((4u + K) << 8) | K);
    const uint32_t hi = __builtin_amdgcn_perm(y3, y2, ((4u + K) << 24) | ((uint32_t)K << 16) | 0x0C0Cu);
    return (lo | hi) ^ 0x80808080u;
}

// Digits of one run of 32 activations held by 8 consecutive lanes (lane & 7
// = the float4 of the run, the 8 lanes of a DPP half-row; all 8 must be
// active): this lane's four plane dwords (byte e of plane k = digit k of
// activation e of v) and the run's scale 2^-s and, with SX, its sum of X
// times 2^-s (exact in fp64; 0 without SX).  A run holding a NaN or an
// infinity gets a NaN scale.
template <bool SX>
QD_DEV void digitize_run(float4 v, uint32_t (&pl)[4], double &scale, double &sxs) {
    // largest |x| of the run, compared as bit patterns (a NaN or an infinity
    // compares above every finite value)
    uint32_t m = max(max(fbits(v.x) & 0x7FFFFFFFu, fbits(v.y) & 0x7FFFFFFFu),
                     max(fbits(v.z) & 0x7FFFFFFFu, fbits(v.w) & 0x7FFFFFFFu));
    m = max8(m);
    const bool bad = m >= 0x7F800000u;
    // m < 2^E with E the frexp exponent of a normal m (subnormal and zero
    // runs take E = -126, their X then fit all the more)
    const int E = (int)(m >> 23) - 126;
    const int s = 30 - E;  // |x 2^s| < 2^30, so |rint| <= 2^30
    const int X0 = (int)rintf(ldexpf(v.x, s)), X1 = (int)rintf(ldexpf(v.y, s));
    const int X2 = (int)rintf(ldexpf(v.z, s)), X3 = (int)rintf(ldexpf(v.w, s));
    const uint32_t y0 = (uint32_t)X0 + 0x80808080u, y1 = (uint32_t)X1 + 0x80808080u;
    const uint32_t y2 = (uint32_t)X2 + 0x80808080u, y3 = (uint32_t)X3 + 0x80808080u;
    pl[0] = digit_plane<0>(y0, y1, y2, y3);
    pl[1] = digit_plane<1>(y0, y1, y2, y3);
    pl[2] = digit_plane<2>(y0, y1, y2, y3);
    pl[3] = digit_plane<3>(y0, y1, y2, y3);
    scale = bad ? __builtin_nan("") : ldexp(1.0, -s);
    sxs = 0.0;
    if constexpr (SX) {
        // the run's sum of X, from its digit sums (each below 2^12 in magnitude)
        const int s0 = sum8(dot4(pl[0], 0x01010101u, 0));
        const int s1 = sum8(dot4(pl[1], 0x01010101u, 0));
        const int s2 = sum8(dot4(pl[2], 0x01010101u, 0));
        const int s3 = sum8(dot4(pl[3], 0x01010101u, 0));
        sxs = fma((double)(s3 * 256 + s2), 65536.0, (double)(s1 * 256 + s0)) * scale;
    }
}

// Stage activations pos..pos+3 (v, already normalised) of a staged
// superunit whose bytes start at `su`.  Called by the 8 consecutive threads
// that hold one run (lane & 7 = the float4 of the run; pos = 32 * run + 4 *
// (lane & 7), the 8 lanes of a DPP half-row); all 8 must be active.  SX: the
// format needs the run sums (Q4_K's min term).
template <bool SX>
QD_DEV void stage_digits(float4 v, uint8_t *su, int pos) {
    uint32_t pl[4];
    double sc, sxs;
    digitize_run<SX>(v, pl, sc, sxs);
#pragma unroll
    for (int k = 0; k < 4; k++) *reinterpret_cast<uint32_t *>(su + dig_at(pos, k)) = pl[k];
    if ((pos & 31) == 0) {
        RunRec rec;
        rec.scale = (float)sc;
        rec.pad = 0;
        rec.sxs = sxs;
        *reinterpret_cast<RunRec *>(su + kDigRuns + 16 * (pos >> 5)) = rec;
    }
}

// Plane sums recombined: (a3 2^8 + a2) 2^16 + (a1 2^8 + a0), exactly in
// fp64 (Q4_K), or rounded once in fp32.
QD_DEV double undigit64(const int (&a)[4]) {
    return fma((double)(a[3] * 256 + a[2]), 65536.0, (double)(a[1] * 256 + a[0]));
}
QD_DEV float undigit32(const int (&a)[4]) {
    return fmaf((float)(a[3] * 256 + a[2]), 65536.f, (float)(a[1] * 256 + a[0]));
}

QD_DEV uint32_t u4c(const uint4 &v, int i) { return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w; }

// ------------------------------------------------ per-superunit steps ---
// One lane's share of a superunit of NR row streams against the staged
// digits of B batch rows, added to y.  xd: the staged superunit of batch
// row 0 (row b at xd + b * xsb); lane c reads the digits of its own
// weights' positions.

// Q4_K: runs 2c (low nibbles, activations 64c..64c+31) and 2c+1 (high
// nibbles, 64c+32..64c+63).
template <int NR, int B>
QD_DEV void q4k_step_dig(const RawQ4K (&r)[NR], const uint8_t *__restrict__ xd, int xsb, int c,
                         const Q4Lane &L, float (&y)[NR][B]) {
    int al[NR][B][4], ah[NR][B][4];
#pragma unroll
    for (int i = 0; i < NR; i++)
#pragma unroll
        for (int b = 0; b < B; b++)
#pragma unroll
            for (int k = 0; k < 4; k++) { al[i][b][k] = 0; ah[i][b][k] = 0; }
#pragma unroll
    for (int half = 0; half < 2; half++) {
        uint4 dl[B][4], dh[B][4];
#pragma unroll
        for (int b = 0; b < B; b++)
#pragma unroll
            for (int k = 0; k < 4; k++) {
                const uint8_t *p = xd + b * xsb + 64 * (4 * c + half) + 16 * ((k + c) & 3);
                dl[b][k] = *reinterpret_cast<const uint4 *>(p);
                dh[b][k] = *reinterpret_cast<const uint4 *>(p + 128);
            }
#pragma unroll
        for (int e = 0; e < 4; e++) {
#pragma unroll
            for (int i = 0; i < NR; i++) {
                const uint32_t v = r[i].q[4 * half + e];
                const uint32_t lo = v & 0x0F0F0F0Fu, hi = (v >> 4) & 0x0F0F0F0Fu;
#pragma unroll
                for (int b = 0; b < B; b++)
#pragma unroll
                    for (int k = 0; k < 4; k++) {
                        const bool first = half == 0 && e == 0;
                        al[i][b][k] = first ? dot4z(lo, u4c(dl[b][k], 0)) : dot4(lo, u4c(dl[b][k], e), al[i][b][k]);
                        ah[i][b][k] = first ? dot4z(hi, u4c(dh[b][k], 0)) : dot4(hi, u4c(dh[b][k], e), ah[i][b][k]);
                    }
            }
        }
    }
#pragma unroll
    for (int i = 0; i < NR; i++) {
        const Q4Scales s = q4k_scales(r[i], L);
        const float A0 = s.d * s.sc0, A1 = s.d * s.sc1;
        const double B0 = -(double)(s.dmin * s.m0), B1 = -(double)(s.dmin * s.m1);
#pragma unroll
        for (int b = 0; b < B; b++) {
            const RunRec rl = *reinterpret_cast<const RunRec *>(xd + b * xsb + kDigRuns + 32 * c);
            const RunRec rh = *reinterpret_cast<const RunRec *>(xd + b * xsb + kDigRuns + 32 * c + 16);
            double t = fma((double)(A0 * rl.scale), undigit64(al[i][b]), B0 * rl.sxs);
            t = fma((double)(A1 * rh.scale), undigit64(ah[i][b]), fma(B1, rh.sxs, t));
            y[i][b] += (float)t;
        }
    }
}

// Q6_K: lane c = 2h + j; group g is run 4h + g, activations 16j.. of it
// (chunk 8h + 2g + j of the superunit).
// The (q - 32) bytes of group g, dword k4, from the re-aligned ql / qh dwords.
template <int G>
QD_DEV uint32_t q6k_group(uint32_t av, uint32_t bv, uint32_t hv) {
    if constexpr (G == 0) return (av & 0x0F0F0F0Fu) | byte_lut(kQ6HiTable, hv & 0x03030303u);
    else if constexpr (G == 1) return (bv & 0x0F0F0F0Fu) | byte_lut(kQ6HiTable, (hv >> 2) & 0x03030303u);
    else if constexpr (G == 2) return ((av >> 4) & 0x0F0F0F0Fu) | byte_lut(kQ6HiTable, (hv >> 4) & 0x03030303u);
    else return ((bv >> 4) & 0x0F0F0F0Fu) | byte_lut(kQ6HiTable, (hv >> 6) & 0x03030303u);
}

template <int G, int NR, int B>
QD_DEV void q6k_group_dig(const uint32_t (&av)[NR][4], const uint32_t (&bv)[NR][4], const uint32_t (&hv)[NR][4],
                          const Q6Scales (&s)[NR], const uint8_t *__restrict__ xd, int xsb, int h, int j,
                          float (&y)[NR][B]) {
    const int chunk = 8 * h + 2 * G + j;
    const int rot = 2 * h + (G >> 1);
    uint4 D[B][4];
#pragma unroll
    for (int b = 0; b < B; b++)
#pragma unroll
        for (int k = 0; k < 4; k++)
            D[b][k] = *reinterpret_cast<const uint4 *>(xd + b * xsb + 64 * chunk + 16 * ((k + rot) & 3));
    int acc[NR][B][4];
#pragma unroll
    for (int i = 0; i < NR; i++)
#pragma unroll
        for (int b = 0; b < B; b++)
#pragma unroll
            for (int k = 0; k < 4; k++) acc[i][b][k] = 0;
#pragma unroll
    for (int k4 = 0; k4 < 4; k4++)
#pragma unroll
        for (int i = 0; i < NR; i++) {
            const uint32_t q = q6k_group<G>(av[i][k4], bv[i][k4], hv[i][k4]);
#pragma unroll
            for (int b = 0; b < B; b++)
#pragma unroll
                for (int k = 0; k < 4; k++)
                    acc[i][b][k] = k4 == 0 ? dot4z(q, u4c(D[b][k], 0)) : dot4(q, u4c(D[b][k], k4), acc[i][b][k]);
        }
#pragma unroll
    for (int b = 0; b < B; b++) {
        const float sc = reinterpret_cast<const RunRec *>(xd + b * xsb + kDigRuns + 16 * (4 * h + G))->scale;
#pragma unroll
        for (int i = 0; i < NR; i++) {
            const float A = s[i].d * s[i].sc[G] * sc;
            y[i][b] = fmaf(A, undigit32(acc[i][b]), y[i][b]);
        }
    }
}

template <int NR, int B, class R>
QD_DEV void q6k_step_dig(const R (&r)[NR], const uint8_t *__restrict__ xd, int xsb, int h, int j,
                         float (&y)[NR][B]) {
    uint32_t av[NR][4], bv[NR][4], hv[NR][4];
    Q6Scales s[NR];
#pragma unroll
    for (int i = 0; i < NR; i++) {
#pragma unroll
        for (int k4 = 0; k4 < 4; k4++) q6k_dwords(r[i], k4, av[i][k4], bv[i][k4], hv[i][k4]);
        s[i] = q6k_scales(r[i], j);
    }
    q6k_group_dig<0, NR, B>(av, bv, hv, s, xd, xsb, h, j, y);
    q6k_group_dig<1, NR, B>(av, bv, hv, s, xd, xsb, h, j, y);
    q6k_group_dig<2, NR, B>(av, bv, hv, s, xd, xsb, h, j, y);
    q6k_group_dig<3, NR, B>(av, bv, hv, s, xd, xsb, h, j, y);
}

// Q8_0: blocks A (run 2c) and B (run 2c+1).
template <int NR, int B>
QD_DEV void q80_step_dig(const RawQ80 (&r)[NR], const uint8_t *__restrict__ xd, int xsb, int c,
                         float (&y)[NR][B]) {
    int aa[NR][B][4], ab[NR][B][4];
#pragma unroll
    for (int i = 0; i < NR; i++)
#pragma unroll
        for (int b = 0; b < B; b++)
#pragma unroll
            for (int k = 0; k < 4; k++) { aa[i][b][k] = 0; ab[i][b][k] = 0; }
#pragma unroll
    for (int half = 0; half < 2; half++) {
        uint4 dl[B][4], dh[B][4];
#pragma unroll
        for (int b = 0; b < B; b++)
#pragma unroll
            for (int k = 0; k < 4; k++) {
                const uint8_t *p = xd + b * xsb + 64 * (4 * c + half) + 16 * ((k + c) & 3);
                dl[b][k] = *reinterpret_cast<const uint4 *>(p);
                dh[b][k] = *reinterpret_cast<const uint4 *>(p + 128);
            }
#pragma unroll
        for (int e = 0; e < 4; e++) {
#pragma unroll
            for (int i = 0; i < NR; i++) {
                const uint2 v = q80_qdwords(r[i], 4 * half + e);
#pragma unroll
                for (int b = 0; b < B; b++)
#pragma unroll
                    for (int k = 0; k < 4; k++) {
                        const bool first = half == 0 && e == 0;
                        aa[i][b][k] = first ? dot4z(v.x, u4c(dl[b][k], 0)) : dot4(v.x, u4c(dl[b][k], e), aa[i][b][k]);
                        ab[i][b][k] = first ? dot4z(v.y, u4c(dh[b][k], 0)) : dot4(v.y, u4c(dh[b][k], e), ab[i][b][k]);
                    }
            }
        }
    }
#pragma unroll
    for (int i = 0; i < NR; i++) {
        const float2 d = q80_d(r[i]);
#pragma unroll
        for (int b = 0; b < B; b++) {
            const float sa = reinterpret_cast<const RunRec *>(xd + b * xsb + kDigRuns + 32 * c)->scale;
            const float sb = reinterpret_cast<const RunRec *>(xd + b * xsb + kDigRuns + 32 * c + 16)->scale;
            const float t = fmaf(d.x * sa, undigit32(aa[i][b]), y[i][b]);
            y[i][b] = fmaf(d.y * sb, undigit32(ab[i][b]), t);
        }
    }
}

}  // namespace qd
