// qd_gemv.hip -- batch-1..8 GEMV and fused FFN gate+up over Q4_K, Q6_K and
// Q8_0 weights, decoded in registers: exact integer dot products against
// activation digits at batch 1-2 (qd_digits.h), fp32 FMAs on weights
// dequantised one at a time at batch 3-8.
//
// What is computed: y[b][n] = sum_k w[n][k] x[b][k] for the decode-path
// projections of the larql "Architecture -> Metal shader map" page (Gemma 3
// table: q4k_matvec, q4k_matvec_8sg, q6k_matvec; q4k_ffn_gate_up_8sg + geglu)
// and dotLLM PR #320's matmul_q8_0.  The Metal/Vulkan kernel shapes those
// pages name (8 or 4 SIMD-groups per threadgroup, one row per threadgroup)
// are not followed; the CDNA4 mapping is:
//
//  * A workgroup is 256 threads = 64 lane groups of 4 lanes.  A lane group
//    owns one row (two for the fused gate/up, or for GEMV with nr = 2) and
//    walks that row's superunits (256 weights: one Q4_K/Q6_K block or eight
//    Q8_0 blocks).  Each lane takes 64 weights of the superunit, so the four
//    lanes read the block bytes with 16-byte (Q4_K) or 4-byte-aligned dword
//    (Q6_K, Q8_0: their 210- and 34-byte blocks start on 2-byte boundaries)
//    loads and the row stream is read exactly once.
//  * K is split p_in ways inside a workgroup (adjacent lane groups take
//    interleaved superunits of the same row, so they read neighbouring
//    blocks together) and p_out ways across workgroups (gridDim.y).  The
//    split across workgroups ends in a deterministic reduction: partial sums
//    go to a workspace and the last workgroup to finish a row tile sums them
//    in slice order.
//  * x (optionally RMS-normalised on the way in) is staged once per
//    workgroup in LDS: at batch 1-2 as activation digits (qd_digits.h), at
//    batch 3-8 as fp32 with a 16-byte skew every 64 floats; either way the
//    four lanes of a group, which read positions 64 apart, hit different
//    banks.
//  * Decoding at batch 3-8: Q4_K nibbles become floats through the fp8
//    converter (two per instruction, exact) and each weight is formed with
//    one fused multiply-add of its sub-block's scale and min; Q6_K quants
//    become signed (q - 32) bytes with a byte-permute lookup of the high
//    bits, then one sign-extending convert, and Q8_0 bytes take one
//    sign-extending convert, their (exact) scales applied once per 16 or 32
//    weights.  At batch 1-2 the same bytes go into v_dot4_i32_i8 against
//    the digit planes.
//  * Per-lane partials are reduced across the 4*p_in lanes of a row with
//    cross-lane shuffles; one lane writes each output (and, for the fused
//    FFN, applies the GELU-tanh or SiLU product).
#include "qd_decode.h"
#include "qd_digits.h"
#include "qd_epilogue.h"

#include <algorithm>

namespace qd {

// Target of the ring's loads past the end of a K-slice (covers every byte a
// lane reads of superunit 0: 144, 212 or 340 bytes).
__device__ __attribute__((aligned(256))) uint8_t g_zero_block[512];

// LDS index of logical activation index k (16-byte skew every 64 floats).
QD_DEV int xphys(int k) { return k + ((k >> 6) << 2); }
// LDS floats per staged superunit per batch row.
constexpr int kSuperPhys = kSuper + kSuper / 16;  // 272

// ------------------------------------------------------------ per-step math ---
// One superunit of NR row streams against B staged activation rows.

// Q4_K.  xp: this lane's 64 activations (logical 256*tl + 64c, contiguous in
// LDS).  Each weight is formed on its own, w = d*sc*q - dmin*m with one fused
// multiply-add (the nibble arrives as q * fp8_unit(), so d*sc is scaled by
// 1/fp8_unit(); both factors are exact), then multiplied by its activation:
// the rounding error is that of a plain dot product of the exact weights,
// whatever the scale and min terms cancel to.  The superunit's sum (two
// chains of 32 terms) is added to y.
template <int NR, int B>
QD_DEV void q4k_step(const RawQ4K (&r)[NR], const float *__restrict__ xp, int xstride, const Q4Lane &L,
                     float (&y)[NR][B]) {
    float alo[NR][B], ahi[NR][B];
    float a0[NR], a1[NR], b0[NR], b1[NR];
#pragma unroll
    for (int i = 0; i < NR; i++) {
        const Q4Scales s = q4k_scales(r[i], L);
        a0[i] = (s.d * s.sc0) * fp8_inv_unit();
        a1[i] = (s.d * s.sc1) * fp8_inv_unit();
        b0[i] = -(s.dmin * s.m0);
        b1[i] = -(s.dmin * s.m1);
#pragma unroll
        for (int b = 0; b < B; b++) { alo[i][b] = 0.f; ahi[i][b] = 0.f; }
    }

#pragma unroll
    for (int dw = 0; dw < 8; dw++) {
        float4 xl[B], xh[B];
#pragma unroll
        for (int b = 0; b < B; b++) {
            xl[b] = *reinterpret_cast<const float4 *>(xp + b * xstride + 4 * dw);
            xh[b] = *reinterpret_cast<const float4 *>(xp + b * xstride + 32 + 4 * dw);
        }
#pragma unroll
        for (int i = 0; i < NR; i++) {
            const Q4Nibbles n = q4k_nibbles(r[i].q[dw]);
            const float l0 = fmaf(n.lo01.x, a0[i], b0[i]), l1 = fmaf(n.lo01.y, a0[i], b0[i]);
            const float l2 = fmaf(n.lo23.x, a0[i], b0[i]), l3 = fmaf(n.lo23.y, a0[i], b0[i]);
            const float h0 = fmaf(n.hi01.x, a1[i], b1[i]), h1 = fmaf(n.hi01.y, a1[i], b1[i]);
            const float h2 = fmaf(n.hi23.x, a1[i], b1[i]), h3 = fmaf(n.hi23.y, a1[i], b1[i]);
#pragma unroll
            for (int b = 0; b < B; b++) {
                float s = alo[i][b];
                s = fmaf(l0, xl[b].x, s);
                s = fmaf(l1, xl[b].y, s);
                s = fmaf(l2, xl[b].z, s);
                s = fmaf(l3, xl[b].w, s);
                alo[i][b] = s;
                float u = ahi[i][b];
                u = fmaf(h0, xh[b].x, u);
                u = fmaf(h1, xh[b].y, u);
                u = fmaf(h2, xh[b].z, u);
                u = fmaf(h3, xh[b].w, u);
                ahi[i][b] = u;
            }
        }
    }

#pragma unroll
    for (int i = 0; i < NR; i++)
#pragma unroll
        for (int b = 0; b < B; b++) y[i][b] += alo[i][b] + ahi[i][b];
}

// Q6_K.  xg0..xg3: this lane's four runs of 16 activations (groups g).
template <int NR, int B, class R>
QD_DEV void q6k_step(const R (&r)[NR], const float *__restrict__ xg0,
                     const float *__restrict__ xg1, const float *__restrict__ xg2,
                     const float *__restrict__ xg3, int xstride, int j, float (&y)[NR][B]) {
    float acc[NR][B][4];
#pragma unroll
    for (int i = 0; i < NR; i++)
#pragma unroll
        for (int b = 0; b < B; b++)
#pragma unroll
            for (int g = 0; g < 4; g++) acc[i][b][g] = 0.f;

#pragma unroll
    for (int k = 0; k < 4; k++) {
        float4 xv[B][4];
#pragma unroll
        for (int b = 0; b < B; b++) {
            xv[b][0] = *reinterpret_cast<const float4 *>(xg0 + b * xstride + 4 * k);
            xv[b][1] = *reinterpret_cast<const float4 *>(xg1 + b * xstride + 4 * k);
            xv[b][2] = *reinterpret_cast<const float4 *>(xg2 + b * xstride + 4 * k);
            xv[b][3] = *reinterpret_cast<const float4 *>(xg3 + b * xstride + 4 * k);
        }
#pragma unroll
        for (int i = 0; i < NR; i++) {
            uint32_t q[4];
            q6k_qbytes(r[i], k, q);
#pragma unroll
            for (int g = 0; g < 4; g++) {
                const float w0 = sbyte(q[g], 0), w1 = sbyte(q[g], 1);
                const float w2 = sbyte(q[g], 2), w3 = sbyte(q[g], 3);
#pragma unroll
                for (int b = 0; b < B; b++) {
                    float s = acc[i][b][g];
                    s = fmaf(w0, xv[b][g].x, s);
                    s = fmaf(w1, xv[b][g].y, s);
                    s = fmaf(w2, xv[b][g].z, s);
                    s = fmaf(w3, xv[b][g].w, s);
                    acc[i][b][g] = s;
                }
            }
        }
    }

#pragma unroll
    for (int i = 0; i < NR; i++) {
        const Q6Scales s = q6k_scales(r[i], j);
#pragma unroll
        for (int b = 0; b < B; b++) {
            float u = s.sc[0] * acc[i][b][0];
            u = fmaf(s.sc[1], acc[i][b][1], u);
            u = fmaf(s.sc[2], acc[i][b][2], u);
            u = fmaf(s.sc[3], acc[i][b][3], u);
            y[i][b] = fmaf(s.d, u, y[i][b]);
        }
    }
}

// Q8_0.  xp: this lane's 64 activations (block A then block B).
template <int NR, int B>
QD_DEV void q80_step(const RawQ80 (&r)[NR], const float *__restrict__ xp, int xstride,
                     float (&y)[NR][B]) {
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
                const float4 xa = *reinterpret_cast<const float4 *>(xp + b * xstride + 4 * k);
                const float4 xb = *reinterpret_cast<const float4 *>(xp + b * xstride + 32 + 4 * k);
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
        for (int b = 0; b < B; b++) y[i][b] = fmaf(d.y, accB[b], fmaf(d.x, accA[b], y[i][b]));
    }
}

// ------------------------------------------------------------- the kernel ---
QD_DEV float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

// Superunits of loads kept in flight ahead of the one being multiplied.
template <int FMT, int B, int NR>
constexpr int lookahead() {
#ifdef QD_LOOKAHEAD
    return QD_LOOKAHEAD;
#else
    return (B * NR <= 2) ? 2 : 1;
#endif
}

QD_DEV void store_out(float *p, float v) { *p = v; }

// One workgroup tile: rows [bx * rows_per_wg, ...) over K-slice ks of
// p_out.  FMT: block format; B: batch rows (1..8); NR: row streams per lane
// group (FFN: 2 = gate, up); FFN: fused gate/up/activation epilogue; DIG:
// activation digits and integer dot products (batch 1-2), else fp32.
template <int FMT, int B, int NR, bool FFN, bool DIG>
QD_DEV void mv_tile(const MvArgs &a, const int bx, const int ks, const int p_out, float *smem) {
    const int tid = threadIdx.x;
    const int c = tid & 3;
    const int grp = tid >> 2;
    const int p_in = a.p_in;
    const int rs = grp / p_in;            // row slot in this workgroup
    const int pi = grp - rs * p_in;       // K-interleave index
    const int RS = kGroups / p_in;        // row slots per workgroup
    const int t_beg = a.coef ? 0 : ks * a.nk;  // expert slots each take the whole row
    const int t_end = min(a.nb, t_beg + a.nk);
    const int xstride = a.nk * kSuperPhys;
    // batch 1-2: activation digits (qd_digits.h), nk * kDigSU bytes per
    // batch row; else fp32 activations, nk * 272 floats per batch row
    static_assert(!DIG || B <= 2, "activation digits: batch 1-2");
    const int xsb = a.nk * kDigSU;
    float *xl = smem;                                 // [B][nk * 272] or digits
    float *red = reinterpret_cast<float *>(reinterpret_cast<uint8_t *>(smem) +
                                           (DIG ? (size_t)B * xsb : (size_t)B * xstride * 4));  // [4 waves][B]

    // ---- rows of this lane group: row slots bx * RS * rpg + r * RS + rs for
    // r < rpg (a row slot is one row of each matrix for the fused FFN, NR
    // consecutive rows otherwise); the group walks them one after another
    const int rpg = a.rpg > 1 ? a.rpg : 1;
    const int64_t slot0 = (int64_t)bx * RS * rpg + rs;
    const int64_t rstep = (int64_t)RS * (FFN ? 1 : NR);  // rows between a group's row slots
    int64_t row0[NR];
    const uint8_t *mat[NR];
#pragma unroll
    for (int i = 0; i < NR; i++) {
        row0[i] = FFN ? slot0 : slot0 * NR + i;
        mat[i] = (FFN && i == 1) ? a.W1 : a.W0;
    }

    const int64_t K = a.K;
    const int F = a.nk * (kSuper / 4);   // float4 per batch row in this slice
    const int64_t k0 = (int64_t)t_beg * kSuper;
    const bool norm = a.norm_w != nullptr;

    // ---- small activation slices are loaded into registers (with the norm
    // weight) before any weight load is issued, so they return ahead of the
    // weight stream instead of queueing behind it
    constexpr int kXr = 6;  // float4 per thread held this way
    const bool early = B * F <= kXr * kThreads;
    float4 xr[kXr], wr[kXr];
#pragma unroll
    for (int i = 0; i < kXr; i++) {
        xr[i] = make_float4(0.f, 0.f, 0.f, 0.f);
        wr[i] = make_float4(1.f, 1.f, 1.f, 1.f);
        const int f = tid + kThreads * i;
        if (early && f < B * F) {
            const int b = f / F;
            const int64_t k = k0 + 4 * (f - b * F);
            if (k < K) {
                xr[i] = *reinterpret_cast<const float4 *>(a.x + (int64_t)b * K + k);
                if (norm) wr[i] = *reinterpret_cast<const float4 *>(a.norm_w + k);
            }
        }
    }

    // ---- the first D superunits' loads.  The group's work is Q = rpg * nsu
    // units: unit q is superunit t0 + (q % nsu) * p_in of its row slot q / nsu.
    // Units past the end of the K-slice or of the matrix read a small zero
    // block (which stays in cache) and add nothing.
    using Raw = typename RawOf<FMT>::T;
    constexpr int D = lookahead<FMT, B, NR>();
    Raw buf[D + 1][NR];
    const int t0 = t_beg + pi;
    const int nsu = (a.nk + p_in - 1) / p_in;
    const int Q = rpg * nsu;
    // Q4_K / Q6_K: each lane's block of unit (0, 0) per row stream, once; unit
    // (r, u) lies r * rstep rows and u * p_in blocks further (uniform byte
    // offsets, so no per-lane 64-bit multiply per load).  Q8_0 keeps the
    // block index for its partial-superunit check.
    constexpr int64_t kUB = FMT == kQ4K ? 144 : 210;
    const uint8_t *ub0[NR];
#pragma unroll
    for (int i = 0; i < NR; i++) ub0[i] = mat[i] + row0[i] * a.row_bytes + (int64_t)t0 * kUB;
    const int64_t rstride_b = rstep * a.row_bytes;
    const int64_t ustride_b = (int64_t)p_in * kUB;
    auto load_at = [&](Raw (&dst)[NR], int r, int u, bool inq) {
        const int t = t0 + u * p_in;
#pragma unroll
        for (int i = 0; i < NR; i++) {
            const int64_t rw = row0[i] + r * rstep;
            const bool live = inq && t < t_end && rw < a.N;
            if constexpr (FMT == kQ80) {
                load_unit<FMT>(dst[i], live ? mat[i] + rw * a.row_bytes : g_zero_block, live ? t : 0, c, a.nblk);
            } else {
                const uint8_t *blk = ub0[i] + (r * rstride_b + u * ustride_b);
                load_unit<FMT>(dst[i], live ? blk : g_zero_block, 0, c, a.nblk);
            }
        }
    };
    int rl = 0, ul = 0;  // row slot and unit of the next unit to load
#pragma unroll
    for (int d = 0; d < D; d++) {
        load_at(buf[d], rl, ul, d < Q);
        if (++ul == nsu) { ul = 0; rl++; }
    }

    // ---- inverse RMS of each batch row (RMS-norm fused into staging)
    float inv_rms[B];
#pragma unroll
    for (int b = 0; b < B; b++) inv_rms[b] = 1.0f;
    if (norm) {
        const int wave = tid >> 6;
        float ss[B];
#pragma unroll
        for (int b = 0; b < B; b++) ss[b] = 0.f;
        if (early && t_beg == 0 && t_end == a.nb) {
            // the registers hold all of x
#pragma unroll
            for (int i = 0; i < kXr; i++) {
                const int f = tid + kThreads * i;
                const int bi = f / F;
                float q = fmaf(xr[i].x, xr[i].x, 0.f);
                q = fmaf(xr[i].y, xr[i].y, q);
                q = fmaf(xr[i].z, xr[i].z, q);
                q = fmaf(xr[i].w, xr[i].w, q);
#pragma unroll
                for (int b = 0; b < B; b++)
                    if (b == bi) ss[b] += q;
            }
        } else {
#pragma unroll
            for (int b = 0; b < B; b++) {
                const float *xb = a.x + (int64_t)b * K;
                for (int64_t k = 4 * tid; k < K; k += 4 * kThreads) {
                    float4 v = *reinterpret_cast<const float4 *>(xb + k);
                    ss[b] = fmaf(v.x, v.x, ss[b]);
                    ss[b] = fmaf(v.y, v.y, ss[b]);
                    ss[b] = fmaf(v.z, v.z, ss[b]);
                    ss[b] = fmaf(v.w, v.w, ss[b]);
                }
            }
        }
#pragma unroll
        for (int b = 0; b < B; b++) {
            const float w = wave_sum(ss[b]);
            if ((tid & 63) == 0) red[wave * B + b] = w;
        }
        __syncthreads();
#pragma unroll
        for (int b = 0; b < B; b++) {
            float sq = (red[b] + red[B + b]) + (red[2 * B + b] + red[3 * B + b]);
            inv_rms[b] = 1.0f / sqrtf(sq / (float)K + a.eps);
        }
    }

    // ---- stage x[b][t_beg*256 ...) into LDS (zero past K)
    {
        // normalise (if asked) and store one float4 of x
        auto stage_one = [&](int f, float4 v, float4 w) {
            const int b = f / F;
            const int f4 = f - b * F;
            if (norm) {
                float ir = inv_rms[0];
#pragma unroll
                for (int bb = 1; bb < B; bb++)
                    if (bb == b) ir = inv_rms[bb];
                v.x = v.x * ir * w.x;
                v.y = v.y * ir * w.y;
                v.z = v.z * ir * w.z;
                v.w = v.w * ir * w.w;
            }
            if constexpr (DIG) {
                uint8_t *su = reinterpret_cast<uint8_t *>(xl) + b * xsb + (f4 >> 6) * kDigSU;
                stage_digits<FMT == kQ4K>(v, su, 4 * (f4 & 63));
            } else {
                *reinterpret_cast<float4 *>(xl + b * xstride + xphys(4 * f4)) = v;
            }
        };
        if (early) {
#pragma unroll
            for (int i = 0; i < kXr; i++) {
                const int f = tid + kThreads * i;
                if (f < B * F) stage_one(f, xr[i], wr[i]);  // uniform per wave
            }
        } else {
            for (int f = tid; f < B * F; f += kThreads) {
                const int b = f / F;
                const int64_t k = k0 + 4 * (f - b * F);
                float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
                float4 w = make_float4(1.f, 1.f, 1.f, 1.f);
                if (k < K) {
                    v = *reinterpret_cast<const float4 *>(a.x + (int64_t)b * K + k);
                    if (norm) w = *reinterpret_cast<const float4 *>(a.norm_w + k);
                }
                stage_one(f, v, w);
            }
        }
    }
    __syncthreads();

    // ---- main loop over this group's units
    float acc[NR][B];
#pragma unroll
    for (int i = 0; i < NR; i++)
#pragma unroll
        for (int b = 0; b < B; b++) acc[i][b] = 0.f;

    Q4Lane L4;
    if constexpr (FMT == kQ4K) L4 = q4k_lane(c);
    const bool leader = (pi == 0) && (c == 0);
    const int64_t N = a.N;
    constexpr int NP = FFN ? 2 : 1;  // split-K partial planes per batch row

    // A row slot is complete: combine per lane, reduce over the 4 * p_in
    // lanes of the row, and store the result (or this K-slice's partial).
    auto finish_row = [&](int r) {
        float v[NR][B];
#pragma unroll
        for (int i = 0; i < NR; i++)
#pragma unroll
            for (int b = 0; b < B; b++) {
                v[i][b] = acc[i][b];
                acc[i][b] = 0.f;
            }
        for (int off = 1; off < 4 * p_in; off <<= 1) {
#pragma unroll
            for (int i = 0; i < NR; i++)
#pragma unroll
                for (int b = 0; b < B; b++) v[i][b] += __shfl_xor(v[i][b], off);
        }
        if (!leader) return;
        int64_t row[NR];
#pragma unroll
        for (int i = 0; i < NR; i++) row[i] = row0[i] + r * rstep;
        if (p_out == 1) {
            if constexpr (FFN) {
                if (row[0] < N) {
#pragma unroll
                    for (int b = 0; b < B; b++) {
                        const float gv = v[0][b], uv = v[1][b];
                        store_out(a.y + (int64_t)b * N + row[0], act_apply(a.act, gv) * uv);
                        if (a.g_out) a.g_out[(int64_t)b * N + row[0]] = gv;
                        if (a.u_out) a.u_out[(int64_t)b * N + row[0]] = uv;
                    }
                }
            } else {
#pragma unroll
                for (int i = 0; i < NR; i++)
                    if (row[i] < N)
#pragma unroll
                        for (int b = 0; b < B; b++) {
                            const int64_t o = (int64_t)b * N + row[i];
                            const float vv = a.coef ? a.coef[ks] * v[i][b] : v[i][b];
                            if (a.pn.w1) xstore(a.pn.p + o, vv);  // the row epilogue forms y
                            else store_out(a.y + o, a.res ? vv + a.res[o] : vv);
                        }
            }
        } else {
#pragma unroll
            for (int i = 0; i < NR; i++)
                if (row[i] < N)
#pragma unroll
                    for (int b = 0; b < B; b++)
                        xstore(a.partials + (((int64_t)ks * B + b) * NP + (FFN ? i : 0)) * N + row[i], v[i][b]);
        }
    };

    // Ring of D + 1 load buffers: while unit q is being multiplied, the loads
    // of units q + 1 .. q + D are in flight, across row-slot boundaries.  The
    // inner loop is fully unrolled so every buffer index is a compile-time
    // constant (no register copies, no wait for loads issued in the same
    // iteration).
    int rc = 0, uc = 0;  // row slot and unit being multiplied
    for (int q0 = 0; q0 < Q; q0 += D + 1) {
#pragma unroll
        for (int s = 0; s <= D; s++) {
            const int q = q0 + s;
            if (q >= Q) break;
            // issued on every path so the wait counts are the same on every path
            load_at(buf[(s + D) % (D + 1)], rl, ul, q + D < Q);
            if (++ul == nsu) { ul = 0; rl++; }
            const int tlo = min(t0 + uc * p_in, t_end - 1) - t_beg;  // dead units: zero weights
            if constexpr (DIG) {
                const uint8_t *xd = reinterpret_cast<const uint8_t *>(xl) + tlo * kDigSU;
                if constexpr (FMT == kQ4K) q4k_step_dig<NR, B>(buf[s], xd, xsb, c, L4, acc);
                else if constexpr (FMT == kQ6K) q6k_step_dig<NR, B>(buf[s], xd, xsb, c >> 1, c & 1, acc);
                else q80_step_dig<NR, B>(buf[s], xd, xsb, c, acc);
            } else if constexpr (FMT == kQ4K) {
                const float *xp = xl + xphys(kSuper * tlo + 64 * c);
                q4k_step<NR, B>(buf[s], xp, xstride, L4, acc);
            } else if constexpr (FMT == kQ6K) {
                const int h = c >> 1, j = c & 1;
                const int base = kSuper * tlo + 128 * h + 16 * j;
                q6k_step<NR, B>(buf[s], xl + xphys(base), xl + xphys(base + 32),
                                xl + xphys(base + 64), xl + xphys(base + 96), xstride, j, acc);
            } else {
                q80_step<NR, B>(buf[s], xl + xphys(kSuper * tlo + 64 * c), xstride, acc);
            }
            if (++uc == nsu) {
                finish_row(rc);
                uc = 0;
                rc++;
            }
        }
    }
    __shared__ int s_last;
    if (p_out == 1) {
        if (!FFN && a.pn.w1) post_norm_tail<kThreads>(a.pn, a.y, B, N, red, &s_last);
        return;
    }

    // ---- split-K: the last workgroup of this row tile sums the partials in
    // slice order (the hand-off of qd_epilogue.h on the tile's counter)
    if (!arrive_last<kThreads>(a.counters + bx, (unsigned)p_out, &s_last)) return;
    const int rows_here = (FFN ? RS : RS * NR) * rpg;
    const int64_t tile0 = (int64_t)bx * rows_here;
    for (int e = tid; e < rows_here * B; e += kThreads) {
        const int b = e / rows_here;
        const int64_t r = tile0 + (e - b * rows_here);
        if (r >= N) continue;
        float s0 = 0.f, s1 = 0.f;
        for (int k = 0; k < p_out; k++) {
            const float *p = a.partials + (((int64_t)k * B + b) * NP) * N + r;
            const float pv = xload(p);
            s0 = a.coef ? fmaf(a.coef[k], pv, s0) : s0 + pv;
            if constexpr (FFN) s1 += xload(p + N);
        }
        if constexpr (FFN) {
            store_out(a.y + (int64_t)b * N + r, act_apply(a.act, s0) * s1);
            if (a.g_out) a.g_out[(int64_t)b * N + r] = s0;
            if (a.u_out) a.u_out[(int64_t)b * N + r] = s1;
        } else {
            const int64_t o = (int64_t)b * N + r;
            if (a.pn.w1) xstore(a.pn.p + o, s0);
            else store_out(a.y + o, a.res ? s0 + a.res[o] : s0);
        }
    }
    if (tid == 0)  // ready for the next call
        __hip_atomic_store(a.counters + bx, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (!FFN && a.pn.w1) post_norm_tail<kThreads>(a.pn, a.y, B, N, red, &s_last);
}

template <int FMT, int B, int NR, bool FFN, bool DIG>
__global__ __launch_bounds__(kThreads) void mv_kernel(MvArgs a) {
    extern __shared__ __attribute__((aligned(16))) float smem[];
    mv_tile<FMT, B, NR, FFN, DIG>(a, blockIdx.x, blockIdx.y, gridDim.y, smem);
}

// ------------------------------------------- mixture-of-experts decode ---
// The larql MoE rows (Gemma 4 26B-A4B and the other expert models) run the
// FFN of each routed expert: gate/up with the activation, then down, with
// the experts' outputs summed with their routing weights.  The expert ids
// and weights stay on the device (no host round trip): slot z of the launch
// reads ids[z] and offsets the weight pointers by that expert's matrix.
// This register-kernel form runs rows that are not whole superunits and
// forced launch shapes; the streaming kernel runs the rest.
//  * gate/up (FFN = true, grid (tiles, 1, n_sel)): slot z = blockIdx.z
//    writes its h rows at y + z * y_sstride; an id outside [0, n_experts)
//    writes zeros (the slot contributes nothing);
//  * down (FFN = false, grid (tiles, n_sel)): slot z = blockIdx.y reads
//    h_z over the whole row as split-K slice z, and the last workgroup of a
//    row tile sums coef[z] * partial_z in slot order (deterministic).  An
//    invalid id reads expert 0's weights against its zero h.
template <int FMT, bool FFN>
__global__ __launch_bounds__(kThreads) void moe_kernel(MvArgs a) {
    extern __shared__ __attribute__((aligned(16))) float smem[];
    const int slot = FFN ? (int)blockIdx.z : (int)blockIdx.y;
    int e = a.ids[slot];
    const bool valid = e >= 0 && e < a.n_experts;
    e = valid ? e : 0;
    MvArgs b = a;
    b.W0 = a.W0 + (int64_t)e * a.w_estride;
    if constexpr (FFN) {
        b.W1 = a.W1 + (int64_t)e * a.w_estride;
        b.y = a.y + (int64_t)slot * a.y_sstride;
        if (!valid) {
            const int rows = kGroups / a.p_in;
            const int64_t r0 = (int64_t)blockIdx.x * rows;
            for (int r = threadIdx.x; r < rows; r += kThreads)
                if (r0 + r < a.N) b.y[r0 + r] = 0.f;
            return;
        }
        mv_tile<FMT, 1, 2, true, false>(b, blockIdx.x, 0, 1, smem);
    } else {
        b.x = a.x + (int64_t)slot * a.x_sstride;
        mv_tile<FMT, 1, 1, false, false>(b, blockIdx.x, slot, gridDim.y, smem);
    }
}

template <int FMT>
static hipError_t launch_moe_f(bool ffn, const MvArgs &a, int64_t tiles, int n_sel, hipStream_t st) {
    const size_t lds = mv_lds_bytes(FMT, 1, a.nk);
    if (ffn)
        hipLaunchKernelGGL((moe_kernel<FMT, true>), dim3((unsigned)tiles, 1, (unsigned)n_sel), dim3(kThreads), lds,
                           st, a);
    else
        hipLaunchKernelGGL((moe_kernel<FMT, false>), dim3((unsigned)tiles, (unsigned)n_sel), dim3(kThreads), lds,
                           st, a);
    return hipGetLastError();
}

hipError_t launch_moe(int fmt, bool ffn, const MvArgs &a, int64_t tiles, int n_sel, hipStream_t st) {
    switch (fmt) {
    case kQ4K: return launch_moe_f<kQ4K>(ffn, a, tiles, n_sel, st);
    case kQ6K: return launch_moe_f<kQ6K>(ffn, a, tiles, n_sel, st);
    case kQ80: return launch_moe_f<kQ80>(ffn, a, tiles, n_sel, st);
    default: return hipErrorInvalidValue;
    }
}

// ------------------------------------------------ fused Q/K/V projection ---
// The larql Gemma 3 table runs the input RMS-norm and the Q, K and V
// projections of attention as one fused dispatch (Q and K in Q4_K, V in
// Q6_K).  This register-kernel form serves batch 2-8 (and rows that are not
// whole superunits, and forced launch shapes; batch 1 runs on the streaming
// kernel).  The three projections share one launch: workgroup t belongs
// to matrix 0, 1 or 2 by its index, and runs that matrix's row tile in that
// matrix's format.  Every tile stages (and RMS-normalises) the activation
// rows itself, so the tiles are independent and the launch needs no
// workspace.
template <int B>
__global__ __launch_bounds__(kThreads) void qkv_kernel(QkvArgs q) {
    extern __shared__ __attribute__((aligned(16))) float smem[];
    int t = (int)blockIdx.x;
    int s = 0;
    if (t >= q.tiles[0]) {
        t -= q.tiles[0];
        s = 1;
        if (t >= q.tiles[1]) {
            t -= q.tiles[1];
            s = 2;
        }
    }
    const MvArgs &a = q.a[s];
    switch (q.fmt[s]) {
    case kQ4K: mv_tile<kQ4K, B, 1, false, false>(a, t, 0, 1, smem); break;
    case kQ6K: mv_tile<kQ6K, B, 1, false, false>(a, t, 0, 1, smem); break;
    default: mv_tile<kQ80, B, 1, false, false>(a, t, 0, 1, smem); break;
    }
}

hipError_t launch_qkv(const QkvArgs &q, int batch, size_t lds, hipStream_t st) {
    const unsigned grid = (unsigned)(q.tiles[0] + q.tiles[1] + q.tiles[2]);
#define QD_QKV(Bv)                                                                       \
    case Bv:                                                                             \
        hipLaunchKernelGGL((qkv_kernel<Bv>), dim3(grid), dim3(kThreads), lds, st, q);    \
        break;
    switch (batch) {
        QD_QKV(1) QD_QKV(2) QD_QKV(3) QD_QKV(4) QD_QKV(5) QD_QKV(6) QD_QKV(7) QD_QKV(8)
    default: return hipErrorInvalidValue;
    }
#undef QD_QKV
    return hipGetLastError();
}

// ------------------------------------------------------------ launchers ---
size_t mv_lds_bytes(int fmt, int batch, int nk) {
    // staged activations: digits at batch 1-2, fp32 beyond
    const size_t x = batch <= 2 ? (size_t)batch * nk * kDigSU : (size_t)batch * nk * kSuperPhys * sizeof(float);
    return x + 4 * 8 * sizeof(float);  // cross-wave scratch: [4 waves][batch]
}

// Activation digits for the batch-1..2 register GEMVs of tall matrices,
// where the decode's VALU work matters (lm_head 262144 x 2560 Q4_K, graph
// replay: 86 -> 78 us); the smaller, latency-bound shapes (and the Q/K/V
// and MoE launches) stage fp32, whose staging is shorter (Gemma-3 Q/K/V in
// one launch: 8.1 us on digits, 7.6 on fp32).
constexpr int64_t kDigMinRows = 16384;

template <int FMT, int B, int NR, bool FFN>
static hipError_t launch_one(const MvArgs &a, dim3 grid, hipStream_t st) {
    size_t lds = mv_lds_bytes(FMT, B, a.nk);
    if constexpr (B <= 2) {
        if (a.N >= kDigMinRows) {
            hipLaunchKernelGGL((mv_kernel<FMT, B, NR, FFN, true>), grid, dim3(kThreads), lds, st, a);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((mv_kernel<FMT, B, NR, FFN, false>), grid, dim3(kThreads), lds, st, a);
    return hipGetLastError();
}

template <int FMT, int B>
static hipError_t launch_fb(const MvArgs &a, bool ffn, int nr, dim3 grid, hipStream_t st) {
    if (ffn) return launch_one<FMT, B, 2, true>(a, grid, st);
    if (nr == 2) return launch_one<FMT, B, 2, false>(a, grid, st);
    return launch_one<FMT, B, 1, false>(a, grid, st);
}

template <int FMT>
static hipError_t launch_f(const MvArgs &a, int batch, bool ffn, int nr, dim3 grid, hipStream_t st) {
    switch (batch) {
    case 1: return launch_fb<FMT, 1>(a, ffn, nr, grid, st);
    case 2: return launch_fb<FMT, 2>(a, ffn, nr, grid, st);
    case 3: return launch_fb<FMT, 3>(a, ffn, nr, grid, st);
    case 4: return launch_fb<FMT, 4>(a, ffn, nr, grid, st);
    case 5: return launch_fb<FMT, 5>(a, ffn, nr, grid, st);
    case 6: return launch_fb<FMT, 6>(a, ffn, nr, grid, st);
    case 7: return launch_fb<FMT, 7>(a, ffn, nr, grid, st);
    case 8: return launch_fb<FMT, 8>(a, ffn, nr, grid, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_gemv(int fmt, int batch, bool ffn, MvArgs a, Shape s, hipStream_t st) {
    a.p_in = s.p_in;
    a.p_out = s.p_out;
    a.rpg = s.rpg;
    const int nr = ffn ? 2 : s.nr;
    const int rows_per_wg = (kGroups / s.p_in) * (ffn ? 1 : nr) * std::max(1, s.rpg);
    const int64_t tiles = (a.N + rows_per_wg - 1) / rows_per_wg;
    dim3 grid((unsigned)tiles, (unsigned)s.p_out);
    switch (fmt) {
    case kQ4K: return launch_f<kQ4K>(a, batch, ffn, nr, grid, st);
    case kQ6K: return launch_f<kQ6K>(a, batch, ffn, nr, grid, st);
    case kQ80: return launch_f<kQ80>(a, batch, ffn, nr, grid, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace qd
