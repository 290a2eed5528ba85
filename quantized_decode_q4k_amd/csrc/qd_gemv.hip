// qd_gemv.hip -- batch-1..8 GEMV and fused FFN gate+up over Q4_K, Q6_K and
// Q8_0 weights, dequantised in registers and fused into fp32 FMAs.
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
//    workgroup in LDS with a 16-byte skew every 64 floats, so the four lanes
//    of a group, which read the same offsets 64 floats apart, hit different
//    banks.  Q4_K also stages per-32 sums of x for its min term.
//  * Decoding: Q4_K nibbles become floats through the fp8 converter (two
//    per instruction, exact); Q6_K quants become signed (q - 32) bytes with a
//    byte-permute lookup of the high bits, then one sign-extending convert;
//    Q8_0 bytes take one sign-extending convert.  Scales are applied once per
//    16 or 32 weights.
//  * Per-lane partials are reduced across the 4*p_in lanes of a row with
//    cross-lane shuffles; one lane writes each output (and, for the fused
//    FFN, applies the GELU-tanh or SiLU product).
#include "qd_decode.h"

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
// LDS); sp: the staged sums of x over sub-blocks 2c and 2c+1.  Accumulates,
// per row stream and batch row,
//   yq += d * (sc0 * sum(q x) over the low nibbles + sc1 * sum(q x) high)
//         (in units of fp8_unit())
//   ym += dmin * (m0 * X0 + m1 * X1)
// so that the row result is yq / fp8_unit() - ym.
template <int NR, int B>
QD_DEV void q4k_step(const RawQ4K (&r)[NR], const float *__restrict__ xp, int xstride,
                     const float *__restrict__ sp, int sstride, const Q4Lane &L,
                     float (&yq)[NR][B], float (&ym)[NR][B]) {
    float alo[NR][B], ahi[NR][B];
#pragma unroll
    for (int i = 0; i < NR; i++)
#pragma unroll
        for (int b = 0; b < B; b++) { alo[i][b] = 0.f; ahi[i][b] = 0.f; }

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
#pragma unroll
            for (int b = 0; b < B; b++) {
                float s = alo[i][b];
                s = fmaf(n.lo01.x, xl[b].x, s);
                s = fmaf(n.lo01.y, xl[b].y, s);
                s = fmaf(n.lo23.x, xl[b].z, s);
                s = fmaf(n.lo23.y, xl[b].w, s);
                alo[i][b] = s;
                float u = ahi[i][b];
                u = fmaf(n.hi01.x, xh[b].x, u);
                u = fmaf(n.hi01.y, xh[b].y, u);
                u = fmaf(n.hi23.x, xh[b].z, u);
                u = fmaf(n.hi23.y, xh[b].w, u);
                ahi[i][b] = u;
            }
        }
    }

#pragma unroll
    for (int i = 0; i < NR; i++) {
        const Q4Scales s = q4k_scales(r[i], L);
#pragma unroll
        for (int b = 0; b < B; b++) {
            const float2 X = *reinterpret_cast<const float2 *>(sp + b * sstride);
            yq[i][b] = fmaf(s.d, fmaf(s.sc1, ahi[i][b], s.sc0 * alo[i][b]), yq[i][b]);
            ym[i][b] = fmaf(s.dmin, fmaf(s.m1, X.y, s.m0 * X.x), ym[i][b]);
        }
    }
}

// Q6_K.  xg0..xg3: this lane's four runs of 16 activations (groups g).
template <int NR, int B>
QD_DEV void q6k_step(const RawQ6K (&r)[NR], const float *__restrict__ xg0,
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

// Where a tile's activations come from and where its outputs go.
enum : int {
    kPlain = 0,     // ordinary loads / stores
    kCoherent = 1,  // device-scope loads / stores: data produced or consumed by
                    // other workgroups of the same launch (fused FFN)
};

template <int YM>
QD_DEV void store_out(float *p, float v) {
    if constexpr (YM == kCoherent) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else *p = v;
}

// Bounded wait of thread 0 until *ctr >= target (device-scope loads).  The
// bound is a safety net: the producers of every counter waited on here are
// already running when the wait starts, so it ends long before the bound.
QD_DEV void wait_counter(const unsigned *ctr, unsigned target) {
    for (int it = 0; it < (1 << 20); it++) {
        if (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= target) return;
        __builtin_amdgcn_s_sleep(4);
    }
}

// One workgroup tile: rows [bx * rows_per_wg, ...) over K-slice ks of
// p_out.  FMT: block format; B: batch rows (1..8); NR: row streams per lane
// group (FFN: 2 = gate, up); FFN: fused gate/up/activation epilogue.
// XM / YM: kPlain or kCoherent activation loads / output stores.  If
// wait_ctr is set, thread 0 waits for *wait_ctr >= wait_target after the
// first weight loads are issued and before x is staged.
// Wait hook of a tile that consumes data produced in the same launch: wait
// until *ready >= target; then count this workgroup in *arrived, and the
// last of `readers` workgroups resets both counters for the next launch.
struct WaitSpec {
    unsigned *ready = nullptr;
    unsigned target = 0;
    unsigned *arrived = nullptr;
    unsigned readers = 0;
};

template <int FMT, int B, int NR, bool FFN, int XM, int YM>
QD_DEV void mv_tile(const MvArgs &a, const int bx, const int ks, const int p_out, float *smem,
                    const WaitSpec ws = WaitSpec()) {
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
    float *xl = smem;                                 // [B][nk * 272]
    float *xsum = smem + B * xstride;                 // Q4_K: [B][nk * 8]
    const int sstride = a.nk * 8;
    float *red = xsum + (FMT == kQ4K ? B * sstride : 0);  // [4 waves][B], then [B]

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
    const bool early = (XM == kPlain) && (B * F <= kXr * kThreads);
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

    if (ws.ready != nullptr) {
        if (tid == 0) {
            wait_counter(ws.ready, ws.target);
            const unsigned n = __hip_atomic_fetch_add(ws.arrived, 1u, __ATOMIC_RELAXED,
                                                      __HIP_MEMORY_SCOPE_AGENT);
            if (n == ws.readers - 1) {  // every reader has seen the count
                __hip_atomic_store(ws.ready, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(ws.arrived, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        __syncthreads();
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
    if constexpr (XM == kCoherent) {
        // x was written by other workgroups of this launch: device-scope
        // dword loads, consecutive lanes on consecutive dwords (coalesced)
        for (int e = tid; e < B * 4 * F; e += kThreads) {
            const int b = e / (4 * F);
            const int kk = e - b * 4 * F;
            const int64_t k = k0 + kk;
            float v = 0.f;
            if (k < K) v = __hip_atomic_load(a.x + (int64_t)b * K + k, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
            xl[b * xstride + xphys(kk)] = v;
        }
        if constexpr (FMT == kQ4K) {
            __syncthreads();
            for (int e = tid; e < B * 8 * a.nk; e += kThreads) {
                const int b = e / (8 * a.nk);
                const int j = e - b * 8 * a.nk;  // 32-run index
                const float *q = xl + b * xstride + xphys(32 * j);
                float sacc = 0.f;
#pragma unroll
                for (int m = 0; m < 8; m++) {
                    const float4 w4 = *reinterpret_cast<const float4 *>(q + 4 * m);
                    sacc += (w4.x + w4.y) + (w4.z + w4.w);
                }
                xsum[b * sstride + j] = sacc;
            }
        }
    } else {
        // normalise (if asked) and store one float4 of x; for Q4_K also the
        // sum of each 32-run (8 consecutive float4 sit in 8 consecutive
        // lanes of one wave, and every lane of a wave takes part)
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
            *reinterpret_cast<float4 *>(xl + b * xstride + xphys(4 * f4)) = v;
            if constexpr (FMT == kQ4K) {
                float sm = (v.x + v.y) + (v.z + v.w);
                sm += __shfl_xor(sm, 1);
                sm += __shfl_xor(sm, 2);
                sm += __shfl_xor(sm, 4);
                if ((tid & 7) == 0) xsum[b * sstride + (f4 >> 3)] = sm;
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
    float acc[NR][B], acc2[NR][B];
#pragma unroll
    for (int i = 0; i < NR; i++)
#pragma unroll
        for (int b = 0; b < B; b++) { acc[i][b] = 0.f; acc2[i][b] = 0.f; }

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
                if constexpr (FMT == kQ4K) v[i][b] = fmaf(acc[i][b], fp8_inv_unit(), -acc2[i][b]);
                else v[i][b] = acc[i][b];
                acc[i][b] = 0.f;
                acc2[i][b] = 0.f;
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
                        store_out<YM>(a.y + (int64_t)b * N + row[0], act_apply(a.act, gv) * uv);
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
                            store_out<YM>(a.y + o, a.res ? vv + a.res[o] : vv);
                        }
            }
        } else {
            // partials are written with device-scope stores (write-through,
            // no cache-wide writeback needed before the counter below)
#pragma unroll
            for (int i = 0; i < NR; i++)
                if (row[i] < N)
#pragma unroll
                    for (int b = 0; b < B; b++)
                        __hip_atomic_store(
                            a.partials + (((int64_t)ks * B + b) * NP + (FFN ? i : 0)) * N + row[i],
                            v[i][b], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
            if constexpr (FMT == kQ4K) {
                const float *xp = xl + xphys(kSuper * tlo + 64 * c);
                const float *sp = xsum + 8 * tlo + 2 * c;
                q4k_step<NR, B>(buf[s], xp, xstride, sp, sstride, L4, acc, acc2);
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
    if (p_out == 1) return;

    // ---- split-K: the last workgroup of this row tile sums the partials in
    // slice order.  Each wave waits until its partial stores have completed,
    // the workgroup synchronises, and only then bumps the tile's counter with
    // a device-scope atomic.
    __atomic_signal_fence(__ATOMIC_SEQ_CST);  // keep the stores above the wait
    __builtin_amdgcn_s_waitcnt(0);            // this wave's stores are complete
    __syncthreads();
    __shared__ int s_last;
    if (tid == 0) {
        unsigned prev = __hip_atomic_fetch_add(a.counters + bx, 1u, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
        s_last = (prev == (unsigned)p_out - 1) ? 1 : 0;
    }
    __syncthreads();
    if (!s_last) return;
    const int rows_here = (FFN ? RS : RS * NR) * rpg;
    const int64_t tile0 = (int64_t)bx * rows_here;
    for (int e = tid; e < rows_here * B; e += kThreads) {
        const int b = e / rows_here;
        const int64_t r = tile0 + (e - b * rows_here);
        if (r >= N) continue;
        float s0 = 0.f, s1 = 0.f;
        for (int k = 0; k < p_out; k++) {
            const float *p = a.partials + (((int64_t)k * B + b) * NP) * N + r;
            const float pv = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            s0 = a.coef ? fmaf(a.coef[k], pv, s0) : s0 + pv;
            if constexpr (FFN) s1 += __hip_atomic_load(p + N, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        if constexpr (FFN) {
            store_out<YM>(a.y + (int64_t)b * N + r, act_apply(a.act, s0) * s1);
            if (a.g_out) a.g_out[(int64_t)b * N + r] = s0;
            if (a.u_out) a.u_out[(int64_t)b * N + r] = s1;
        } else {
            const int64_t o = (int64_t)b * N + r;
            store_out<YM>(a.y + o, a.res ? s0 + a.res[o] : s0);
        }
    }
    if (tid == 0)  // ready for the next call
        __hip_atomic_store(a.counters + bx, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int FMT, int B, int NR, bool FFN>
__global__ __launch_bounds__(kThreads) void mv_kernel(MvArgs a) {
    extern __shared__ __attribute__((aligned(16))) float smem[];
    mv_tile<FMT, B, NR, FFN, kPlain, kPlain>(a, blockIdx.x, blockIdx.y, gridDim.y, smem);
}

// ------------------------------------------------------ fused decode FFN ---
// One launch for y = Wd (act(Wg xn) * (Wu xn)).  Workgroups [0, nA) are
// gate/up row tiles (phase A): they publish their slice of h with
// device-scope stores and count themselves done in the h-slice they belong
// to.  The remaining workgroups are down-projection tiles (phase B), ordered
// slice by slice: each issues its first weight loads, waits until every
// phase-A tile of its h-slice is done, stages that slice of h with
// device-scope loads and runs as a split-K GEMV tile.  Workgroups are
// dispatched in index order on each XCD, so every phase-A workgroup is
// resident or finished before a phase-B workgroup can hold a slot on the
// same XCD: a waiting workgroup only waits on work that is already running
// (and the wait is bounded).  Counters live on separate 128-byte lines; the
// last phase-B reader of a slice resets them for the next launch.
constexpr int kCtlStride = 32;  // unsigned per counter (one 128-byte line)

template <int FA, int FB, int B>
__global__ __launch_bounds__(kThreads) void ffn_kernel(FfnArgs f) {
    extern __shared__ __attribute__((aligned(16))) float smem[];
    const int t = (int)blockIdx.x;
    if (t < f.nA) {
        mv_tile<FA, B, 2, true, kPlain, kCoherent>(f.a, t, 0, 1, smem);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);  // keep the h stores above the wait
        __builtin_amdgcn_s_waitcnt(0);            // this wave's h stores are complete
        __syncthreads();
        if (threadIdx.x == 0) {
            const int slice = (t * f.rowsA) / f.sliceRows;
            __hip_atomic_fetch_add(f.ctl + (2 * slice) * kCtlStride, 1u, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
    } else {
        const int j = t - f.nA;
        const int ks = j / f.nBx;
        const int bx = j - ks * f.nBx;
        const int per = f.sliceRows / f.rowsA;  // phase-A tiles per h-slice
        WaitSpec ws;
        ws.ready = f.ctl + (2 * ks) * kCtlStride;
        ws.target = (unsigned)(min(f.nA, (ks + 1) * per) - ks * per);
        ws.arrived = f.ctl + (2 * ks + 1) * kCtlStride;
        ws.readers = (unsigned)f.nBx;
        mv_tile<FB, B, 1, false, kCoherent, kPlain>(f.b, bx, ks, f.pB, smem, ws);
    }
}

// ------------------------------------------- mixture-of-experts decode ---
// The larql MoE rows (Gemma 4 26B-A4B and the other expert models) run the
// FFN of each routed expert: gate/up with the activation, then down, with
// the experts' outputs summed with their routing weights.  The expert ids
// and weights stay on the device (no host round trip): slot z of the launch
// reads ids[z] and offsets the weight pointers by that expert's matrix.
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
        mv_tile<FMT, 1, 2, true, kPlain, kPlain>(b, blockIdx.x, 0, 1, smem);
    } else {
        b.x = a.x + (int64_t)slot * a.x_sstride;
        mv_tile<FMT, 1, 1, false, kPlain, kPlain>(b, blockIdx.x, slot, gridDim.y, smem);
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
// Q6_K).  Here the three projections share one launch: workgroup t belongs
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
    case kQ4K: mv_tile<kQ4K, B, 1, false, kPlain, kPlain>(a, t, 0, 1, smem); break;
    case kQ6K: mv_tile<kQ6K, B, 1, false, kPlain, kPlain>(a, t, 0, 1, smem); break;
    default: mv_tile<kQ80, B, 1, false, kPlain, kPlain>(a, t, 0, 1, smem); break;
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
    size_t floats = (size_t)batch * nk * kSuperPhys;
    if (fmt == kQ4K) floats += (size_t)batch * nk * 8;
    floats += 4 * 8;  // cross-wave scratch: [4 waves][batch]
    return floats * sizeof(float);
}

template <int FMT, int B, int NR, bool FFN>
static hipError_t launch_one(const MvArgs &a, dim3 grid, hipStream_t st) {
    size_t lds = mv_lds_bytes(FMT, B, a.nk);
    hipLaunchKernelGGL((mv_kernel<FMT, B, NR, FFN>), grid, dim3(kThreads), lds, st, a);
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

template <int FA, int FB>
static hipError_t launch_ffn_f(const FfnArgs &f, int batch, size_t lds, unsigned grid,
                               hipStream_t st) {
#define QD_FFN(Bv)                                                                       \
    case Bv:                                                                             \
        hipLaunchKernelGGL((ffn_kernel<FA, FB, Bv>), dim3(grid), dim3(kThreads), lds, st, f); \
        break;
    switch (batch) {
        QD_FFN(1) QD_FFN(2) QD_FFN(3) QD_FFN(4) QD_FFN(5) QD_FFN(6) QD_FFN(7) QD_FFN(8)
    default: return hipErrorInvalidValue;
    }
#undef QD_FFN
    return hipGetLastError();
}

bool ffn_fused_supported(int fmt_a, int fmt_b) {
    return (fmt_a == kQ4K && (fmt_b == kQ6K || fmt_b == kQ4K)) || (fmt_a == kQ80 && fmt_b == kQ80);
}

hipError_t launch_ffn(int fmt_a, int fmt_b, int batch, FfnArgs f, hipStream_t st) {
    f.a.p_out = 1;
    const size_t lds = std::max(mv_lds_bytes(fmt_a, batch, f.a.nk), mv_lds_bytes(fmt_b, batch, f.b.nk));
    const unsigned grid = (unsigned)(f.nA + f.nBx * f.pB);
    if ((size_t)f.pB * 2 * kCtlStride > (size_t)kFfnCtlWords) return hipErrorInvalidValue;
    if (fmt_a == kQ4K && fmt_b == kQ6K) return launch_ffn_f<kQ4K, kQ6K>(f, batch, lds, grid, st);
    if (fmt_a == kQ4K && fmt_b == kQ4K) return launch_ffn_f<kQ4K, kQ4K>(f, batch, lds, grid, st);
    if (fmt_a == kQ80 && fmt_b == kQ80) return launch_ffn_f<kQ80, kQ80>(f, batch, lds, grid, st);
    return hipErrorInvalidValue;
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
