// qd_decode.h -- in-register block decoders shared by the GEMV, FFN,
// dequantise and prefill kernels.
//
// Every format is processed in superunits of 256 weights (one Q4_K or Q6_K
// block, or eight Q8_0 blocks).  Four lanes share a superunit and each lane
// owns 64 of its weights; the functions below load one lane's bytes and
// decode them.  Bit placement follows the GGUF k-quant layout named on the
// larql "Architecture -> Metal shader map" page (144-byte GGUF-direct Q4_K)
// and the 34-byte Q8_0 block of dotLLM PR #320.
#pragma once

#include "qd_device.h"
#include "qd_internal.h"

namespace qd {

// ------------------------------------------------------------------ Q4_K ---
// Block: [0,2) d, [2,4) dmin, [4,16) s[0..11] (packed 6-bit scales and mins),
// [16,144) quants.  Quant run c (32 bytes) holds weights 64c..64c+31 in its
// low nibbles and 64c+32..64c+63 in its high nibbles.  Lane c takes run c:
// sub-block 2c (low nibbles, weights 64c + l) and 2c+1 (high nibbles,
// weights 64c + 32 + l), l = 0..31.
struct RawQ4K {
    uint32_t h[4];  // d|dmin, s[0..3], s[4..7], s[8..11]
    uint32_t q[8];  // quant run c
};

// Per-lane constants of the scale/min gather.
struct Q4Lane {
    uint32_t selT, selU;
    uint32_t mA, mB, mC, mD;
};

QD_DEV Q4Lane q4k_lane(int c) {
    Q4Lane L;
    const uint32_t j0 = (uint32_t)(c & 1) * 2u, j1 = j0 + 1u;  // (2c) & 3, (2c+1) & 3
    // T = [s[j0], s[j1], s[4+j0], s[4+j1]]: perm(h2, h1) takes selectors 0..3
    // from h1 = s[0..3] and 4..7 from h2 = s[4..7].
    L.selT = j0 | (j1 << 8) | ((4u + j0) << 16) | ((4u + j1) << 24);
    // U = [s[8+j0], s[8+j1], s[8+j0], s[8+j1]]
    L.selU = j0 | (j1 << 8) | (j0 << 16) | (j1 << 24);
    if (c < 2) {
        // sub-block j < 4: scale = low 6 bits of s[j], min = low 6 bits of s[j+4]
        L.mA = 0x3F3F3F3Fu; L.mB = 0u; L.mC = 0u; L.mD = 0u;
    } else {
        // sub-block j >= 4: scale = low nibble of s[j+4] | top 2 bits of s[j-4] << 4,
        //                   min   = high nibble of s[j+4] | top 2 bits of s[j] << 4
        L.mA = 0u; L.mB = 0x30303030u; L.mC = 0x00000F0Fu; L.mD = 0x0F0F0000u;
    }
    return L;
}

QD_DEV void load_q4k(RawQ4K &r, const uint8_t *blk, int c) {
    const uint4 h = ld128(blk);
    const uint4 a = ld128(blk + 16 + 32 * c);
    const uint4 b = ld128(blk + 32 + 32 * c);
    r.h[0] = h.x; r.h[1] = h.y; r.h[2] = h.z; r.h[3] = h.w;
    r.q[0] = a.x; r.q[1] = a.y; r.q[2] = a.z; r.q[3] = a.w;
    r.q[4] = b.x; r.q[5] = b.y; r.q[6] = b.z; r.q[7] = b.w;
}

// Scales and mins of this lane's two sub-blocks, as exact floats, and the
// block's d and dmin.
struct Q4Scales {
    float sc0, sc1, m0, m1, d, dmin;
};

QD_DEV Q4Scales q4k_scales(const RawQ4K &r, const Q4Lane &L) {
    const uint32_t T = __builtin_amdgcn_perm(r.h[2], r.h[1], L.selT);
    const uint32_t U = __builtin_amdgcn_perm(r.h[3], r.h[3], L.selU);
    // (T >> 2) moves the top 2 bits of each byte to bits 4..5; the masks keep
    // exactly one rule per lane
    const uint32_t R = (T & L.mA) | ((T >> 2) & L.mB) | (U & L.mC) | ((U >> 4) & L.mD);
    Q4Scales s;
    s.sc0 = (float)(R & 0xFFu);
    s.sc1 = (float)((R >> 8) & 0xFFu);
    s.m0 = (float)((R >> 16) & 0xFFu);
    s.m1 = (float)(R >> 24);
    s.d = f16_lo(r.h[0]);
    s.dmin = f16_hi(r.h[0]);
    return s;
}

// Quant dword dw of the run (bytes 4dw..4dw+3): the four low-nibble weights
// 64c + 4dw + e and the four high-nibble weights 64c + 32 + 4dw + e, each as
// q * fp8_unit() (exact).
struct Q4Nibbles {
    float2 lo01, lo23, hi01, hi23;
};

QD_DEV Q4Nibbles q4k_nibbles(uint32_t v) {
    const uint32_t lo = v & 0x0F0F0F0Fu;
    const uint32_t hi = (v >> 4) & 0x0F0F0F0Fu;
    Q4Nibbles n;
    n.lo01 = nib2_lo(lo);
    n.lo23 = nib2_hi(lo);
    n.hi01 = nib2_lo(hi);
    n.hi23 = nib2_hi(hi);
    return n;
}

// ------------------------------------------------------------------ Q6_K ---
// Block: [0,128) ql, [128,192) qh, [192,208) int8 scales, [208,210) d.
// Lane c = 2h + j takes, in half h, the weights 128h + 32g + 16j + l
// (g = 0..3, l = 0..15): low 4 bits from ql[64h + 16j + l] (g = 0: low
// nibble, g = 2: high nibble) and ql[64h + 32 + 16j + l] (g = 1, 3); high 2
// bits from qh[32h + 16j + l] (bits 2g, 2g+1); scale sc[8h + 2g + j].
// Blocks start on 2-byte boundaries.  Read out of LDS (the streaming
// kernel), every field is taken as whole dwords from the 4-byte-aligned
// address at or below it and re-aligned by `sh` bytes (RawQ6K); read from
// global memory (the register kernels), each field is one 16-byte (quants),
// 8-byte (scales) or 2-byte (d) load at its own address, which global
// memory takes unaligned (RawQ6KA).  No read leaves the block.
struct RawQ6K {
    uint32_t a[5], b[5], h[5];  // ql[64h+16j..], ql[64h+32+16j..], qh[32h+16j..] (+1 dword)
    uint32_t s[3];              // scales of half h (+ slack)
    uint32_t d;                 // dword holding d
    uint32_t sh;                // block start & 3
};
struct RawQ6KA {
    uint32_t a[4], b[4], h[4];  // ql[64h+16j..], ql[64h+32+16j..], qh[32h+16j..]
    uint32_t s[2];              // scales 8h .. 8h + 7
    uint32_t d;                 // f16 d in the low half
};

typedef uint32_t q6_u4a2 __attribute__((ext_vector_type(4), aligned(2)));
typedef uint32_t q6_u2a2 __attribute__((ext_vector_type(2), aligned(2)));
QD_DEV void load_q6k(RawQ6KA &r, const uint8_t *blk, int h, int j) {
    const uint8_t *pa = blk + 64 * h + 16 * j;
    const q6_u4a2 A = *reinterpret_cast<const q6_u4a2 *>(pa);
    const q6_u4a2 Bq = *reinterpret_cast<const q6_u4a2 *>(pa + 32);
    const q6_u4a2 H = *reinterpret_cast<const q6_u4a2 *>(blk + 128 + 32 * h + 16 * j);
    const q6_u2a2 S = *reinterpret_cast<const q6_u2a2 *>(blk + 192 + 8 * h);
#pragma unroll
    for (int k = 0; k < 4; k++) {
        r.a[k] = A[k];
        r.b[k] = Bq[k];
        r.h[k] = H[k];
    }
    r.s[0] = S[0];
    r.s[1] = S[1];
    r.d = *reinterpret_cast<const uint16_t *>(blk + 208);
}

// The ql (a, b) and qh dwords k of a lane's share.
QD_DEV void q6k_dwords(const RawQ6K &r, int k, uint32_t &av, uint32_t &bv, uint32_t &hv) {
    av = align_bytes(r.a[k + 1], r.a[k], r.sh);
    bv = align_bytes(r.b[k + 1], r.b[k], r.sh);
    hv = align_bytes(r.h[k + 1], r.h[k], r.sh);
}
QD_DEV void q6k_dwords(const RawQ6KA &r, int k, uint32_t &av, uint32_t &bv, uint32_t &hv) {
    av = r.a[k];
    bv = r.b[k];
    hv = r.h[k];
}

// Byte lookup of the high bits: hi (0..3) -> (hi - 2) << 4 as a two's
// complement byte, so that (low nibble | table[hi]) is the int8 q - 32.
constexpr uint32_t kQ6HiTable = 0x1000F0E0u;

// Signed bytes (q - 32) of group g = 0..3 for dword k (weights l = 4k..4k+3).
template <class R>
QD_DEV void q6k_qbytes(const R &r, int k, uint32_t (&q)[4]) {
    uint32_t av, bv, hv;
    q6k_dwords(r, k, av, bv, hv);
    q[0] = (av & 0x0F0F0F0Fu) | byte_lut(kQ6HiTable, hv & 0x03030303u);
    q[1] = (bv & 0x0F0F0F0Fu) | byte_lut(kQ6HiTable, (hv >> 2) & 0x03030303u);
    q[2] = ((av >> 4) & 0x0F0F0F0Fu) | byte_lut(kQ6HiTable, (hv >> 4) & 0x03030303u);
    q[3] = ((bv >> 4) & 0x0F0F0F0Fu) | byte_lut(kQ6HiTable, (hv >> 6) & 0x03030303u);
}

struct Q6Scales {
    float sc[4];
    float d;
};

QD_DEV Q6Scales q6k_scales(const RawQ6K &r, int j) {
    const uint32_t s01 = align_bytes(r.s[1], r.s[0], r.sh) >> (8 * j);  // sc[8h+j], sc[8h+2+j]
    const uint32_t s23 = align_bytes(r.s[2], r.s[1], r.sh) >> (8 * j);  // sc[8h+4+j], sc[8h+6+j]
    Q6Scales s;
    s.sc[0] = sbyte(s01, 0);
    s.sc[1] = sbyte(s01, 2);
    s.sc[2] = sbyte(s23, 0);
    s.sc[3] = sbyte(s23, 2);
    s.d = f16_lo(align_bytes(r.d, r.d, r.sh));
    return s;
}
QD_DEV Q6Scales q6k_scales(const RawQ6KA &r, int j) {
    const uint32_t s01 = r.s[0] >> (8 * j);  // sc[8h+j], sc[8h+2+j]
    const uint32_t s23 = r.s[1] >> (8 * j);  // sc[8h+4+j], sc[8h+6+j]
    Q6Scales s;
    s.sc[0] = sbyte(s01, 0);
    s.sc[1] = sbyte(s01, 2);
    s.sc[2] = sbyte(s23, 0);
    s.sc[3] = sbyte(s23, 2);
    s.d = f16_lo(r.d);
    return s;
}

// ------------------------------------------------------------------ Q8_0 ---
// Block: [0,2) d, [2,34) int8 quants.  Lane c takes blocks 8t+2c (A) and
// 8t+2c+1 (B) of superunit t: 68 bytes starting 2-byte aligned.  Of the two,
// one block's quants start on a dword ("P") and the other's 2 bytes past one
// ("Q"); which is which depends only on the row start.  P is read as 8
// aligned dwords plus the dword holding its d (high half); Q as 9 dwords from
// its d onwards (d in the low half, quants re-aligned by 2 bytes).  A block
// past the end of a row (K not a multiple of 256) is not read and decodes to
// zeros with d = 0.
struct RawQ80 {
    uint32_t p[8], pd;
    uint32_t q[9];
    uint32_t a_is_p;  // block A is P (row start & 3 == 2)
};

QD_DEV void load_q80(RawQ80 &r, const uint8_t *rowp, int t, int c, int nblk) {
    const uint8_t *region = rowp + 272 * t + 68 * c;
    const uint32_t s = (uint32_t)(reinterpret_cast<uintptr_t>(region) & 3u);
    r.a_is_p = s ? 1u : 0u;
    const int ia = 8 * t + 2 * c;
    const bool va = ia < nblk, vb = ia + 1 < nblk;
    const bool vp = s ? va : vb, vq = s ? vb : va;
    const uint8_t *qp = region + (s ? 2 : 36);
    const uint8_t *qq = region + (s ? 36 : 2) - 2;
    if (vp) {
        r.pd = ld32(qp - 4);
#pragma unroll
        for (int k = 0; k < 8; k++) r.p[k] = ld32(qp + 4 * k);
    } else {
        r.pd = 0u;
#pragma unroll
        for (int k = 0; k < 8; k++) r.p[k] = 0u;
    }
    if (vq) {
#pragma unroll
        for (int k = 0; k < 9; k++) r.q[k] = ld32(qq + 4 * k);
    } else {
#pragma unroll
        for (int k = 0; k < 9; k++) r.q[k] = 0u;
    }
}

// d of blocks A and B.
QD_DEV float2 q80_d(const RawQ80 &r) {
    const float dp = f16_hi(r.pd), dq = f16_lo(r.q[0]);
    return r.a_is_p ? make_float2(dp, dq) : make_float2(dq, dp);
}

// Quant dword k (weights 4k..4k+3) of blocks A and B.
QD_DEV uint2 q80_qdwords(const RawQ80 &r, int k) {
    const uint32_t vp = r.p[k];
    const uint32_t vq = align_bytes(r.q[k + 1], r.q[k], 2u);
    return r.a_is_p ? make_uint2(vp, vq) : make_uint2(vq, vp);
}

// ----------------------------------------------------------- dispatch ---
template <int FMT>
struct RawOf;
template <> struct RawOf<kQ4K> { using T = RawQ4K; };
template <> struct RawOf<kQ6K> { using T = RawQ6KA; };
template <> struct RawOf<kQ80> { using T = RawQ80; };

// Load lane c's share of superunit t of the row starting at rowp.
template <int FMT>
QD_DEV void load_unit(typename RawOf<FMT>::T &r, const uint8_t *rowp, int t, int c, int nblk) {
    if constexpr (FMT == kQ4K) load_q4k(r, rowp + 144 * t, c);
    else if constexpr (FMT == kQ6K) load_q6k(r, rowp + 210 * t, c >> 1, c & 1);
    else load_q80(r, rowp, t, c, nblk);
}

}  // namespace qd
