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
//    Q4_K or Q6_K block, eight Q8_0 blocks).  Copying waves put the steps
//    into a ring in LDS with global_load_lds_dwordx4 (1 KB of consecutive
//    bytes per instruction, no registers), several steps in flight;
//    decoding waves take them out of the ring as they land.
//  * Decoding reads a lane group's block (4 lanes per superunit, the lane
//    split of the GEMV kernels) and its activation digits from LDS, and
//    writes the superunit's partial sum to LDS.  After the stream, each
//    row's partials are added in an order fixed by the row length alone
//    (8 lanes per row), so a result does not depend on the launch shape.
//  * x is multiplied by the RMS-norm weight and staged once per workgroup
//    as activation digits (qd_digits.h: exact integer products); the
//    inverse RMS is applied to each row's sum at the end.
//  * The same body serves the routed experts of the MoE decode FFN (the
//    slots share the CUs, each workgroup a row range of one slot's expert)
//    and the Q, K and V projections in one launch (the CUs shared by the
//    three matrices, each workgroup in its own matrix's format).
// The copies are ordered by explicit waits (qd_lds.h).
#include "qd_decode.h"
#include "qd_digits.h"
#include "qd_epilogue.h"
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

// ------------------------------------------------------ one step ---
// A lane's share of one superunit (per row stream) out of the ring; the
// activations are read as digits (qd_digits.h) while multiplying.
// Q6_K out of LDS keeps the re-aligned dword form (LDS takes no unaligned
// 16-byte reads).
template <int FMT>
struct LdsRaw { using T = typename RawOf<FMT>::T; };
template <> struct LdsRaw<kQ6K> { using T = RawQ6K; };
template <int FMT, int NR>
struct StepRegs {
    typename LdsRaw<FMT>::T raw[NR];
};

// blk0: the lane group's superunit in row stream 0 (stream m is m * mstride
// bytes further).
template <int FMT, int NR>
QD_DEV void read_step(StepRegs<FMT, NR> &st, const uint8_t *blk0, int mstride, int c) {
#pragma unroll
    for (int m = 0; m < NR; m++) {
        const uint8_t *blk = blk0 + m * mstride;
        if constexpr (FMT == kQ4K) lds_q4k(st.raw[m], blk, c);
        else if constexpr (FMT == kQ6K) lds_q6k(st.raw[m], blk, c >> 1, c & 1);
        else lds_q80(st.raw[m], blk, c);
    }
}

// xd: the staged digits of superunit su of batch row 0; xsb: bytes per
// batch row of staged digits.
template <int FMT, int B, int NR>
QD_DEV void dot_step(const StepRegs<FMT, NR> &st, const uint8_t *xd, int xsb, const Q4Lane &L4, int c,
                     float (&v)[NR][B]) {
#pragma unroll
    for (int m = 0; m < NR; m++)
#pragma unroll
        for (int b = 0; b < B; b++) v[m][b] = 0.f;
    if constexpr (FMT == kQ4K) q4k_step_dig<NR, B>(st.raw, xd, xsb, c, L4, v);
    else if constexpr (FMT == kQ6K) q6k_step_dig<NR, B>(st.raw, xd, xsb, c >> 1, c & 1, v);
    else q80_step_dig<NR, B>(st.raw, xd, xsb, c, v);
}

// ------------------------------------------------ producer / consumer ---
// The same products with the two jobs given to different waves, which never
// wait on a workgroup barrier inside the stream.  A wave that issues copies
// stalls at issue whenever the memory pipeline backs up, so the copying waves
// do little else, and their copies are issued from scalar registers:
//   * waves 0 .. NC-1 decode (consumers).  First they stage x as digits
//     (qd_digits.h), one superunit of one batch row per slice, each wave
//     its own slices: loaded straight into registers with the norm weight
//     (each wave counts itself on `landed` once its first slices have
//     arrived), x * w_norm, each wave's sum of squares of x (added in wave
//     order, so the inverse RMS does not depend on timing), digits and run
//     records into LDS; they meet on `staged`.  Then consumer c takes steps
//     c, c + NC, ... and, after reading a step's weights out of its slot
//     (the digits stay), stores the number of its steps read so far in
//     done[c];
//   * waves NC .. NC + 3 copy the weights (producers; as many as the launch
//     asks for, 1, 2 or 4, and the others idle).  Where x holds more than
//     kXFirstSlices slices they issue nothing before it has landed, so x
//     does not queue behind the weight stream (MI355X, graph replay: the
//     Gemma-3 down's 40 KB of h lands 0.9 us later without the wait); a
//     shorter x goes out alongside the first weights (the Gemma-3 gate/up,
//     10 slices: 10.55 -> 10.28 us with no wait).  Producer p takes the
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
constexpr int kXFirstSlices = 16;  // longer staged x: the copying waves wait for it

// Mixture-of-experts slots (MOE): the launch holds n_sel * wps workgroups,
// workgroup i serving routed slot z = i / wps with row range i % wps of that
// slot's expert e = ids[z] (an id outside [0, n_experts) streams expert 0
// and its result is dropped).  The copying waves read the id while x lands.
//   * gate/up (FFN): x is shared by the slots; slot z writes h_z at
//     y + z * y_sstride (zeros for an invalid id);
//   * down: slot z reads h_z at x + z * x_sstride and stores its rows into
//     part[z]; the last of the n_sel workgroups of a row range (counter per
//     range) forms y = sum of coef[z] * part[z] over the valid slots, in slot
//     order, and returns the counter to zero.
// wg: the workgroup's index in its launch (or in its matrix's share of one).
template <int FMT, int B, int NR, bool FFN, int NC, bool MOE>
QD_DEV void stream_pc_body(StreamArgs a, int wg) {
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

    int z = 0;                 // routed slot (MOE)
    const float *xin = a.x;
    if constexpr (MOE) {
        z = wg / a.wps;
        wg -= z * a.wps;
        if constexpr (!FFN) xin += (int64_t)z * a.x_sstride;
    }
    const int64_t r0 = (int64_t)wg * a.rows_base + min(wg, a.rows_extra);
    const int cnt = a.rows_base + (wg < a.rows_extra ? 1 : 0);
    const int U = cnt * nb;
    const int S = (U + kStepUnits - 1) / kStepUnits;

    uint8_t *ring = smem;
    uint8_t *xd = smem + a.off_x;  // [B][nb] staged digit superunits
    float *part = reinterpret_cast<float *>(smem + a.off_part);
    int *ready = reinterpret_cast<int *>(smem + a.off_red);
    int *done = ready + R;     // [NC]
    int *landed = done + NC;
    int *staged = landed + 1;
    float *rinv = reinterpret_cast<float *>(staged + 1);  // [B]
    float *ssq = rinv + B;                                // [NC][B]
    const int xsb = nb * kDigSU;  // bytes per batch row of staged digits
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
            const uint8_t *W0 = a.W0, *W1 = a.W1;
            if constexpr (MOE) {
                int e = a.ids[z];
                e = (e >= 0 && e < a.n_experts) ? e : 0;
                W0 += (int64_t)e * a.w_estride;
                if constexpr (FFN) W1 += (int64_t)e * a.w_estride;
            }
            if (B * nb > kXFirstSlices) lds_wait_eq(landed, NC);
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
                            const uint8_t *sp = (m == 0 ? W0 : W1) + a0;
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
                                    lds_copy16((m == 0 ? W0 : W1) + off, dst + m * SLOTM + 1024 * q);
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
        // stage x as digits (qd_digits.h): slice it (one superunit of one
        // batch row, 64 float4) goes to wave it % NC.  The wave loads a
        // chunk of its slices straight into registers (x and the norm
        // weight), counts itself on `landed` once its first chunk has
        // arrived (the copying waves start then, so x does not queue behind
        // the weight stream), multiplies by the norm weight, adds its sums
        // of squares, and writes the digits.
        const int nslices = B * nb;
        float ss[B];
#pragma unroll
        for (int b = 0; b < B; b++) ss[b] = 0.f;
        constexpr int CH = 6;  // slices per chunk
        for (int c0 = 0;; c0 += CH) {
            float4 xv[CH], nv[CH];
#pragma unroll
            for (int i = 0; i < CH; i++) {
                const int it = wv + NC * (c0 + i);
                nv[i] = make_float4(1.f, 1.f, 1.f, 1.f);
                if (it < nslices) {  // uniform per wave
                    const int b = it / nb;
                    const int64_t k = (int64_t)(it - b * nb) * kSuper + 4 * lane;
                    xv[i] = *reinterpret_cast<const float4 *>(xin + (int64_t)b * K + k);
                    if (norm) nv[i] = *reinterpret_cast<const float4 *>(a.norm_w + k);
                }
            }
            if (c0 == 0) {
                vm_wait<0>();
                if (lane == 0) lds_add(landed, 1);
            }
#pragma unroll
            for (int i = 0; i < CH; i++) {
                const int it = wv + NC * (c0 + i);
                if (it >= nslices) break;  // uniform per wave
                const int b = it / nb;
                const int su = it - b * nb;
                float4 v = xv[i];
                if (norm) {
                    float sq = fmaf(v.x, v.x, 0.f);
                    sq = fmaf(v.y, v.y, sq);
                    sq = fmaf(v.z, v.z, sq);
                    sq = fmaf(v.w, v.w, sq);
#pragma unroll
                    for (int bb = 0; bb < B; bb++)
                        if (bb == b) ss[bb] += sq;
                    v.x *= nv[i].x;
                    v.y *= nv[i].y;
                    v.z *= nv[i].z;
                    v.w *= nv[i].w;
                }
                uint8_t *sup = xd + b * xsb + su * kDigSU;
                stage_digits<FMT == kQ4K>(v, sup, 4 * lane);
            }
            if (wv + NC * (c0 + CH) >= nslices) break;
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
            StepRegs<FMT, NR> st;
            read_step<FMT, NR>(st, ring + slot * NR * SLOTM + off0 + g * UB, SLOTM, c);
            lgkm_wait();  // the slot may be refilled from here on
            if (lane == 0) lds_flag(&done[wv], ++nread);
            float v[NR][B];
            dot_step<FMT, B, NR>(st, xd + su * kDigSU, xsb, L4, c, v);
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

    // ---- rows: partials summed in a fixed order (lane t of a row's 8 adds
    // superunits t, t + 8, ... in order, then the 8 sums are added by a
    // fixed cross-lane tree), times the inverse RMS
    const int Umax = a.units_max;
    const int l8 = tid & 7;
    for (int e0 = 0; e0 < cnt * B; e0 += NT / 8) {
        const int e = e0 + (tid >> 3);
        const bool on = e < cnt * B;  // the same for the 8 lanes of a row
        const int b = on ? e / cnt : 0;
        const int lr = on ? e - b * cnt : 0;
        const int64_t row = r0 + lr;
        float sr[NR];
#pragma unroll
        for (int m = 0; m < NR; m++) {
            const float *pp = part + (m * B + b) * Umax + lr * nb;
            float acc = 0.f;
            if (on)
                for (int t = l8; t < nb; t += 8) acc += pp[t];
            sr[m] = oct_sum(acc) * rinv[b];
        }
        if (!on || l8 != 0) continue;
        if constexpr (MOE) {
            if constexpr (FFN) {
                const int e = a.ids[z];
                const bool valid = e >= 0 && e < a.n_experts;
                a.y[(int64_t)z * a.y_sstride + row] = valid ? act_apply(a.act, sr[0]) * sr[1] : 0.f;
            } else {
                xstore(a.part + (int64_t)z * N + row, sr[0]);
            }
            continue;
        }
        if constexpr (FFN) {
            a.y[(int64_t)b * N + row] = act_apply(a.act, sr[0]) * sr[1];
            if (a.g_out) a.g_out[(int64_t)b * N + row] = sr[0];
            if (a.u_out) a.u_out[(int64_t)b * N + row] = sr[1];
        } else {
            const int64_t o = (int64_t)b * N + row;
            if (a.pn.w1) xstore(a.pn.p + o, sr[0]);  // the row epilogue forms y
            else a.y[o] = a.res ? sr[0] + a.res[o] : sr[0];
        }
    }
    if constexpr (MOE && !FFN) {
        // the slots' rows of this range: the last of the n_sel workgroups
        // sums them (the ring, offset 0, is free once every step is decoded)
        if (!arrive_last<NT>(a.counters + wg, (unsigned)a.n_sel, reinterpret_cast<int *>(smem))) return;
        for (int lr = tid; lr < cnt; lr += NT) {
            const int64_t row = r0 + lr;
            float s = 0.f;
            for (int z0 = 0; z0 < a.n_sel; z0 += 8) {
                float v[8];  // eight slots' loads in flight together
#pragma unroll
                for (int i = 0; i < 8; i++)
                    v[i] = z0 + i < a.n_sel ? xload(a.part + (int64_t)(z0 + i) * N + row) : 0.f;
#pragma unroll
                for (int i = 0; i < 8; i++) {
                    const int zz = z0 + i;
                    if (zz >= a.n_sel) break;
                    const int e = a.ids[zz];
                    if (e >= 0 && e < a.n_experts) s = fmaf(a.coef[zz], v[i], s);
                }
            }
            a.y[row] = s;
        }
        if (tid == 0) __hip_atomic_store(a.counters + wg, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else if constexpr (!FFN) {
        // the ring (offset 0) is free once every step has been decoded
        if (a.pn.w1)
            post_norm_tail<NT>(a.pn, a.y, B, N, reinterpret_cast<float *>(smem), reinterpret_cast<int *>(smem + 64));
    }
}

template <int FMT, int B, int NR, bool FFN, int NC, bool MOE>
__global__ __launch_bounds__(64 * (NC + kPcMaxProducers)) void stream_pc_kernel(StreamArgs a) {
    stream_pc_body<FMT, B, NR, FFN, NC, MOE>(a, blockIdx.x);
}

// Q, K and V projections of one token in one launch (batch 1): workgroup t
// belongs to matrix 0, 1 or 2 by its index and streams that matrix's share
// of rows in that matrix's format; every workgroup stages (and
// RMS-normalises) x itself, so the three matrices' workgroups are
// independent.
__global__ __launch_bounds__(64 * (8 + kPcMaxProducers)) void stream_qkv_kernel(StreamQkvArgs q) {
    int t = (int)blockIdx.x;
    int s = 0;
    if (t >= q.wgs[0]) {
        t -= q.wgs[0];
        s = 1;
        if (t >= q.wgs[1]) {
            t -= q.wgs[1];
            s = 2;
        }
    }
    const StreamArgs &a = q.a[s];
    switch (q.fmt[s]) {
    case kQ4K: stream_pc_body<kQ4K, 1, 1, false, 8, false>(a, t); break;
    case kQ6K: stream_pc_body<kQ6K, 1, 1, false, 8, false>(a, t); break;
    default: stream_pc_body<kQ80, 1, 1, false, 8, false>(a, t); break;
    }
}

}  // namespace

// LDS layout of the producer / consumer kernel with `slots` ring slots; returns
// the bytes used.
size_t stream_pc_layout(int fmt, int batch, bool ffn, int nb, int units_max, int slots,
                        StreamArgs *a) {
    const int NR = ffn ? 2 : 1;
    int nch = fmt == kQ4K ? StreamFmt<kQ4K>::NCH : fmt == kQ6K ? StreamFmt<kQ6K>::NCH
                                                                : StreamFmt<kQ80>::NCH;
    size_t off = (size_t)slots * NR * nch * 16;
    a->off_x = (int)off;
    off += (size_t)batch * nb * kDigSU;
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

template <int FMT, int B, bool FFN, int NC, bool MOE = false>
static hipError_t launch_pc(const StreamArgs &a, unsigned grid, size_t lds, hipStream_t st) {
    constexpr int NR = FFN ? 2 : 1;
    if (allow_lds<stream_pc_kernel<FMT, B, NR, FFN, NC, MOE>>() != hipSuccess) return hipErrorInvalidValue;
    hipLaunchKernelGGL((stream_pc_kernel<FMT, B, NR, FFN, NC, MOE>), dim3(grid), dim3(64 * (NC + kPcMaxProducers)),
                       lds, st, a);
    return hipGetLastError();
}

template <int FMT, int B>
static hipError_t launch_sb(const StreamArgs &a, bool ffn, unsigned grid, size_t lds, hipStream_t st) {
    if (a.consumers == 4)
        return ffn ? launch_pc<FMT, B, true, 4>(a, grid, lds, st) : launch_pc<FMT, B, false, 4>(a, grid, lds, st);
    if (a.consumers == 8)
        return ffn ? launch_pc<FMT, B, true, 8>(a, grid, lds, st) : launch_pc<FMT, B, false, 8>(a, grid, lds, st);
    return hipErrorInvalidValue;
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

hipError_t launch_stream_qkv(const StreamQkvArgs &q, size_t lds, hipStream_t st) {
    for (int i = 0; i < 3; i++)
        if (q.a[i].consumers != 8) return hipErrorInvalidValue;
    if (allow_lds<stream_qkv_kernel>() != hipSuccess) return hipErrorInvalidValue;
    const unsigned grid = (unsigned)(q.wgs[0] + q.wgs[1] + q.wgs[2]);
    hipLaunchKernelGGL(stream_qkv_kernel, dim3(grid), dim3(64 * (8 + kPcMaxProducers)), lds, st, q);
    return hipGetLastError();
}

// The routed experts' launches of the MoE decode FFN (batch 1, 8 decoding
// waves).
hipError_t launch_stream_moe(int fmt, bool ffn, const StreamArgs &a, unsigned grid, size_t lds,
                             hipStream_t st) {
    if (a.consumers != 8) return hipErrorInvalidValue;
    switch (fmt) {
    case kQ4K: return ffn ? launch_pc<kQ4K, 1, true, 8, true>(a, grid, lds, st) : launch_pc<kQ4K, 1, false, 8, true>(a, grid, lds, st);
    case kQ6K: return ffn ? launch_pc<kQ6K, 1, true, 8, true>(a, grid, lds, st) : launch_pc<kQ6K, 1, false, 8, true>(a, grid, lds, st);
    case kQ80: return ffn ? launch_pc<kQ80, 1, true, 8, true>(a, grid, lds, st) : launch_pc<kQ80, 1, false, 8, true>(a, grid, lds, st);
    default: return hipErrorInvalidValue;
    }
}


}  // namespace qd
