// qd_prefill.hip -- multi-token prefill: Y = X bf16(W)^T on the bf16 matrix
// cores (v_mfma_f32_32x32x16_bf16, fp32 accumulation), and the gate/up
// variant H = bf16(act(X Wg^T) * (X Wu^T)).
//
// The pages' instance is the tiled Q8_0 GEMM for multi-token prefill of
// dotLLM PR #320 (the Vulkan backend section of that PR); the larql
// architecture page runs gate and up per position instead.  Here every
// format is handled, and the weights are the bf16 rounding (nearest even) of
// the exact fp32 dequantised value.
//
// Work split.  A workgroup of eight waves (two per SIMD) owns 32*TM tokens
// by 256 accumulator columns.  The waves split the columns only (32 each:
// one 32-row weight slice; for the gate/up variant waves 0-3 take 32 gate
// rows each and waves 4-7 the same rows of up), so each weight is decoded
// once per workgroup, straight from its quantized bytes into the B operand
// of the MFMA, in registers.  Two waves per SIMD let one wave's decode (the
// vector ALU) run while the other's MFMAs execute.  The activations of a
// K-tile (bf16, 128 per token) are shared through LDS: copied there by
// global_load_lds_dwordx4, triple-buffered, with the sixteen 16-byte chunks
// of each token's row XOR-swizzled by the token index so that the operand
// reads of 16 consecutive tokens hit 16 different bank groups.
//
// Operand layout.  In a 32x32x16 MFMA, lane l holds A[l % 32][8 h + j] and
// B[8 h + j][l % 32] (h = l / 32, j = 0..7): the two lane halves hold
// k-positions 0..7 and 8..15 of the step.  A K-tile of 128 weights is half
// a superunit (p = 0, 1) and lane half h decodes exactly the 64 weights that
// the GEMV kernels give to decoder lane c = 2p + h.  Those 64 weights come
// out in runs of 8 consecutive k, in a format-dependent order; each of the
// eight MFMA steps of the K-tile takes one run per lane half and reads the 8
// matching activations from LDS (xchunk below).  The contraction only needs
// both operands to agree on the k of each position, not the natural order.
//
// Split-K.  Shapes with too few output tiles to fill the chip split K across
// workgroups; each writes its partial tile with device-scope stores and the
// last to arrive (device-scope counter) sums the partials in split order, so
// results do not depend on arrival order.
#include "qd_decode.h"


namespace qd {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) const void gbl_void;

constexpr int kXRowBytes = 2 * kGemmKT;  // one token's K-tile of activations

// The 16-byte chunk (8 activations) of a token's K-tile that lane half h
// pairs with its weights in MFMA step s.
template <int FMT>
QD_DEV int xchunk(int s, int h) {
    if constexpr (FMT == kQ4K) {
        // lane c = 2p + h decodes quant run c: low nibbles are weights
        // 64h + i, high nibbles 64h + 32 + i of the K-tile (i = 0..31);
        // steps 0..3 take the low runs of 8, steps 4..7 the high ones
        return 8 * h + 4 * (s >> 2) + (s & 3);
    } else if constexpr (FMT == kQ6K) {
        // lane c = 2p + h decodes weights 32 g + 16 h + l (g = 0..3,
        // l = 0..15) of the K-tile; step s = 2 g + u takes l = 8u..8u+7
        return 4 * (s >> 1) + 2 * h + (s & 1);
    } else {
        // lane c = 2p + h decodes weights 64 h + e (blocks 4p + 2h and
        // 4p + 2h + 1); step s takes e = 8s..8s+7
        return 8 * h + s;
    }
}

// Q6_K rows are 210 bytes, so a block starts on a 2-byte boundary; its
// fields are read as 16-byte (quants), 8-byte (scales) and 2-byte (d) loads
// at 2-byte-aligned addresses, which the hardware reads unaligned.  Lane
// c = 2p + h of superunit t: half p, quant run h (as the GEMV kernels split
// the block).
typedef uint32_t pf_u4a2 __attribute__((ext_vector_type(4), aligned(2)));
typedef uint32_t pf_u2a2 __attribute__((ext_vector_type(2), aligned(2)));
struct RawQ6KU {
    pf_u4a2 a, b, h;  // ql[64p + 16h ..], ql[64p + 32 + 16h ..], qh[32p + 16h ..]
    pf_u2a2 s;        // scales 8p .. 8p + 7
    uint32_t d;       // f16 d in the low half
};
QD_DEV void load_q6k_u(RawQ6KU &r, const uint8_t *blk, int p, int h) {
    const uint8_t *pa = blk + 64 * p + 16 * h;
    r.a = *reinterpret_cast<const pf_u4a2 *>(pa);
    r.b = *reinterpret_cast<const pf_u4a2 *>(pa + 32);
    r.h = *reinterpret_cast<const pf_u4a2 *>(blk + 128 + 32 * p + 16 * h);
    r.s = *reinterpret_cast<const pf_u2a2 *>(blk + 192 + 8 * p);
    r.d = *reinterpret_cast<const uint16_t *>(blk + 208);
}
template <int FMT> struct PfRaw { using T = typename RawOf<FMT>::T; };
template <> struct PfRaw<kQ6K> { using T = RawQ6KU; };
template <int FMT>
QD_DEV void pf_load(typename PfRaw<FMT>::T &r, const uint8_t *rowp, int t, int c, int nblk) {
    if constexpr (FMT == kQ6K) load_q6k_u(r, rowp + 210 * t, c >> 1, c & 1);
    else load_unit<FMT>(r, rowp, t, c, nblk);
}

// Decoded state of one weight row's share of a K-tile, and the bf16 B
// operand of each step.  The bf16 value is the nearest-even rounding of the
// same exact fp32 weight that the dequantise kernel writes.
template <int FMT>
struct Dec;

template <>
struct Dec<kQ4K> {
    uint32_t q[8];
    float a0, b0, a1, b1;  // w = a * (q * unit) + b for the low / high sub-block

    QD_DEV void prep(const RawQ4K &r, int c) {
        const Q4Scales s = q4k_scales(r, q4k_lane(c));
        const float inv_unit = fp8_inv_unit();
        a0 = s.d * s.sc0 * inv_unit;
        a1 = s.d * s.sc1 * inv_unit;
        b0 = -(s.dmin * s.m0);
        b1 = -(s.dmin * s.m1);
#pragma unroll
        for (int i = 0; i < 8; i++) q[i] = r.q[i];
    }
    template <int S>
    QD_DEV bf16x8 step() const {
        constexpr int nib = S >> 2, dw = 2 * (S & 3);
        const float a = nib ? a1 : a0, b = nib ? b1 : b0;
        bf16x8 o;
#pragma unroll
        for (int e = 0; e < 2; e++) {
            const uint32_t v = nib ? (q[dw + e] >> 4) & 0x0F0F0F0Fu : q[dw + e] & 0x0F0F0F0Fu;
            const float2 lo = nib2_lo(v), hi = nib2_hi(v);
            o[4 * e + 0] = (__bf16)fmaf(a, lo.x, b);
            o[4 * e + 1] = (__bf16)fmaf(a, lo.y, b);
            o[4 * e + 2] = (__bf16)fmaf(a, hi.x, b);
            o[4 * e + 3] = (__bf16)fmaf(a, hi.y, b);
        }
        return o;
    }
};

template <>
struct Dec<kQ6K> {
    uint32_t qa[4], qb[4], qh[4];  // ql (two runs) and qh dwords
    float ds[4];                   // d * scale of groups 0..3

    QD_DEV void prep(const RawQ6KU &r, int c) {
        // groups g = 0..3 of run h use scales 8p + h + 2g
        const int sh = 8 * (c & 1);
        const float d = f16_lo(r.d);
        ds[0] = d * sbyte(r.s.x >> sh, 0);
        ds[1] = d * sbyte(r.s.x >> sh, 2);
        ds[2] = d * sbyte(r.s.y >> sh, 0);
        ds[3] = d * sbyte(r.s.y >> sh, 2);
#pragma unroll
        for (int k = 0; k < 4; k++) {
            qa[k] = r.a[k];
            qb[k] = r.b[k];
            qh[k] = r.h[k];
        }
    }
    template <int S>
    QD_DEV bf16x8 step() const {
        constexpr int g = S >> 1, u = S & 1;
        bf16x8 o;
#pragma unroll
        for (int e = 0; e < 2; e++) {
            const int k = 2 * u + e;
            const uint32_t lo = (g & 1) ? qb[k] : qa[k];
            const uint32_t q = ((g >= 2 ? lo >> 4 : lo) & 0x0F0F0F0Fu) |
                               byte_lut(kQ6HiTable, (qh[k] >> (2 * g)) & 0x03030303u);
#pragma unroll
            for (int i = 0; i < 4; i++) o[4 * e + i] = (__bf16)(ds[g] * sbyte(q, i));
        }
        return o;
    }
};

template <>
struct Dec<kQ80> {
    uint32_t qa[8], qb[8];
    float da, db;

    QD_DEV void prep(const RawQ80 &r, int) {
        const float2 d = q80_d(r);
        da = d.x;
        db = d.y;
#pragma unroll
        for (int k = 0; k < 8; k++) {
            const uint2 v = q80_qdwords(r, k);
            qa[k] = v.x;
            qb[k] = v.y;
        }
    }
    template <int S>
    QD_DEV bf16x8 step() const {
        constexpr int blk = S >> 2, k0 = 2 * (S & 3);
        const float d = blk ? db : da;
        bf16x8 o;
#pragma unroll
        for (int e = 0; e < 2; e++) {
            const uint32_t v = blk ? qb[k0 + e] : qa[k0 + e];
#pragma unroll
            for (int i = 0; i < 4; i++) o[4 * e + i] = (__bf16)(d * sbyte(v, i));
        }
        return o;
    }
};

constexpr int kGemmWaves = 8;
constexpr int kGemmThreads = 64 * kGemmWaves;

// Loads are issued two K-tiles ahead: K-tile kt's activations and weights
// are requested while K-tile kt - 2 is multiplied, into the third of three
// activation buffers and three weight register sets.  Global load
// instructions per lane for one K-tile's weights (load_unit): the wait at
// the top of a K-tile leaves the next K-tile's loads in flight.  The count
// only has to be exact for speed; the activations of the current K-tile are
// complete for any value up to twice the true count, and the compiler itself
// waits for weight registers before their first use.
template <int FMT>
constexpr int kPfWeightLoads = FMT == kQ4K ? 3 : FMT == kQ6K ? 5 : 6;

// s_waitcnt with vmcnt(n) and no wait on the other counters
template <int N>
QD_DEV void pf_vm_wait() {
    static_assert(N >= 0 && N < 64, "vmcnt");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// One workgroup per CU, two waves per SIMD (at most 256 registers each).
template <int FMT, bool FFN, int TM>
__global__ __launch_bounds__(kGemmThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void gemm_kernel(GemmArgs a) {
    constexpr int BM = 32 * TM;
    constexpr int XBUF = BM * kXRowBytes;          // bytes per activation buffer
    constexpr int XLOADS = BM / (4 * kGemmWaves);  // global_load_lds per wave per K-tile
    constexpr int TILEF = BM * kGemmCols;          // floats per partial tile
    constexpr int WAVEF = TILEF / kGemmWaves;
    static_assert(XLOADS >= 1 && BM % (4 * kGemmWaves) == 0, "token tile");
    constexpr int NLD = XLOADS + kPfWeightLoads<FMT>;  // load instructions per K-tile
    static_assert(!FFN || 2 * WAVEF * 4 <= XBUF, "up exchange fits two activation buffers");
    // one array per buffer, so that the compiler sees that copies into one
    // cannot alias operand reads of another
    __shared__ __attribute__((aligned(1024))) uint8_t xs0[XBUF];
    __shared__ __attribute__((aligned(1024))) uint8_t xs1[XBUF];
    __shared__ __attribute__((aligned(1024))) uint8_t xs2[XBUF];
    auto xbuf = [&](auto jc) -> uint8_t * {
        constexpr int J = decltype(jc)::value;
        return J == 0 ? xs0 : J == 1 ? xs1 : xs2;
    };
    __shared__ int s_last;

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int h = lane >> 5, l32 = lane & 31;

    const int64_t M = a.M, N = a.N, K = a.K;
    const int KT = a.kt_total;

    // activation staging: load i of this wave fills LDS rows 32 i + 4 w .. +3;
    // lane l writes chunk slot l % 16 of row 32 i + 4 w + l / 16, which holds
    // logical chunk kap = slot ^ (row % 16)
    const int srow = 4 * w + (lane >> 4);
    const int kap = (lane & 15) ^ (srow & 15);
    // A-operand address of token row 32 tm + l32 for chunk kap: the slot is
    // kap ^ (row % 16) = kap ^ (lane % 16)
    const int xa = l32 * kXRowBytes;
    const int sw = lane & 15;

    // ---- this workgroup's segments, each a tile and a range of its K-tiles.
    // Split-K: one segment, K-slice blockIdx / tiles of the tile.  Stream-K
    // (sk_per > 0): the (tile, K-tile) units numbered tile-major, sk_per
    // consecutive units per workgroup, cut where a tile ends.  A tile whose
    // units are shared by nc workgroups is summed by the last of them to
    // arrive, in contributor order, so results do not depend on timing.
    const int64_t units = (int64_t)a.m_tiles * a.n_tiles * KT;
    int64_t u = a.sk_per > 0 ? (int64_t)blockIdx.x * a.sk_per : 0;
    const int64_t u_end = a.sk_per > 0 ? min(units, u + a.sk_per) : 0;
    for (bool more = true; more;) {
        int64_t tile, gf = 0;
        int kt0, kt1, nc, idx;
        if (a.sk_per > 0) {
            if (u >= u_end) break;
            tile = u / KT;
            kt0 = (int)(u - tile * KT);
            kt1 = (int)min<int64_t>(KT, kt0 + (u_end - u));
            gf = tile * KT / a.sk_per;  // contributors gf .. gl
            nc = (int)((tile * KT + KT - 1) / a.sk_per - gf + 1);
            idx = (int)(blockIdx.x - gf);
            u += kt1 - kt0;
        } else {
            more = false;
            const int tiles = a.m_tiles * a.n_tiles;
            const int ks = blockIdx.x / tiles;
            tile = blockIdx.x - (int64_t)ks * tiles;
            kt0 = ks * a.kt_per_split;
            kt1 = min(KT, kt0 + a.kt_per_split);
            nc = a.splits;
            idx = ks;
        }
        // partial-sum slot of contributor c: split-K, tile * splits + c;
        // stream-K, 2 g (+1 when the tile is not g's first), g = gf + c
        auto slot_of = [&](int c) -> int64_t {
            if (a.sk_per <= 0) return tile * a.splits + c;
            const int64_t g = gf + c;
            return 2 * g + ((g * a.sk_per) / KT == tile ? 0 : 1);
        };
        const int mt = (int)(tile % a.m_tiles), nt = (int)(tile / a.m_tiles);
        const int64_t m0 = (int64_t)mt * BM;

        // weight row of this lane (rows past N read row N-1; never stored)
        int64_t nrow;
        const uint8_t *rowp;
        if constexpr (FFN) {
            nrow = (int64_t)nt * 128 + 32 * (w & 3) + l32;
            rowp = (w < 4 ? a.Wg : a.Wu) + min(nrow, N - 1) * a.row_bytes;
        } else {
            nrow = (int64_t)nt * kGemmCols + 32 * w + l32;
            rowp = a.Wg + min(nrow, N - 1) * a.row_bytes;
        }
        uint32_t xoff[XLOADS];  // element offset of each staged row (rows past M read row M-1)
#pragma unroll
        for (int i = 0; i < XLOADS; i++)
            xoff[i] = (uint32_t)(min(m0 + 4 * kGemmWaves * i + srow, M - 1) * K) + 8 * kap;

        typename PfRaw<FMT>::T raw[3];  // [buffer]
        Dec<FMT> dec;
        f32x16 acc[TM];
#pragma unroll
        for (int i = 0; i < TM; i++) acc[i] = f32x16{};

        auto issue = [&](int kt, auto jc, typename PfRaw<FMT>::T &rw) {
            const int64_t kbase = (int64_t)kt * kGemmKT;
            const bool kin = kbase + 8 * kap < K;
            uint8_t *dst = xbuf(jc) + w * 1024;
            // a chunk past K reads X[0..7] (always in bounds) and is zeroed in
            // LDS before use, so both arms of the select share one address form
#pragma unroll
            for (int i = 0; i < XLOADS; i++)
                __builtin_amdgcn_global_load_lds((gbl_void *)(a.X + (kin ? xoff[i] + kbase : 0)),
                                                 (lds_void *)(dst + i * 1024 * kGemmWaves), 16, 0, 0);
            const int t = kt >> 1, c = 2 * (kt & 1) + h;
            pf_load<FMT>(rw, rowp, t, c, a.nblk);
        };

        auto body = [&](int kt, auto jc) {
            constexpr int buf = decltype(jc)::value, nbuf = (buf + 2) % 3;
            // K-tile kt's loads are complete; kt + 1's may still be in flight
            pf_vm_wait<NLD>();
            if ((int64_t)(kt + 1) * kGemmKT > K &&
                (int64_t)kt * kGemmKT + 8 * kap >= K) {  // zero the chunks past K
                uint8_t *dst = xbuf(jc) + w * 1024 + 16 * lane;
#pragma unroll
                for (int i = 0; i < XLOADS; i++)
                    *reinterpret_cast<uint4 *>(dst + i * 1024 * kGemmWaves) = make_uint4(0u, 0u, 0u, 0u);
            }
            // ... and every wave's; the buffer of kt - 1 is free.  A plain
            // barrier: __syncthreads() would also wait for the loads in flight
            __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4) | (0 << 8));  // lgkmcnt(0)
            __builtin_amdgcn_s_barrier();
            dec.prep(raw[buf], 2 * (kt & 1) + h);
            // every body issues (the last two repeat the segment's last K-tile
            // into buffers nobody reads), so each buffer keeps its registers and
            // the count of loads in flight is the same at every wait
            issue(min(kt + 2, kt1 - 1), std::integral_constant<int, nbuf>{}, raw[nbuf]);
            const uint8_t *xb = xbuf(jc) + xa;
            // A operands of step S (TM token rows) from LDS
            auto load_a = [&](auto sc, bf16x8 (&A)[TM]) {
                constexpr int S = decltype(sc)::value;
                const int off = 16 * (xchunk<FMT>(S, h) ^ sw);
#pragma unroll
                for (int i = 0; i < TM; i++)
                    A[i] = *reinterpret_cast<const bf16x8 *>(xb + i * 32 * kXRowBytes + off);
                // keep these reads ahead of the MFMAs that follow (the scheduler
                // would otherwise sink them next to their own, later MFMAs)
                __builtin_amdgcn_sched_barrier(0);
            };
            // step S's MFMAs on A; the operands of step S + 1 are read into the
            // other buffer first, so their LDS latency overlaps these MFMAs
            auto mstep = [&](auto sc, const bf16x8 (&A)[TM]) {
                constexpr int S = decltype(sc)::value;
                const bf16x8 B = dec.template step<S>();
#pragma unroll
                for (int i = 0; i < TM; i++) acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[i], B, acc[i], 0, 0, 0);
            };
            bf16x8 Ae[TM], Ao[TM];
            load_a(std::integral_constant<int, 0>{}, Ae);
            load_a(std::integral_constant<int, 1>{}, Ao);
            mstep(std::integral_constant<int, 0>{}, Ae);
            load_a(std::integral_constant<int, 2>{}, Ae);
            mstep(std::integral_constant<int, 1>{}, Ao);
            load_a(std::integral_constant<int, 3>{}, Ao);
            mstep(std::integral_constant<int, 2>{}, Ae);
            load_a(std::integral_constant<int, 4>{}, Ae);
            mstep(std::integral_constant<int, 3>{}, Ao);
            load_a(std::integral_constant<int, 5>{}, Ao);
            mstep(std::integral_constant<int, 4>{}, Ae);
            load_a(std::integral_constant<int, 6>{}, Ae);
            mstep(std::integral_constant<int, 5>{}, Ao);
            load_a(std::integral_constant<int, 7>{}, Ao);
            mstep(std::integral_constant<int, 6>{}, Ae);
            mstep(std::integral_constant<int, 7>{}, Ao);
        };

        issue(kt0, std::integral_constant<int, 0>{}, raw[0]);
        __builtin_amdgcn_sched_barrier(0);  // K-tile kt0's loads all go first
        issue(min(kt0 + 1, kt1 - 1), std::integral_constant<int, 1>{}, raw[1]);
        // whole rounds of three K-tiles, then the one or two left (no path
        // through the loop skips a stage, so the wait counts above hold on it)
        int kt = kt0;
        for (; kt + 2 < kt1; kt += 3) {
            body(kt, std::integral_constant<int, 0>{});
            body(kt + 1, std::integral_constant<int, 1>{});
            body(kt + 2, std::integral_constant<int, 2>{});
        }
        if (kt < kt1) body(kt, std::integral_constant<int, 0>{});
        if (kt + 1 < kt1) body(kt + 1, std::integral_constant<int, 1>{});
        pf_vm_wait<0>();  // the repeated loads have landed before LDS is reused or released

        // ---- a tile shared by several workgroups: publish, then the last
        // to arrive sums the partials in contributor order
        bool owner = true;
        if (nc > 1) {
            float *own = a.partials + slot_of(idx) * TILEF + w * WAVEF + lane;
#pragma unroll
            for (int i = 0; i < TM; i++)
#pragma unroll
                for (int r = 0; r < 16; r++)
                    __hip_atomic_store(own + (i * 16 + r) * 64, acc[i][r], __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
            __atomic_signal_fence(__ATOMIC_SEQ_CST);  // keep the stores above the wait
            __builtin_amdgcn_s_waitcnt(0);            // this wave's stores are complete
            __syncthreads();
            if (tid == 0) {
                const unsigned prev = __hip_atomic_fetch_add(a.counters + tile, 1u, __ATOMIC_RELAXED,
                                                             __HIP_MEMORY_SCOPE_AGENT);
                s_last = prev == (unsigned)nc - 1 ? 1 : 0;
            }
            __syncthreads();
            owner = s_last != 0;
            if (owner) {
#pragma unroll
                for (int i = 0; i < TM; i++)
#pragma unroll
                    for (int r = 0; r < 16; r++) acc[i][r] = 0.f;
                for (int c = 0; c < nc; c++) {
                    const float *p = a.partials + slot_of(c) * TILEF + w * WAVEF + lane;
#pragma unroll
                    for (int i = 0; i < TM; i++)
#pragma unroll
                        for (int r = 0; r < 16; r++)
                            acc[i][r] += __hip_atomic_load(p + (i * 16 + r) * 64, __ATOMIC_RELAXED,
                                                           __HIP_MEMORY_SCOPE_AGENT);
                }
                if (tid == 0)  // ready for the next call
                    __hip_atomic_store(a.counters + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }

        // ---- epilogue: accumulator register r of lane l is token
        // 8 (r / 4) + 4 h + r % 4 of the 32-token slice, column l % 32
        if (owner) {
            if constexpr (FFN) {
                // the up waves hand their sums to the gate waves of the same rows
                // through the (now idle) activation buffers
                float *ub = reinterpret_cast<float *>((w & 2) ? xs1 : xs0) + (w & 1) * WAVEF + lane;
                __syncthreads();  // every wave's last operand reads are done
                if (w >= 4) {
#pragma unroll
                    for (int i = 0; i < TM; i++)
#pragma unroll
                        for (int r = 0; r < 16; r++) ub[(i * 16 + r) * 64] = acc[i][r];
                }
                __syncthreads();
                if (w < 4 && nrow < N) {
#pragma unroll
                    for (int i = 0; i < TM; i++)
#pragma unroll
                        for (int r = 0; r < 16; r++) {
                            const int64_t m = m0 + 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
                            if (m >= M) continue;
                            const float g = acc[i][r], uu = ub[(i * 16 + r) * 64];
                            const int64_t o = m * N + nrow;
                            a.H[o] = f32_to_bf16(act_apply(a.act, g) * uu);
                            if (a.g_out) a.g_out[o] = g;
                            if (a.u_out) a.u_out[o] = uu;
                        }
                }
            } else if (nrow < N) {
#pragma unroll
                for (int i = 0; i < TM; i++)
#pragma unroll
                    for (int r = 0; r < 16; r++) {
                        const int64_t m = m0 + 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
                        if (m < M) a.Y[m * N + nrow] = acc[i][r];
                    }
            }
        }
        __syncthreads();  // LDS and s_last free for the next segment
    }
}

template <int FMT, bool FFN>
hipError_t launch_f(int tm, const GemmArgs &a, hipStream_t st) {
    const int64_t units = (int64_t)a.m_tiles * a.n_tiles * a.kt_total;
    const int64_t grid = a.sk_per > 0 ? (units + a.sk_per - 1) / a.sk_per : (int64_t)a.m_tiles * a.n_tiles * a.splits;
    if (grid <= 0 || grid > 0x7FFFFFFF) return hipErrorInvalidValue;
    if (tm == 4)
        hipLaunchKernelGGL((gemm_kernel<FMT, FFN, 4>), dim3((unsigned)grid), dim3(kGemmThreads), 0, st, a);
    else if (tm == 2)
        hipLaunchKernelGGL((gemm_kernel<FMT, FFN, 2>), dim3((unsigned)grid), dim3(kGemmThreads), 0, st, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(int fmt, bool ffn, int tm, const GemmArgs &a, hipStream_t st) {
    switch (fmt) {
    case kQ4K: return ffn ? launch_f<kQ4K, true>(tm, a, st) : launch_f<kQ4K, false>(tm, a, st);
    case kQ6K: return ffn ? launch_f<kQ6K, true>(tm, a, st) : launch_f<kQ6K, false>(tm, a, st);
    case kQ80: return ffn ? launch_f<kQ80, true>(tm, a, st) : launch_f<kQ80, false>(tm, a, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace qd
