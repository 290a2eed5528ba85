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
// Work split.  A workgroup of four waves owns 32*TM tokens by 256
// accumulator columns.  The waves split the columns only (64 each: two
// 32-row weight slices, or 32 gate rows and the same 32 up rows), so each
// weight is decoded once per workgroup, straight from its quantized bytes
// into the B operand of the MFMA, in registers.  The activations of a
// K-tile (bf16, 128 per token) are shared through LDS: copied there by
// global_load_lds_dwordx4, double-buffered, with the sixteen 16-byte chunks
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
    uint32_t qa[4], qb[4], qh[4];  // re-aligned ql (two runs) and qh dwords
    float ds[4];                   // d * scale of groups 0..3

    QD_DEV void prep(const RawQ6K &r, int c) {
        const Q6Scales s = q6k_scales(r, c & 1);
#pragma unroll
        for (int g = 0; g < 4; g++) ds[g] = s.d * s.sc[g];
#pragma unroll
        for (int k = 0; k < 4; k++) {
            qa[k] = align_bytes(r.a[k + 1], r.a[k], r.sh);
            qb[k] = align_bytes(r.b[k + 1], r.b[k], r.sh);
            qh[k] = align_bytes(r.h[k + 1], r.h[k], r.sh);
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

// One workgroup per CU and so one wave per SIMD: the whole register file is
// this wave's, which lets the next step's activation operands load while the
// current step's MFMAs run.
template <int FMT, bool FFN, int TM>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_kernel(GemmArgs a) {
    constexpr int BM = 32 * TM;
    constexpr int XBUF = BM * kXRowBytes;     // bytes per activation buffer
    constexpr int XLOADS = BM / 16;           // global_load_lds per wave per K-tile
    constexpr int TILEF = BM * kGemmCols;     // floats per partial tile
    constexpr int WAVEF = TILEF / 4;
    __shared__ __attribute__((aligned(1024))) uint8_t xs[2 * XBUF];
    __shared__ int s_last;

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int h = lane >> 5, l32 = lane & 31;

    int bid = blockIdx.x;
    const int mt = bid % a.m_tiles;
    bid /= a.m_tiles;
    const int nt = bid % a.n_tiles;
    const int ks = bid / a.n_tiles;
    const int64_t M = a.M, N = a.N, K = a.K;
    const int64_t m0 = (int64_t)mt * BM;
    const int kt0 = ks * a.kt_per_split;
    const int kt1 = min(a.kt_total, kt0 + a.kt_per_split);

    // weight rows of this lane (rows past N read row N-1; never stored)
    int64_t nrow[2];
    const uint8_t *rowp[2];
    if constexpr (FFN) {
        nrow[0] = nrow[1] = (int64_t)nt * 128 + 32 * w + l32;
        const int64_t nc = min(nrow[0], N - 1);
        rowp[0] = a.Wg + nc * a.row_bytes;
        rowp[1] = a.Wu + nc * a.row_bytes;
    } else {
#pragma unroll
        for (int i = 0; i < 2; i++) {
            nrow[i] = (int64_t)nt * kGemmCols + 64 * w + 32 * i + l32;
            rowp[i] = a.Wg + min(nrow[i], N - 1) * a.row_bytes;
        }
    }

    // activation staging: load i of this wave fills LDS rows 16 i + 4 w .. +3;
    // lane l writes chunk slot l % 16 of row 16 i + 4 w + l / 16, which holds
    // logical chunk kap = slot ^ (row % 16)
    const int srow = 4 * w + (lane >> 4);
    const int kap = (lane & 15) ^ (srow & 15);
    uint32_t xoff[XLOADS];  // element offset of each staged row (rows past M read row M-1)
#pragma unroll
    for (int i = 0; i < XLOADS; i++)
        xoff[i] = (uint32_t)(min(m0 + 16 * i + srow, M - 1) * K) + 8 * kap;

    typename RawOf<FMT>::T raw[2][2];  // [buffer][row]
    Dec<FMT> dec[2];
    f32x16 acc[TM][2];
#pragma unroll
    for (int i = 0; i < TM; i++) acc[i][0] = acc[i][1] = f32x16{};

    auto issue = [&](int kt, int buf, typename RawOf<FMT>::T (&rw)[2]) {
        const int64_t kbase = (int64_t)kt * kGemmKT;
        const bool kin = kbase + 8 * kap < K;
        uint8_t *dst = xs + buf * XBUF + w * 1024;
        // a chunk past K reads X[0..7] (always in bounds) and is zeroed in
        // LDS before use, so both arms of the select share one address form
#pragma unroll
        for (int i = 0; i < XLOADS; i++)
            __builtin_amdgcn_global_load_lds((gbl_void *)(a.X + (kin ? xoff[i] + kbase : 0)),
                                             (lds_void *)(dst + i * 4096), 16, 0, 0);
        const int t = kt >> 1, c = 2 * (kt & 1) + h;
        load_unit<FMT>(rw[0], rowp[0], t, c, a.nblk);
        load_unit<FMT>(rw[1], rowp[1], t, c, a.nblk);
    };

    // A-operand address of token row 32 tm + l32 for chunk kap: the slot is
    // kap ^ (row % 16) = kap ^ (lane % 16)
    const uint8_t *xa = xs + l32 * kXRowBytes;
    const int sw = lane & 15;

    auto body = [&](int kt, int buf, typename RawOf<FMT>::T (&cur)[2],
                    typename RawOf<FMT>::T (&nxt)[2]) {
        __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of K-tile kt are complete
        if ((int64_t)(kt + 1) * kGemmKT > K &&
            (int64_t)kt * kGemmKT + 8 * kap >= K) {  // zero the chunks past K
            uint8_t *dst = xs + buf * XBUF + w * 1024 + 16 * lane;
#pragma unroll
            for (int i = 0; i < XLOADS; i++)
                *reinterpret_cast<uint4 *>(dst + i * 4096) = make_uint4(0u, 0u, 0u, 0u);
        }
        __syncthreads();                // ... and every wave's; buffer buf^1 is free
        const int c = 2 * (kt & 1) + h;
        dec[0].prep(cur[0], c);
        dec[1].prep(cur[1], c);
        if (kt + 1 < kt1) issue(kt + 1, buf ^ 1, nxt);
        const uint8_t *xb = xa + buf * XBUF;
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
            const bf16x8 B0 = dec[0].template step<S>();
            const bf16x8 B1 = dec[1].template step<S>();
#pragma unroll
            for (int i = 0; i < TM; i++) {
                acc[i][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[i], B0, acc[i][0], 0, 0, 0);
                acc[i][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[i], B1, acc[i][1], 0, 0, 0);
            }
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

    if (kt0 < kt1) issue(kt0, 0, raw[0]);
    for (int kt = kt0; kt < kt1; kt += 2) {
        body(kt, 0, raw[0], raw[1]);
        if (kt + 1 < kt1) body(kt + 1, 1, raw[1], raw[0]);
    }

    // ---- split-K: publish, then the last workgroup of the tile sums.
    if (a.splits > 1) {
        const int64_t tile = (int64_t)nt * a.m_tiles + mt;
        float *part = a.partials + tile * a.splits * (int64_t)TILEF + w * WAVEF + lane;
        float *own = part + (int64_t)ks * TILEF;
#pragma unroll
        for (int i = 0; i < TM; i++)
#pragma unroll
            for (int j = 0; j < 2; j++)
#pragma unroll
                for (int r = 0; r < 16; r++)
                    __hip_atomic_store(own + ((i * 2 + j) * 16 + r) * 64, acc[i][j][r],
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);  // keep the stores above the wait
        __builtin_amdgcn_s_waitcnt(0);            // this wave's stores are complete
        __syncthreads();
        if (tid == 0) {
            const unsigned prev = __hip_atomic_fetch_add(a.counters + tile, 1u, __ATOMIC_RELAXED,
                                                         __HIP_MEMORY_SCOPE_AGENT);
            s_last = prev == (unsigned)a.splits - 1 ? 1 : 0;
        }
        __syncthreads();
        if (!s_last) return;
#pragma unroll
        for (int i = 0; i < TM; i++)
#pragma unroll
            for (int j = 0; j < 2; j++)
#pragma unroll
                for (int r = 0; r < 16; r++) {
                    const float *p = part + ((i * 2 + j) * 16 + r) * 64;
                    float s = 0.f;
                    for (int k = 0; k < a.splits; k++)
                        s += __hip_atomic_load(p + (int64_t)k * TILEF, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
                    acc[i][j][r] = s;
                }
        if (tid == 0)  // ready for the next call
            __hip_atomic_store(a.counters + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    // ---- epilogue: accumulator register r of lane l is token
    // 8 (r / 4) + 4 h + r % 4 of the 32-token slice, column l % 32
#pragma unroll
    for (int i = 0; i < TM; i++)
#pragma unroll
        for (int r = 0; r < 16; r++) {
            const int64_t m = m0 + 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
            if (m >= M) continue;
            if constexpr (FFN) {
                if (nrow[0] >= N) continue;
                const float g = acc[i][0][r], u = acc[i][1][r];
                const int64_t o = m * N + nrow[0];
                a.H[o] = f32_to_bf16(act_apply(a.act, g) * u);
                if (a.g_out) a.g_out[o] = g;
                if (a.u_out) a.u_out[o] = u;
            } else {
#pragma unroll
                for (int j = 0; j < 2; j++)
                    if (nrow[j] < N) a.Y[m * N + nrow[j]] = acc[i][j][r];
            }
        }
}

template <int FMT, bool FFN>
hipError_t launch_f(int tm, const GemmArgs &a, hipStream_t st) {
    const int64_t grid = (int64_t)a.m_tiles * a.n_tiles * a.splits;
    if (grid <= 0 || grid > 0x7FFFFFFF) return hipErrorInvalidValue;
    if (tm == 4)
        hipLaunchKernelGGL((gemm_kernel<FMT, FFN, 4>), dim3((unsigned)grid), dim3(kThreads), 0, st, a);
    else if (tm == 2)
        hipLaunchKernelGGL((gemm_kernel<FMT, FFN, 2>), dim3((unsigned)grid), dim3(kThreads), 0, st, a);
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
