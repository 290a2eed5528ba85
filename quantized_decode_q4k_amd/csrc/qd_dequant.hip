// qd_dequant.hip -- write out the dequantised weights (fp32, or bf16 rounded
// to nearest even) using the same lane decoders as the GEMV kernels, so that
// tests can check those decoders bit for bit against the CPU oracle.
//
// fp32 results are exact: for Q4_K the weight d*sc*q - dmin*m is formed with
// one fused multiply-add of exact fp32 factors (single rounding); Q6_K
// d*sc*(q-32) and Q8_0 d*q are exact products.
#include "qd_decode.h"

namespace qd {

template <int FMT, bool BF16>
__global__ __launch_bounds__(kThreads) void dequant_kernel(const uint8_t *W, float *out,
                                                           uint16_t *outb, int64_t N, int64_t K,
                                                           int64_t row_bytes, int nb, int nblk) {
    const int c = threadIdx.x & 3;
    const int64_t unit = (int64_t)blockIdx.x * kGroups + (threadIdx.x >> 2);
    if (unit >= N * nb) return;
    const int64_t n = unit / nb;
    const int t = (int)(unit - n * nb);
    const uint8_t *rowp = W + n * row_bytes;
    const int64_t obase = n * K + (int64_t)t * kSuper;

    auto put = [&](int idx, float w) {   // idx: weight index within the superunit
        if ((int64_t)t * kSuper + idx >= K) return;
        if constexpr (BF16) outb[obase + idx] = f32_to_bf16(w);
        else out[obase + idx] = w;
    };

    typename RawOf<FMT>::T r;
    load_unit<FMT>(r, rowp, t, c, nblk);
    if constexpr (FMT == kQ4K) {
        const Q4Scales s = q4k_scales(r, q4k_lane(c));
        const float inv_unit = fp8_inv_unit();
        const float a0 = s.d * s.sc0 * inv_unit, a1 = s.d * s.sc1 * inv_unit;
        const float b0 = -(s.dmin * s.m0), b1 = -(s.dmin * s.m1);
        for (int dw = 0; dw < 8; dw++) {
            const Q4Nibbles q = q4k_nibbles(r.q[dw]);
            const int lo = 64 * c + 4 * dw, hi = lo + 32;
            put(lo + 0, fmaf(a0, q.lo01.x, b0));
            put(lo + 1, fmaf(a0, q.lo01.y, b0));
            put(lo + 2, fmaf(a0, q.lo23.x, b0));
            put(lo + 3, fmaf(a0, q.lo23.y, b0));
            put(hi + 0, fmaf(a1, q.hi01.x, b1));
            put(hi + 1, fmaf(a1, q.hi01.y, b1));
            put(hi + 2, fmaf(a1, q.hi23.x, b1));
            put(hi + 3, fmaf(a1, q.hi23.y, b1));
        }
    } else if constexpr (FMT == kQ6K) {
        const int h = c >> 1, j = c & 1;
        const Q6Scales s = q6k_scales(r, j);
        for (int k = 0; k < 4; k++) {
            uint32_t q[4];
            q6k_qbytes(r, k, q);
            for (int g = 0; g < 4; g++) {
                const float ds = s.d * s.sc[g];
                const int base = 128 * h + 32 * g + 16 * j + 4 * k;
                for (int e = 0; e < 4; e++) put(base + e, ds * sbyte(q[g], e));
            }
        }
    } else {
        const float2 d = q80_d(r);
        for (int k = 0; k < 8; k++) {
            const uint2 v = q80_qdwords(r, k);
            for (int e = 0; e < 4; e++) {
                put(64 * c + 4 * k + e, d.x * sbyte(v.x, e));
                put(64 * c + 32 + 4 * k + e, d.y * sbyte(v.y, e));
            }
        }
    }
}

hipError_t launch_dequant(int fmt, const uint8_t *W, float *out, uint16_t *out_bf16, int64_t N,
                          int64_t K, hipStream_t st) {
    const int qk = fmt == kQ80 ? 32 : 256;
    const int bb = fmt == kQ4K ? 144 : (fmt == kQ6K ? 210 : 34);
    const int nblk = (int)(K / qk);
    const int nb = (int)((K + kSuper - 1) / kSuper);
    const int64_t row_bytes = (int64_t)nblk * bb;
    const int64_t units = N * nb;
    dim3 grid((unsigned)((units + kGroups - 1) / kGroups));
    const bool bf = out_bf16 != nullptr;
#define QD_DQ(F)                                                                              \
    if (bf) hipLaunchKernelGGL((dequant_kernel<F, true>), grid, dim3(kThreads), 0, st, W, out, \
                               out_bf16, N, K, row_bytes, nb, nblk);                           \
    else hipLaunchKernelGGL((dequant_kernel<F, false>), grid, dim3(kThreads), 0, st, W, out,   \
                            out_bf16, N, K, row_bytes, nb, nblk);
    switch (fmt) {
    case kQ4K: QD_DQ(kQ4K) break;
    case kQ6K: QD_DQ(kQ6K) break;
    case kQ80: QD_DQ(kQ80) break;
    default: return hipErrorInvalidValue;
    }
#undef QD_DQ
    return hipGetLastError();
}

}  // namespace qd
