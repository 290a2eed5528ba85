// qd_gemv_i8.hip -- Q8_0 GEMV on int8-quantized activations (opt-in).
//
// What is computed: dotLLM PR #320's CPU Q8_0 path quantizes the activation
// row to Q8_0 form before an integer dot product (GemmQ8_0 on pre-quantized
// input).  Here, per run of 32 activations, d = max|x| / 127 and
// q = round(x / d) (fp32 division, halves away from zero; zeros for an
// all-zero run), and
//   y[b][n] = sum over runs j of dw[n][j] * dx[b][j] * sum_i qw[n][32j+i] * qx[b][32j+i],
// the inner sum an exact int32 from v_dot4_i32_i8 (four int8 products per
// instruction, so the weights are never converted to float).  This is a
// different result from the fp32 GEMV (the activations are rounded): it is
// held to the usual bound against the same quantized computation, and its
// distance from the fp32 GEMV is a separate, wider tolerance class.
//
// Mapping: q8quant_kernel quantizes x once (8 lanes per run of 32); each
// GEMV workgroup copies the codes and scales into LDS once, then takes row
// tiles strided over the grid; in a tile, lane groups of 4 lanes walk a
// row's superunits of 8 blocks (lane c takes blocks 2c and 2c+1, as the fp32
// kernels do, with the same alignment-safe block loads); P lane groups share
// a row and split its superunits, loading the next superunit before decoding
// the current one;
// the 4 * P lanes of a row are summed with cross-lane shuffles.  With K split
// across workgroups (grid.y slices), a workgroup stages only its slice of the
// codes and takes one row tile; the last of a tile's workgroups to finish sums
// the partials in slice order.
#include "qd_decode.h"

namespace qd {
namespace {

QD_DEV float row_sum(float v, int width) {
    for (int off = 1; off < width; off <<= 1) v += __shfl_xor(v, off);
    return v;
}

// Quantize x [runs][32] per run: 8 lanes per run, 4 values per lane; the
// run's max |x| from 3 cross-lane steps, then one correctly rounded fp32
// division per value and round half away from zero.
__global__ __launch_bounds__(kThreads) void q8quant_kernel(const float *__restrict__ x, int8_t *__restrict__ q,
                                                         float *__restrict__ d, int64_t runs) {
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;  // lane i: values 4i .. 4i+3
    const bool live = i < runs * 8;
    const float4 v = live ? reinterpret_cast<const float4 *>(x)[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    float amax = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
    amax = fmaxf(amax, __shfl_xor(amax, 1));
    amax = fmaxf(amax, __shfl_xor(amax, 2));
    amax = fmaxf(amax, __shfl_xor(amax, 4));  // the 8 lanes of a run are aligned in the wave
    const float dr = __fdiv_rn(amax, 127.0f);
    const int q0 = dr > 0.f ? (int)roundf(__fdiv_rn(v.x, dr)) : 0;
    const int q1 = dr > 0.f ? (int)roundf(__fdiv_rn(v.y, dr)) : 0;
    const int q2 = dr > 0.f ? (int)roundf(__fdiv_rn(v.z, dr)) : 0;
    const int q3 = dr > 0.f ? (int)roundf(__fdiv_rn(v.w, dr)) : 0;
    if (live) {
        reinterpret_cast<int *>(q)[i] = (q0 & 0xFF) | ((q1 & 0xFF) << 8) | ((q2 & 0xFF) << 16) | ((q3 & 0xFF) << 24);
        if ((i & 7) == 0) d[i >> 3] = dr;
    }
}

template <int B>
__global__ __launch_bounds__(kThreads) void q8act_kernel(Q8ActArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int tid = threadIdx.x;
    const int64_t K = a.K;
    const int nblk = (int)(K / 32);
    const int nsu = (nblk + 7) / 8;
    // K-slice kz of the row: superunits [su0, su1), activations [kb0, kb0 + klen)
    const int kz = blockIdx.y;
    const int su0 = kz * a.su_per, su1 = min(nsu, su0 + a.su_per);
    const int64_t kb0 = (int64_t)su0 * kSuper;
    const int64_t klen = min(K, (int64_t)su1 * kSuper) - kb0;  // a multiple of 32
    const int nbl = (int)(klen / 32);
    int8_t *xq = reinterpret_cast<int8_t *>(smem);                 // [B][klen]
    float *xd = reinterpret_cast<float *>(smem + a.off_scales);    // [B][nbl]

    // ---- stage this slice of the quantized activation columns
    const int n16 = (int)(klen / 16);
    for (int i = tid; i < B * n16; i += kThreads) {
        const int b = i / n16, j = i - b * n16;
        reinterpret_cast<int4 *>(xq + (int64_t)b * klen)[j] =
            reinterpret_cast<const int4 *>(a.q + (int64_t)b * K + kb0)[j];
    }
    for (int i = tid; i < B * nbl; i += kThreads) {
        const int b = i / nbl;
        xd[i] = a.d[(int64_t)b * nblk + 8 * su0 + (i - b * nbl)];
    }
    __syncthreads();

    // ---- row tiles of kGroups / P rows, strided over the grid (unsplit, the
    // grid is sized so that each workgroup's staging serves several tiles);
    // lane group grp, lane c; P groups per row
    const int c = tid & 3, grp = tid >> 2;
    const int P = a.p;
    const int rows_wg = kGroups / P;
    const int pi = grp - (grp / P) * P;
    for (int64_t base = (int64_t)blockIdx.x * rows_wg; base < a.N; base += (int64_t)gridDim.x * rows_wg) {
        const int64_t row = base + grp / P;
        float acc[B];
#pragma unroll
        for (int b = 0; b < B; b++) acc[b] = 0.f;
        if (row < a.N) {
            const uint8_t *rowp = a.W + row * a.row_bytes;
            RawQ80 cur, nxt;
            if (su0 + pi < su1) load_q80(cur, rowp, su0 + pi, c, nblk);  // blocks past the row: zeros, d = 0
            for (int t = su0 + pi; t < su1; t += P) {
                if (t + P < su1) load_q80(nxt, rowp, t + P, c, nblk);  // next superunit in flight
                const float2 dw = q80_d(cur);
                // slice-local block indexes (clamped blocks carry d = 0)
                const int ja = min(8 * t + 2 * c, nblk - 1) - 8 * su0;
                const int jb = min(8 * t + 2 * c + 1, nblk - 1) - 8 * su0;
#pragma unroll
                for (int b = 0; b < B; b++) {
                    const int *xa = reinterpret_cast<const int *>(xq + (int64_t)b * klen + 32 * ja);
                    const int *xb = reinterpret_cast<const int *>(xq + (int64_t)b * klen + 32 * jb);
                    int sa = 0, sb = 0;
#pragma unroll
                    for (int k = 0; k < 8; k++) {
                        const uint2 v = q80_qdwords(cur, k);
                        sa = __builtin_amdgcn_sdot4((int)v.x, xa[k], sa, false);
                        sb = __builtin_amdgcn_sdot4((int)v.y, xb[k], sb, false);
                    }
                    acc[b] = fmaf(dw.x * xd[b * nbl + ja], (float)sa, acc[b]);
                    acc[b] = fmaf(dw.y * xd[b * nbl + jb], (float)sb, acc[b]);
                }
                cur = nxt;
            }
        }
#pragma unroll
        for (int b = 0; b < B; b++) {
            const float v = row_sum(acc[b], 4 * P);
            if (row < a.N && pi == 0 && c == 0) {
                if (a.ks == 1)
                    a.y[(int64_t)b * a.N + row] = v;
                else  // device-scope store: visible to the last workgroup of the tile
                    __hip_atomic_store(a.partials + ((int64_t)kz * B + b) * a.N + row, v, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
    if (a.ks == 1) return;

    // ---- K split across workgroups (one row tile per workgroup): the last
    // of the tile's ks workgroups sums the partials in slice order.  Every
    // wave's partial stores complete before the workgroup bumps the counter.
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    __shared__ int s_last;
    if (tid == 0) {
        const unsigned prev = __hip_atomic_fetch_add(a.counters + blockIdx.x, 1u, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        s_last = prev == (unsigned)a.ks - 1 ? 1 : 0;
    }
    __syncthreads();
    if (!s_last) return;
    const int64_t tile0 = (int64_t)blockIdx.x * rows_wg;
    for (int e = tid; e < rows_wg * B; e += kThreads) {
        const int b = e / rows_wg;
        const int64_t r = tile0 + (e - b * rows_wg);
        if (r >= a.N) continue;
        float s0 = 0.f;
        for (int k = 0; k < a.ks; k++)
            s0 += __hip_atomic_load(a.partials + ((int64_t)k * B + b) * a.N + r, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT);
        a.y[(int64_t)b * a.N + r] = s0;
    }
    if (tid == 0)  // ready for the next launch
        __hip_atomic_store(a.counters + blockIdx.x, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

size_t q8act_lds_bytes(int batch, int64_t K) {
    const size_t q = ((size_t)batch * (size_t)K + 15) & ~(size_t)15;  // int8 values, then the scales
    return q + (size_t)batch * (size_t)(K / 32) * 4;
}

hipError_t launch_q8quant(const float *x, int8_t *q, float *d, int64_t runs, hipStream_t st) {
    const int64_t lanes = runs * 8;
    const unsigned grid = (unsigned)((lanes + kThreads - 1) / kThreads);
    hipLaunchKernelGGL(q8quant_kernel, dim3(grid), dim3(kThreads), 0, st, x, q, d, runs);
    return hipGetLastError();
}

hipError_t launch_q8act(const Q8ActArgs &a, int batch, unsigned grid, hipStream_t st) {
    const size_t lds = q8act_lds_bytes(batch, std::min<int64_t>(a.K, (int64_t)a.su_per * kSuper));
#define QD_Q8A(Bv)                                                                        \
    case Bv:                                                                              \
        hipLaunchKernelGGL((q8act_kernel<Bv>), dim3(grid, a.ks), dim3(kThreads), lds, st, a);  \
        break;
    switch (batch) {
        QD_Q8A(1) QD_Q8A(2) QD_Q8A(3) QD_Q8A(4) QD_Q8A(5) QD_Q8A(6) QD_Q8A(7) QD_Q8A(8)
    default: return hipErrorInvalidValue;
    }
#undef QD_Q8A
    return hipGetLastError();
}

}  // namespace qd
