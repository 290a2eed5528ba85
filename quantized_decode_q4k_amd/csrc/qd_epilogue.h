// qd_epilogue.h -- row epilogue of a GEMV launch: the post-norm, residual and
// next-norm step that needs the whole output row (larql "Architecture ->
// Metal shader map", Gemma 3 table: post_attn_residual_norm_store after the
// O projection, post_ffn_norm_residual_add after the down projection), and
// the cross-workgroup hand-off it rests on.
//
// Every workgroup that completes a row tile of the projection p stores its
// rows into a buffer and counts itself on a device-scope counter: each
// thread releases its stores at agent scope, the workgroup synchronises,
// and one thread increments the counter with an acquire-release atomic.
// The workgroup that brings the count to the number of tiles acquires and
// forms, per batch column (every sum in a fixed order, so results do not
// depend on which workgroup finishes last):
//   y  = r + p * w1 / sqrt(mean(p^2) + eps)
//   y2 = y * w2 / sqrt(mean(y^2) + eps)            (when w2 is given)
// then returns the counter to zero for the next launch.
#pragma once

#include "qd_device.h"
#include "qd_internal.h"
#include "qd_lds.h"

namespace qd {

// Sum of v over the NT threads of the workgroup, the same value in every
// thread: per wave with cross-lane adds, then the wave totals in wave order.
// red: NT / 64 floats of LDS.
template <int NT>
QD_DEV float block_total(float v, float *red) {
    constexpr int NW = NT / 64;
    const float t = wave_total(v);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = t;
    __syncthreads();
    float s = red[0];
#pragma unroll
    for (int w = 1; w < NW; w++) s += red[w];
    __syncthreads();
    return s;
}

// Release this workgroup's global stores and count it on *ctr; true (in
// every thread) for the workgroup that completes the count of `total`,
// which has then acquired every counted workgroup's stores.  flag: one int
// of LDS.
template <int NT>
QD_DEV bool arrive_last(unsigned *ctr, unsigned total, int *flag) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned prev = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        *flag = prev == total - 1 ? 1 : 0;
    }
    __syncthreads();
    const bool last = *flag != 0;
    if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    return last;
}

// The row epilogue, called by every thread of a workgroup after it has
// stored the final p rows of the tiles it completed (p at pn.p).  y: the
// call's output [batch][N].  red: NT / 64 floats of LDS; flag: one int.
template <int NT>
QD_DEV void post_norm_tail(const PostNorm &pn, float *y, int batch, int64_t N, float *red, int *flag) {
    if (!arrive_last<NT>(pn.ctr, pn.tiles, flag)) return;
    const int tid = threadIdx.x;
    const float invN = 1.0f / (float)N;
    for (int b = 0; b < batch; b++) {
        const float *pb = pn.p + (int64_t)b * N;
        const float *rb = pn.r + (int64_t)b * N;
        float *yb = y + (int64_t)b * N;
        float ss = 0.f;
        for (int64_t n = tid; n < N; n += NT) ss = fmaf(pb[n], pb[n], ss);
        ss = block_total<NT>(ss, red);
        const float rinv = 1.0f / sqrtf(ss * invN + pn.eps);
        float ss2 = 0.f;
        for (int64_t n = tid; n < N; n += NT) {
            const float v = rb[n] + pb[n] * rinv * pn.w1[n];
            yb[n] = v;
            ss2 = fmaf(v, v, ss2);
        }
        if (pn.w2) {
            ss2 = block_total<NT>(ss2, red);
            const float rinv2 = 1.0f / sqrtf(ss2 * invN + pn.eps);
            float *y2b = pn.y2 + (int64_t)b * N;
            for (int64_t n = tid; n < N; n += NT) y2b[n] = yb[n] * rinv2 * pn.w2[n];
        }
    }
    if (tid == 0) __hip_atomic_store(pn.ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace qd
