// qd_epilogue.h -- row epilogue of a GEMV launch: the post-norm, residual and
// next-norm step that needs the whole output row (larql "Architecture ->
// Metal shader map", Gemma 3 table: post_attn_residual_norm_store after the
// O projection, post_ffn_norm_residual_add after the down projection), and
// the cross-workgroup hand-off it rests on.
//
// Every workgroup that completes a row tile of the projection p stores its
// rows into a buffer and counts itself on a device-scope counter; the
// workgroup that brings the count to the number of tiles forms, per batch
// column (every sum in a fixed order, so results do not depend on which
// workgroup finishes last):
//   y  = r + p * w1 / sqrt(mean(p^2) + eps)
//   y2 = y * w2 / sqrt(mean(y^2) + eps)            (when w2 is given)
// then returns the counter to zero for the next launch.
//
// Hand-off between workgroups.  Values that another workgroup of the same
// launch reads are stored and loaded as agent-scope atomics (xstore /
// xload): on gfx950 these are the device-coherent forms of the global
// store and load (scope bits set), so they neither leave a stale line in
// one XCD's L2 nor read one.  A workgroup counts itself only after every
// wave has waited for its own such stores to complete (s_waitcnt vmcnt(0)),
// so the count can reach the last workgroup only after the values have.
// This is what the compiler's release / acquire at agent scope would order,
// without its whole-L2 writeback and invalidate per wave, which measured
// about 15 us per hand-off under a running weight stream.
#pragma once

#include "qd_device.h"
#include "qd_internal.h"
#include "qd_lds.h"

namespace qd {

QD_DEV void xstore(float *p, float v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
QD_DEV float xload(const float *p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
// This wave's global stores (and loads) have completed.
QD_DEV void vm_drain() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

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

// Count this workgroup on *ctr once its xstore-d values have completed;
// true (in every thread) for the workgroup that completes the count of
// `total`, which then reads the others' values with xload.  flag: one int
// of LDS.
template <int NT>
QD_DEV bool arrive_last(unsigned *ctr, unsigned total, int *flag) {
    vm_drain();
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned prev = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *flag = prev == total - 1 ? 1 : 0;
    }
    __syncthreads();
    return *flag != 0;
}

// The row epilogue, called by every thread of a workgroup after it has
// stored (xstore) the final p rows of the tiles it completed (p at pn.p).  y: the
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
        for (int64_t n = tid; n < N; n += NT) {
            const float v = xload(pb + n);
            ss = fmaf(v, v, ss);
        }
        ss = block_total<NT>(ss, red);
        const float rinv = 1.0f / sqrtf(ss * invN + pn.eps);
        float ss2 = 0.f;
        for (int64_t n = tid; n < N; n += NT) {
            const float v = rb[n] + xload(pb + n) * rinv * pn.w1[n];
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
