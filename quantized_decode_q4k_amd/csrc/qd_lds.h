// qd_lds.h -- streaming bytes into LDS with global_load_lds_dwordx4 (1 KB of
// consecutive bytes per wave instruction, no registers), ordered by explicit
// waits.
//
// The copies are issued as inline assembly.  The compiler does not see them,
// so it neither waits for them in front of every later LDS access (which it
// does, draining the whole stream, for the builtin form when it cannot tell
// the addresses apart) nor counts them in its own waits; LDS reads and
// writes stay ordinary C++ with the compiler's usual lgkmcnt tracking.  The
// kernel orders copies and reads itself:
//   * vm_wait<N>()  at most N copies of this wave are outstanding; copies
//                   complete in issue order, so all but the last N issued
//                   have landed in LDS;
//   * lgkm_wait()   this wave's LDS reads and writes are complete (before a
//                   slot is refilled);
//   * block_sync()  lgkm_wait(), then a workgroup barrier that does not wait
//                   on outstanding copies.
// All carry a memory clobber, so no memory access moves across them.
#pragma once

#include "qd_device.h"

namespace qd {

// 32-bit LDS address of a pointer into shared memory.
QD_DEV uint32_t lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

// Copy 16 bytes per active lane from src (per lane) to LDS base + 16 * lane.
// base must be wave-uniform; M0 is saved and restored around the copy.
QD_DEV void lds_copy16(const void *src, uint32_t base) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "global_load_lds_dwordx4 %1, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(src), "s"(__builtin_amdgcn_readfirstlane(base))
        : "memory");
}

// The same copy with device-scope coherence (sc1): data another workgroup
// stored with device-scope stores earlier in the same launch.
QD_DEV void lds_copy16_coh(const void *src, uint32_t base) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "global_load_lds_dwordx4 %1, off sc1\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(src), "s"(__builtin_amdgcn_readfirstlane(base))
        : "memory");
}

// The same copy from a wave-uniform 64-bit base (scalar registers) plus a
// per-lane 32-bit byte offset voff: issuing it takes no vector ALU
// instruction.  No immediate offset is used: on an LDS-DMA load the
// instruction offset moves the LDS destination as well as the source.
QD_DEV void lds_copy16_s(const void *sbase, uint32_t voff, uint32_t base) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "global_load_lds_dwordx4 %1, %2\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(sbase), "s"(base)
        : "memory");
}

template <int N>
QD_DEV void vm_wait() {
    static_assert(N >= 0 && N < 64, "vmcnt field");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

QD_DEV void lgkm_wait() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

QD_DEV void block_sync() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Flags in LDS shared between the waves of a workgroup: a load that is
// executed every time (ds_read_b32) and a plain store (ds_write_b32).  The
// caller orders them against its other accesses with lgkm_wait / vm_wait and
// the compiler barrier after a poll.
QD_DEV int lds_poll(const int *p) {
    return __atomic_load_n((const __attribute__((address_space(3))) int *)p, __ATOMIC_RELAXED);
}
QD_DEV void lds_flag(int *p, int v) {
    __atomic_store_n((__attribute__((address_space(3))) int *)p, v, __ATOMIC_RELAXED);
}
// *p += v in LDS (ds_add_u32).
QD_DEV void lds_add(int *p, int v) {
    __atomic_fetch_add((__attribute__((address_space(3))) int *)p, v, __ATOMIC_RELAXED);
}
// Spin (with a short sleep between polls) until *p == v.
QD_DEV void lds_wait_eq(const int *p, int v) {
    while (lds_poll(p) != v) __builtin_amdgcn_s_sleep(1);
    asm volatile("" ::: "memory");
}
// Spin until *p >= v.
QD_DEV void lds_wait_ge(const int *p, int v) {
    while (lds_poll(p) < v) __builtin_amdgcn_s_sleep(1);
    asm volatile("" ::: "memory");
}

// Cross-lane sums with DPP (no LDS traffic).
// v + v of lane ^ 1, then ^ 2 (every lane of a quad gets the quad's sum).
QD_DEV float quad_sum(float v) {
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                       0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));  // [1,0,3,2]
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                       0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));  // [2,3,0,1]
    return v;
}
// Sum over each group of 8 lanes (every lane gets its group's sum).
QD_DEV float oct_sum(float v) {
    v = quad_sum(v);
    // row_half_mirror: lane i of each 8 reads lane 7 - i
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                       0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false));
    return v;
}
// Sum over the 64 lanes of a wave (uniform result).
QD_DEV float wave_total(float v) {
    v = oct_sum(v);
    // row_mirror: lane i of each 16 reads lane 15 - i (adds the other half-row)
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                       0, __builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false));
    float s = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
    s += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
    s += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
    s += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
    return s;
}

}  // namespace qd
