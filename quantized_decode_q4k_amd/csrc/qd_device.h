// qd_device.h -- device helpers shared by the HIP kernels of this library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define QD_DEV __device__ __forceinline__

namespace qd {

// f16 bits in the low / high half of a dword -> fp32 (v_cvt_f32_f16, exact).
QD_DEV float f16_lo(uint32_t v) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xFFFFu));
}
QD_DEV float f16_hi(uint32_t v) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16));
}

// Signed byte k of v as fp32 (v_cvt_f32_i32 with a sign-extended byte select).
QD_DEV float sbyte(uint32_t v, int k) {
    return (float)(int)(int8_t)(v >> (8 * k));
}

// ({hi, lo} >> 8*s) & 0xffffffff: re-align a dword stream by s bytes.
QD_DEV uint32_t align_bytes(uint32_t hi, uint32_t lo, uint32_t s) {
    return __builtin_amdgcn_alignbyte(hi, lo, s);
}

// Byte permute: each selector byte 0..3 picks that byte of `table`.
QD_DEV uint32_t byte_lut(uint32_t table, uint32_t sel) {
    return __builtin_amdgcn_perm(0u, table, sel);
}

// Two bytes of v, each holding a value 0..15, as fp32 via the fp8 (e4m3)
// converter: a byte 0000bbbb is a subnormal (bbbb < 8) or the first normal
// binade (bbbb >= 8), and on both the encoded value is bbbb times the
// smallest subnormal.  So the conversion returns q * unit exactly, where
// unit = fp8_unit() (2^-9 for OCP e4m3).
QD_DEV float2 nib2_lo(uint32_t v) {  // bytes 0, 1
    auto r = __builtin_amdgcn_cvt_pk_f32_fp8((int)v, false);
    return make_float2(r[0], r[1]);
}
QD_DEV float2 nib2_hi(uint32_t v) {  // bytes 2, 3
    auto r = __builtin_amdgcn_cvt_pk_f32_fp8((int)v, true);
    return make_float2(r[0], r[1]);
}
QD_DEV float fp8_unit() { return __builtin_amdgcn_cvt_f32_fp8(1, 0); }
// 1 / fp8_unit() as a constant: gfx950's converter reads OCP e4m3, whose
// smallest subnormal is 2^-9 (a division by the converted value would not
// fold and costs a full-precision divide wherever it is used).
QD_DEV constexpr float fp8_inv_unit() { return 512.0f; }

// Activations in fp32 (the larql Gemma 3 table's GELU-tanh geglu; the Llama
// table's SiLU).
QD_DEV float gelu_tanh(float g) {
    const float k0 = 0.7978845608028654f;  // sqrt(2/pi)
    const float k1 = 0.044715f;
    return 0.5f * g * (1.0f + tanhf(k0 * fmaf(k1 * g, g * g, g)));
}
QD_DEV float silu(float g) { return g / (1.0f + expf(-g)); }
QD_DEV float act_apply(int act, float g) { return act == 1 ? silu(g) : gelu_tanh(g); }

// fp32 -> bf16 bits, round to nearest even (NaN -> quiet NaN).
QD_DEV uint16_t f32_to_bf16(float f) {
    uint32_t u = __builtin_bit_cast(uint32_t, f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Unaligned-safe 32-bit load of a 4-byte-aligned address.
QD_DEV uint32_t ld32(const uint8_t *p) { return *reinterpret_cast<const uint32_t *>(p); }

// 16-byte load of a 16-byte-aligned address.
QD_DEV uint4 ld128(const uint8_t *p) { return *reinterpret_cast<const uint4 *>(p); }

}  // namespace qd
