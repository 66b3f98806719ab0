// Device-side helpers shared by the gfx950 kernels of libw4a16.
//
// Dequantization w = RNE_fp16((q - z) * s) in packed fp16 arithmetic, exact
// up to the one rounding the definition has:
//   1. A 4-bit code q OR-ed into the low mantissa bits of fp16 1024.0 (0x6400)
//      is the fp16 value 1024 + q, exactly (the fp16 spacing at 1024 is 1).
//   2. (1024 + q) - (1024 + z) = q - z is exact (small integers).
//   3. (q - z) * s in fp16 rounds once, to nearest even -- the definition.
// Two codes are handled per 32-bit register (v_pk_add_f16, v_pk_mul_f16).
// The fused form q * s - z * s is deliberately not used: it rounds twice.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a16 {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ h2_t as_h2(uint32_t u) { return __builtin_bit_cast(h2_t, u); }
__device__ __forceinline__ uint32_t as_u32(h2_t v) { return __builtin_bit_cast(uint32_t, v); }

// fp16 pair (1024 + z, 1024 + z).
__device__ __forceinline__ h2_t zero_pair(uint32_t z) {
    return as_h2((0x6400u | z) * 0x00010001u);
}
// fp16 pair (s, s) from the scale's bit pattern.
__device__ __forceinline__ h2_t scale_pair(uint32_t s_bits) {
    return as_h2(s_bits * 0x00010001u);
}

// (q_lo - z) * s, (q_hi - z) * s for the nibbles at bits [sh, sh+4) and
// [sh+16, sh+20) of w.
__device__ __forceinline__ uint32_t dq_pair(uint32_t w, int sh, h2_t zz, h2_t ss) {
    h2_t v = as_h2(((w >> sh) & 0x000F000Fu) | 0x64006400u);
    v = (v - zz) * ss;
    return as_u32(v);
}

// One word of the device layout: element e in nibble (e >> 1) + 4 (e & 1), so
// nibbles i and i + 4 hold elements 2i and 2i + 1 -> 8 fp16 in K order, the
// operand order of one lane of v_mfma_f32_16x16x32_f16.
__device__ __forceinline__ h8_t dq_dev_word(uint32_t w, h2_t zz, h2_t ss) {
    u4_t o;
    o.x = dq_pair(w, 0, zz, ss);
    o.y = dq_pair(w, 4, zz, ss);
    o.z = dq_pair(w, 8, zz, ss);
    o.w = dq_pair(w, 12, zz, ss);
    return __builtin_bit_cast(h8_t, o);
}

__device__ __forceinline__ f4_t mfma16x16x32(h8_t a, h8_t b, f4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

}  // namespace w4a16
