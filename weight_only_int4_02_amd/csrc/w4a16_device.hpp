// Device-side helpers shared by the gfx950 kernels of libw4a16.
//
// Unpacking four-bit codes straight into fp16 operands, exactly:
//   * a code q OR-ed into bits 0..3 of the fp16 pattern 0x6400 (1024.0) is the
//     fp16 value 1024 + q (the fp16 spacing between 1024 and 2048 is 1);
//   * a code q OR-ed into bits 4..7 of 0x6400 is 1024 + 16 q, and
//     fma(1024 + 16 q, 1/16, -(64 + z)) = q - z exactly (one rounding of an
//     exact small integer);
//   * (1024 + q) - (1024 + z) = q - z exactly.
// With two codes per 32-bit register (bits 0..3 and 16..19, or 4..7 and
// 20..23), a device-layout word of eight codes becomes the four fp16 pairs
// (q - z) of the MFMA operand with one shift, four AND/OR and four packed fp16
// add/fma instructions -- no per-code shifts.
//
// Dequantization w = RNE_fp16((q - z) * s) then takes one packed multiply per
// pair: the product of the exact integer q - z and s rounds once, as the
// definition asks.  (The fused q * s - z * s form is not used: it rounds twice.)
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

// Per-group constants of the unpack: (1024 + z) and -(64 + z) in both halves,
// and the group scale s in both halves.
struct ZeroPair {
    h2_t z1024;   // (1024 + z, 1024 + z)
    h2_t zn64;    // (-(64 + z), -(64 + z))
};

__device__ __forceinline__ ZeroPair zero_pair(uint32_t z) {
    ZeroPair p;
    p.z1024 = as_h2((0x6400u | z) * 0x00010001u);
    // -(64 + z) as fp16: sign (0x8000) | biased exponent of 64 (21 << 10 =
    // 0x5400) | fraction 1024 * z / 64 = 16 z.
    p.zn64 = as_h2((0xD400u | (z << 4)) * 0x00010001u);
    return p;
}

__device__ __forceinline__ h2_t scale_pair(uint32_t s_bits) {
    return as_h2(s_bits * 0x00010001u);
}

// The pattern 0x64006400 in a vector register the compiler cannot see
// through.  gfx9 VOP3 encodings take no literal constant, so with both the
// mask and this pattern as literals each AND/OR pair is compiled to a v_and
// and a v_or; with the pattern in a register (and the mask in a scalar
// register) it is one v_and_or_b32.  Take it once per kernel.
__device__ __forceinline__ uint32_t fp16_1024_pair() {
    uint32_t m;
    asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(m));
    return m;
}

// A device-layout word holds elements 0..7 of an 8-column chunk with element e
// in nibble (e >> 1) + 4 (e & 1).  Returns (q - z) of the eight elements as the
// fp16 operand of one lane (elements in order), exact.  `magic` is 0x64006400
// (fp16_1024_pair()).
__device__ __forceinline__ h8_t unpack_qz(uint32_t w, const ZeroPair &zp, uint32_t magic) {
    const h2_t sixteenth = as_h2(0x2C002C00u);  // 1/16 in both halves
    const uint32_t w8 = w >> 8;
    u4_t o;
    o.x = as_u32(as_h2((w & 0x000F000Fu) | magic) - zp.z1024);
    o.y = as_u32(__builtin_elementwise_fma(as_h2((w & 0x00F000F0u) | magic), sixteenth, zp.zn64));
    o.z = as_u32(as_h2((w8 & 0x000F000Fu) | magic) - zp.z1024);
    o.w = as_u32(__builtin_elementwise_fma(as_h2((w8 & 0x00F000F0u) | magic), sixteenth, zp.zn64));
    return __builtin_bit_cast(h8_t, o);
}

// RNE_fp16((q - z) * s) of the eight elements of a device-layout word.
__device__ __forceinline__ h8_t dequant_word(uint32_t w, const ZeroPair &zp, h2_t ss,
                                             uint32_t magic = 0x64006400u) {
    u4_t d = __builtin_bit_cast(u4_t, unpack_qz(w, zp, magic));
    u4_t o;
    o.x = as_u32(as_h2(d.x) * ss);
    o.y = as_u32(as_h2(d.y) * ss);
    o.z = as_u32(as_h2(d.z) * ss);
    o.w = as_u32(as_h2(d.w) * ss);
    return __builtin_bit_cast(h8_t, o);
}

__device__ __forceinline__ f4_t mfma16x16x32(h8_t a, h8_t b, f4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// ---- bfloat16 variant ------------------------------------------------------
// gfx950 has no packed bf16 arithmetic, so the bf16 weight is formed in fp32:
// each code converted from its byte (v_cvt_f32_ubyteN), q - z (exact), then
// (q - z) * s, exact in fp32 (a 5-bit integer times an 8-bit significand; a
// product past the fp32 range is past the bf16 range too), then one
// nearest-even rounding to bf16 (v_cvt_pk_bf16_f32): RNE_bf16((q - z) s),
// bit-exact, signed zeros and overflow included.  (fma(q, s, -z s) would
// save an instruction but overflows in z s and loses the sign of zero.)
typedef __bf16 bf8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits) {
    return __builtin_bit_cast(float, bits << 16);
}

// Element e of a device-layout word sits in nibble (e >> 1) + 4 (e & 1):
// with lo = w & 0x0F0F0F0F and hi = (w >> 4) & 0x0F0F0F0F, bytes 0 and 2 of lo
// hold elements 0 and 1, of hi 2 and 3; bytes 1 and 3 of lo hold 4 and 5, of
// hi 6 and 7.  s and zf = z in fp32.
__device__ __forceinline__ bf8_t dequant_word_bf16(uint32_t w, float s, float zf) {
    const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
    const float q[8] = {(float)(lo & 0xFFu),         (float)((lo >> 16) & 0xFFu),
                        (float)(hi & 0xFFu),         (float)((hi >> 16) & 0xFFu),
                        (float)((lo >> 8) & 0xFFu),  (float)(lo >> 24),
                        (float)((hi >> 8) & 0xFFu),  (float)(hi >> 24)};
    // each pair rounded to bf16 by one v_cvt_pk_bf16_f32 (nearest-even),
    // element 2p in the low half: written out so that the pairing never
    // depends on how the compiler schedules the surrounding code
    u4_t o;
#pragma unroll
    for (int p = 0; p < 4; p++) {
        const float a = (q[2 * p] - zf) * s, b = (q[2 * p + 1] - zf) * s;
        asm("v_cvt_pk_bf16_f32 %0, %1, %2" : "=v"(o[p]) : "v"(a), "v"(b));
    }
    return __builtin_bit_cast(bf8_t, o);
}

// 0x43004300 (bf16 128.0 in both halves) in a vector register, for
// v_and_or_b32 (see fp16_1024_pair).
__device__ __forceinline__ uint32_t bf16_128_pair() {
    uint32_t m;
    asm volatile("v_mov_b32 %0, 0x43004300" : "=v"(m));
    return m;
}

// The eight codes of a device-layout word as bf16 values 128 + q, in element
// order: pair p (elements 2p, 2p + 1) sits in nibbles p and p + 4, i.e. bits
// 0..3 of both halves of w >> 4p, which OR into the 7 mantissa bits of 128.0
// exactly.  `magic` is 0x43004300 (bf16_128_pair()).
__device__ __forceinline__ bf8_t unpack_q128_bf16(uint32_t w, uint32_t magic) {
    u4_t o;
    o.x = (w & 0x000F000Fu) | magic;
    o.y = ((w >> 4) & 0x000F000Fu) | magic;
    o.z = ((w >> 8) & 0x000F000Fu) | magic;
    o.w = ((w >> 12) & 0x000F000Fu) | magic;
    return __builtin_bit_cast(bf8_t, o);
}

__device__ __forceinline__ f4_t mfma16x16x32_bf16(bf8_t a, bf8_t b, f4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Stores one fp32 result as the output's 16-bit format (nearest-even).
template <bool BF>
__device__ __forceinline__ void store_out16(uint16_t *y, float v) {
    if constexpr (BF)
        *(__bf16 *)y = (__bf16)v;
    else
        *(_Float16 *)y = (_Float16)v;
}

}  // namespace w4a16
