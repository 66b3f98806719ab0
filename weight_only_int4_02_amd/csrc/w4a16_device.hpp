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

// Eight MFMAs acc[m] += a[m] b (m < 8) with the next weight word w
// dequantized in between (the arithmetic of dequant_word, bit-identical),
// returned as the next operand.  The vector instructions sit two or three
// after each MFMA, so a single wave keeps the matrix core busy while it
// unpacks: in the compiler's own order a word's unpack runs ahead of its
// MFMAs while the matrix core idles.
//
// FORM 0: as above.  FORM 2 (prefetch): right after MFMA m has read a[m],
// a[m] is refilled from LDS for the next MFMA step (ds_read_b128 of
// lds_next + 4096 m).  FORM 1 (wait): a was filled by such a prefetch, so
// MFMA m first waits until at most 7 - m LDS reads are outstanding (LDS
// reads complete in order; the prefetch issued its eight in order m =
// 0..7 and the caller issues no LDS read in between).
//
// Hazards: no vector write lands in a register an MFMA of the block reads
// (early clobbers); the returned operand's last write is two MFMAs before
// the block ends (the next block's first MFMA reads it); the caller puts
// wait states before a block whose b was written by compiled code.
// k: the masks 0x000F000F, 0x00F000F0 and 1/16 in both halves, in scalar
// registers.
struct UnpackConsts {
    uint32_t m0, m1, sixteenth;
};

#define W4_M(n) "v_mfma_f32_16x16x32_f16 %[c" #n "], %[a" #n "], %[b], %[c" #n "]\n"
#define W4_DQ_BLOCK(P0, S0, P1, S1, P2, S2, P3, S3, P4, S4, P5, S5, P6, S6, P7, S7)                \
    asm volatile(P0 W4_M(0) S0 P1 W4_M(1) S1                                                     \
                 "v_lshrrev_b32 %[t0], 8, %[w]\n"                                                \
                 "v_and_or_b32 %[t1], %[w], %[m0], %[mg]\n" P2 W4_M(2) S2                        \
                 "v_and_or_b32 %[t2], %[w], %[m1], %[mg]\n"                                      \
                 "v_and_or_b32 %[t3], %[t0], %[m0], %[mg]\n"                                     \
                 "v_and_or_b32 %[t0], %[t0], %[m1], %[mg]\n" P3 W4_M(3) S3                       \
                 "v_pk_add_f16 %[t1], %[t1], %[z1] neg_lo:[0,1] neg_hi:[0,1]\n"                  \
                 "v_pk_fma_f16 %[t2], %[t2], %[s16], %[zn]\n"                                    \
                 "v_pk_add_f16 %[t3], %[t3], %[z1] neg_lo:[0,1] neg_hi:[0,1]\n" P4 W4_M(4) S4    \
                 "v_pk_fma_f16 %[t0], %[t0], %[s16], %[zn]\n"                                    \
                 "v_pk_mul_f16 %[bn0], %[t1], %[ss]\n"                                           \
                 "v_pk_mul_f16 %[bn1], %[t2], %[ss]\n" P5 W4_M(5) S5                             \
                 "v_pk_mul_f16 %[bn2], %[t3], %[ss]\n"                                           \
                 "v_pk_mul_f16 %[bn3], %[t0], %[ss]\n" P6 W4_M(6) S6 P7 W4_M(7) S7               \
                 : [c0] "+v"(c0), [c1] "+v"(c1), [c2] "+v"(c2), [c3] "+v"(c3), [c4] "+v"(c4),    \
                   [c5] "+v"(c5), [c6] "+v"(c6), [c7] "+v"(c7), [bn0] "=&v"(bn0),                \
                   [bn1] "=&v"(bn1), [bn2] "=&v"(bn2), [bn3] "=&v"(bn3), [t0] "=&v"(t0),         \
                   [t1] "=&v"(t1), [t2] "=&v"(t2), [t3] "=&v"(t3), [a0] "+v"(a[0]),              \
                   [a1] "+v"(a[1]), [a2] "+v"(a[2]), [a3] "+v"(a[3]), [a4] "+v"(a[4]),           \
                   [a5] "+v"(a[5]), [a6] "+v"(a[6]), [a7] "+v"(a[7])                             \
                 : [b] "v"(b), [w] "v"(w), [z1] "v"(zp.z1024), [zn] "v"(zp.zn64), [ss] "v"(ss), \
                   [mg] "v"(magic), [m0] "s"(k.m0), [m1] "s"(k.m1), [s16] "s"(k.sixteenth),     \
                   [ln] "v"(lds_next))
#define W4_PF(m, off) "ds_read_b128 %[a" #m "], %[ln] offset:" #off "\n"
#define W4_WT(n) "s_waitcnt lgkmcnt(" #n ")\n"
template <int FORM>
__device__ __forceinline__ h8_t mfma8_dequant(f4_t &c0, f4_t &c1, f4_t &c2, f4_t &c3, f4_t &c4,
                                                f4_t &c5, f4_t &c6, f4_t &c7, h8_t (&a)[8],
                                                h8_t b, uint32_t w, const ZeroPair &zp, h2_t ss,
                                                uint32_t magic, const UnpackConsts &k,
                                                uint32_t lds_next) {
    uint32_t bn0, bn1, bn2, bn3, t0, t1, t2, t3;
    if constexpr (FORM == 0)
        W4_DQ_BLOCK("", "", "", "", "", "", "", "", "", "", "", "", "", "", "", "");
    else if constexpr (FORM == 1)
        W4_DQ_BLOCK(W4_WT(7), "", W4_WT(6), "", W4_WT(5), "", W4_WT(4), "", W4_WT(3), "",
                    W4_WT(2), "", W4_WT(1), "", W4_WT(0), "");
    else
        W4_DQ_BLOCK("", W4_PF(0, 0), "", W4_PF(1, 4096), "", W4_PF(2, 8192), "", W4_PF(3, 12288),
                    "", W4_PF(4, 16384), "", W4_PF(5, 20480), "", W4_PF(6, 24576), "",
                    W4_PF(7, 28672));
    return __builtin_bit_cast(h8_t, u4_t{bn0, bn1, bn2, bn3});
}
#undef W4_PF
#undef W4_WT
#undef W4_DQ_BLOCK
#undef W4_M

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


// The bf16 counterpart of mfma8_dequant: the eight MFMAs of one weight tile
// (v_mfma_f32_16x16x32_bf16) with the next word's bf16 dequantization --
// the same instructions as dequant_word_bf16, in its element order -- spread
// five or six after each of the first six MFMAs, and the same FORMs (0
// plain, 1 wait for the prefetched fragments, 2 prefetch the next step's
// fragments).  The last write of the returned operand is two MFMAs before
// the block ends; every temporary is an early clobber.  s and zf: the
// tile's scale and zero in fp32; m: 0x0F0F0F0F in a scalar register.
#define W4B_M(n) "v_mfma_f32_16x16x32_bf16 %[c" #n "], %[a" #n "], %[b], %[c" #n "]\n"
#define W4B_DQ_BLOCK(P0, S0, P1, S1, P2, S2, P3, S3, P4, S4, P5, S5, P6, S6, P7, S7)               \
    asm volatile(P0 W4B_M(0) S0                                                                  \
                 "v_and_b32 %[lo], %[m], %[w]\n"                                                 \
                 "v_lshrrev_b32 %[hi], 4, %[w]\n"                                                \
                 "v_and_b32 %[hi], %[m], %[hi]\n"                                                \
                 "v_cvt_f32_ubyte0 %[f0], %[lo]\n"                                               \
                 "v_cvt_f32_ubyte2 %[f1], %[lo]\n" P1 W4B_M(1) S1                                \
                 "v_cvt_f32_ubyte0 %[f2], %[hi]\n"                                               \
                 "v_cvt_f32_ubyte2 %[f3], %[hi]\n"                                               \
                 "v_cvt_f32_ubyte1 %[f4], %[lo]\n"                                               \
                 "v_cvt_f32_ubyte3 %[f5], %[lo]\n"                                               \
                 "v_cvt_f32_ubyte1 %[f6], %[hi]\n" P2 W4B_M(2) S2                                \
                 "v_cvt_f32_ubyte3 %[f7], %[hi]\n"                                               \
                 "v_sub_f32 %[f0], %[f0], %[zf]\n"                                               \
                 "v_sub_f32 %[f1], %[f1], %[zf]\n"                                               \
                 "v_sub_f32 %[f2], %[f2], %[zf]\n"                                               \
                 "v_sub_f32 %[f3], %[f3], %[zf]\n" P3 W4B_M(3) S3                                \
                 "v_sub_f32 %[f4], %[f4], %[zf]\n"                                               \
                 "v_sub_f32 %[f5], %[f5], %[zf]\n"                                               \
                 "v_sub_f32 %[f6], %[f6], %[zf]\n"                                               \
                 "v_sub_f32 %[f7], %[f7], %[zf]\n"                                               \
                 "v_mul_f32 %[f0], %[f0], %[s]\n" P4 W4B_M(4) S4                                 \
                 "v_mul_f32 %[f1], %[f1], %[s]\n"                                                \
                 "v_mul_f32 %[f2], %[f2], %[s]\n"                                                \
                 "v_mul_f32 %[f3], %[f3], %[s]\n"                                                \
                 "v_mul_f32 %[f4], %[f4], %[s]\n"                                                \
                 "v_mul_f32 %[f5], %[f5], %[s]\n" P5 W4B_M(5) S5                                 \
                 "v_mul_f32 %[f6], %[f6], %[s]\n"                                                \
                 "v_mul_f32 %[f7], %[f7], %[s]\n"                                                \
                 "v_cvt_pk_bf16_f32 %[bn0], %[f0], %[f1]\n"                                      \
                 "v_cvt_pk_bf16_f32 %[bn1], %[f2], %[f3]\n"                                      \
                 "v_cvt_pk_bf16_f32 %[bn2], %[f4], %[f5]\n"                                      \
                 "v_cvt_pk_bf16_f32 %[bn3], %[f6], %[f7]\n" P6 W4B_M(6) S6 P7 W4B_M(7) S7        \
                 : [c0] "+v"(c0), [c1] "+v"(c1), [c2] "+v"(c2), [c3] "+v"(c3), [c4] "+v"(c4),    \
                   [c5] "+v"(c5), [c6] "+v"(c6), [c7] "+v"(c7), [bn0] "=&v"(bn0),                \
                   [bn1] "=&v"(bn1), [bn2] "=&v"(bn2), [bn3] "=&v"(bn3), [lo] "=&v"(lo),         \
                   [hi] "=&v"(hi), [f0] "=&v"(f0), [f1] "=&v"(f1), [f2] "=&v"(f2),               \
                   [f3] "=&v"(f3), [f4] "=&v"(f4), [f5] "=&v"(f5), [f6] "=&v"(f6),               \
                   [f7] "=&v"(f7), [a0] "+v"(a[0]), [a1] "+v"(a[1]), [a2] "+v"(a[2]),            \
                   [a3] "+v"(a[3]), [a4] "+v"(a[4]), [a5] "+v"(a[5]), [a6] "+v"(a[6]),           \
                   [a7] "+v"(a[7])                                                               \
                 : [b] "v"(b), [w] "v"(w), [zf] "v"(zf), [s] "v"(s), [m] "s"(m),                 \
                   [ln] "v"(lds_next))
#define W4B_PF(m, off) "ds_read_b128 %[a" #m "], %[ln] offset:" #off "\n"
#define W4B_WT(n) "s_waitcnt lgkmcnt(" #n ")\n"
template <int FORM>
__device__ __forceinline__ h8_t mfma8_dequant_bf16(f4_t &c0, f4_t &c1, f4_t &c2, f4_t &c3,
                                                     f4_t &c4, f4_t &c5, f4_t &c6, f4_t &c7,
                                                     h8_t (&a)[8], h8_t b, uint32_t w, float s,
                                                     float zf, uint32_t m, uint32_t lds_next) {
    uint32_t bn0, bn1, bn2, bn3, lo, hi;
    float f0, f1, f2, f3, f4, f5, f6, f7;
    if constexpr (FORM == 0)
        W4B_DQ_BLOCK("", "", "", "", "", "", "", "", "", "", "", "", "", "", "", "");
    else if constexpr (FORM == 1)
        W4B_DQ_BLOCK(W4B_WT(7), "", W4B_WT(6), "", W4B_WT(5), "", W4B_WT(4), "", W4B_WT(3), "",
                     W4B_WT(2), "", W4B_WT(1), "", W4B_WT(0), "");
    else
        W4B_DQ_BLOCK("", W4B_PF(0, 0), "", W4B_PF(1, 4096), "", W4B_PF(2, 8192), "",
                     W4B_PF(3, 12288), "", W4B_PF(4, 16384), "", W4B_PF(5, 20480), "",
                     W4B_PF(6, 24576), "", W4B_PF(7, 28672));
    return __builtin_bit_cast(h8_t, u4_t{bn0, bn1, bn2, bn3});
}
#undef W4B_PF
#undef W4B_WT
#undef W4B_DQ_BLOCK
#undef W4B_M

// Stores one fp32 result as the output's 16-bit format (nearest-even).
template <bool BF>
__device__ __forceinline__ void store_out16(uint16_t *y, float v) {
    if constexpr (BF)
        *(__bf16 *)y = (__bf16)v;
    else
        *(_Float16 *)y = (_Float16)v;
}

}  // namespace w4a16
