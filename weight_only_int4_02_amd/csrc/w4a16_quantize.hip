// Round-to-nearest group quantizer of libw4a16 (gfx950): fp16 W [N][K] ->
// packed codes [N][K/8], fp16 scales [N][G], packed zeros [N][ceil(G/8)].
//
// It produces the group-wise 4-bit format the AWQ conversion of the lmdeploy
// PR "[Feature] Blazing fast W4A16 inference" feeds the GEMM (one scale and one
// zero per group of g consecutive K), and serves a K that is not a multiple of
// g with a partial last group (option 2 of the torchchat issue "linear:int4
// quantization regression testing"); since 0 always lies inside a group's
// range, padding K with zero columns instead gives the same codes, scales and
// zeros for the real columns.
//
// Floating point decides integers here (the codes), so every decision is made
// in fp32 with each operation rounded to nearest-even:
//   asymmetric: lo = min(0, min w), hi = max(0, max w) ([-1, 1] if both 0);
//     s = smallest fp16 >= (hi - lo) / 15;  z = clamp(rint(-lo / s), 0, 15)
//   symmetric:  s = smallest fp16 >= max|w| / 7 (max|w| = 1 if 0);  z = 8
//   q = clamp(rint(w / s) + z, 0, 15)      (rint: half to even)
// Rounding the scale up keeps every code within half a step of its weight.
//
// rint(w / s) without a division per weight: q0 = rint(w * r) with one
// reciprocal r = fp32(1 / s) per group is off by at most one step, and only
// where w / s is an exact half-integer that w * r misses.  The remainder
// w - q0 s is exact in one fma (w and s are fp16, |q0| < 2^5: the result
// needs at most 12 significant bits), so comparing it with s / 2 gives the
// nearest integer to the exact w / s with ties to even -- which is what rint
// of the correctly rounded fp32 quotient gives too, since for fp16 w and s
// that quotient lands on a half-integer only where the exact one does.
//
// One thread per 16 consecutive columns (two 16-byte loads, two packed words)
// and row; a block of 256 threads covers 4096 columns of one row, a whole
// number of groups (and of zero words) for every g in {32, 64, 128, 256}, and
// a thread issues both its loads before it uses either.  (Measured on the
// Llama-2 7B weights: one row per block 4911 GB/s, two 4835, four 4359, eight
// 3873.)
// A group's g/16 lanes are adjacent in one wave and reduce its range with
// lane shuffles, on packed fp16 pairs (exact: min and max do not round); the
// block's zeros are gathered in LDS and packed eight per word.  Each lane of a
// group computes the group's scale and zero (two divisions, the shuffles):
// with 16 columns a lane that work is shared by twice the weights of 8, which
// matters because the kernel issues about as many vector instructions as the
// chip can at the HBM rate.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "w4a16_device.hpp"
#include "w4a16_internal.hpp"

namespace w4a16 {

namespace {

constexpr int kQThreads = 256;
constexpr int kQWords = 2;                       // packed words per thread and row
constexpr int kQCols = kQThreads * 8 * kQWords;  // columns per block
constexpr int kQRows = 1;              // weight rows per block

__device__ __forceinline__ float f16_bits_to_f32(uint32_t b) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
}

// Smallest fp16 >= t, for t >= 0 (the conversion rounds to nearest-even;
// stepping the bit pattern up by one moves to the next fp16 above).
__device__ __forceinline__ uint32_t f16_round_up(float t) {
    uint32_t h = __builtin_bit_cast(uint16_t, (_Float16)t);
    if (f16_bits_to_f32(h) < t)
        h += 1;
    return h;
}

// rint(w / s), half to even, from r = fp32(1 / s): q0 = rint(w r), then the
// exact remainder w - q0 s moves q0 one step towards w where q0 is not the
// nearest integer, or is the odd one of an exact tie.
//
// The common case needs no remainder: |w r - w / s| <= 2^-19 for |w / s| <
// 16 (two roundings of relative size 2^-24 each), so where w r lies more
// than 2^-18 from a half-integer, rint(w r) is already the nearest integer to
// the exact quotient.  kNearTie is that distance from the rounding boundary.
constexpr float kNearTie = 0.5f - 0x1p-18f;

__device__ __forceinline__ int rtn_div(float w, float s, float r, float hs) {
    const float q0 = rintf(w * r);
    const float rem = __builtin_fmaf(-q0, s, w);
    const float a = __builtin_fabsf(rem);
    const int qi = (int)q0;
    const bool fix = a > hs || (a == hs && (qi & 1));
    return fix ? qi + (rem > 0.0f ? 1 : -1) : qi;
}

// A group's range on the packed fp16 weights: min and max of fp16 values are
// exact, so the range is taken two at a time on the raw words and carried as
// the pair (lo, -hi) -- one packed minimum per step of the shuffle reduction
// -- and widened to fp32 once.  Symmetric: (-amax, -amax) the same way.
__device__ __forceinline__ h2_t pk_min(h2_t a, h2_t b) { return __builtin_elementwise_min(a, b); }
__device__ __forceinline__ h2_t pk_max(h2_t a, h2_t b) { return __builtin_elementwise_max(a, b); }

template <int LPG, bool SYM>  // lanes per group = g / 16
__global__ __launch_bounds__(kQThreads) void quantize_kernel(
    const uint16_t *__restrict__ W, int64_t N, int64_t K, int64_t KB, int G, int GW,
    uint32_t *__restrict__ qp, uint16_t *__restrict__ scales, uint32_t *__restrict__ zeros) {
#pragma clang fp contract(off)
    constexpr int g = LPG * 8 * kQWords;
    constexpr int GB = kQCols / g;  // groups per block and row (a multiple of 8)
    constexpr int EL = 8 * kQWords;  // columns per thread
    __shared__ uint8_t zs[kQRows][GB];
    const int64_t nb = (int64_t)blockIdx.x / KB;
    const int64_t kb = (int64_t)blockIdx.x - nb * KB;
    const int t = threadIdx.x;
    const int64_t KW = K / 8;
    const int64_t word = (kb * kQThreads + t) * kQWords;  // the thread's first word
    bool valid[kQWords];
#pragma unroll
    for (int j = 0; j < kQWords; j++)
        valid[j] = word + j < KW;
    const int gib = t / LPG;  // group index inside the block
    const int64_t grp = kb * GB + gib;

    // the block's kQRows rows: every load issued before any is used, so each
    // thread has kQRows * kQWords 16-byte loads in flight
    u4_t raw[kQRows][kQWords];
#pragma unroll
    for (int rr = 0; rr < kQRows; rr++) {
        const int64_t n = nb * kQRows + rr;
#pragma unroll
        for (int j = 0; j < kQWords; j++)
            raw[rr][j] = (valid[j] && n < N) ? *(const u4_t *)(W + n * K + (word + j) * 8)
                                             : u4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int rr = 0; rr < kQRows; rr++) {
        const int64_t n = nb * kQRows + rr;
        // past K (or past N): zeros, neutral since 0 is inside every range
        float v[EL];
#pragma unroll
        for (int e = 0; e < EL; e++)
            v[e] = f16_bits_to_f32((raw[rr][e >> 3][(e >> 1) & 3] >> (16 * (e & 1))) & 0xFFFFu);
        // (lo, -hi) of the thread's weights and 0, or (-amax, -amax)
        h2_t m2;
        if constexpr (SYM) {
            h2_t a = __builtin_elementwise_abs(as_h2(raw[rr][0][0]));
#pragma unroll
            for (int i = 1; i < 4 * kQWords; i++)
                a = pk_max(a, __builtin_elementwise_abs(as_h2(raw[rr][i >> 2][i & 3])));
            const _Float16 am = a[0] > a[1] ? a[0] : a[1];
            m2 = h2_t{-am, -am};
        } else {
            h2_t l = as_h2(raw[rr][0][0]), h = l;
#pragma unroll
            for (int i = 1; i < 4 * kQWords; i++) {
                l = pk_min(l, as_h2(raw[rr][i >> 2][i & 3]));
                h = pk_max(h, as_h2(raw[rr][i >> 2][i & 3]));
            }
            m2 = pk_min(h2_t{l[0] < l[1] ? l[0] : l[1], -(h[0] > h[1] ? h[0] : h[1])},
                        h2_t{(_Float16)0.0f, (_Float16)0.0f});
        }
#pragma unroll
        for (int m = 1; m < LPG; m <<= 1)
            m2 = pk_min(m2, as_h2((uint32_t)__shfl_xor((int)as_u32(m2), m)));

        uint32_t sb;
        int z;
        float lo = 0.0f, hi = 0.0f;
        if constexpr (SYM) {
            const float amax = -(float)m2[0];
            sb = f16_round_up((amax == 0.0f ? 1.0f : amax) / 7.0f);
            z = 8;
        } else {
            lo = (float)m2[0];
            hi = -(float)m2[1];
            if (hi == lo) {
                lo = -1.0f;
                hi = 1.0f;
            }
            sb = f16_round_up((hi - lo) / 15.0f);
        }
        const float sf = f16_bits_to_f32(sb);
        const float r = 1.0f / sf;
        const float hs = 0.5f * sf;
        if constexpr (!SYM) {
            const int zr = rtn_div(-lo, sf, r, hs);
            z = zr < 0 ? 0 : (zr > 15 ? 15 : zr);
        }

        // rint(w r) for every weight, and whether any of them lies within
        // 2^-18 of a half-integer; only then (rare: exact ties and their
        // neighbours) the exact remainder decides
        int qi[EL];
        bool near = false;
#pragma unroll
        for (int e = 0; e < EL; e++) {
            const float t = v[e] * r;
            const float q0 = rintf(t);
            near |= __builtin_fabsf(t - q0) > kNearTie;
            qi[e] = (int)q0;
        }
        if (__builtin_expect(near, 0)) {
#pragma unroll
            for (int e = 0; e < EL; e++)
                qi[e] = rtn_div(v[e], sf, r, hs);
        }
        uint32_t packed[kQWords];
#pragma unroll
        for (int j = 0; j < kQWords; j++) {
            packed[j] = 0;
#pragma unroll
            for (int e = 0; e < 8; e++) {
                int q = qi[8 * j + e] + z;
                q = q < 0 ? 0 : (q > 15 ? 15 : q);
                packed[j] |= (uint32_t)q << (4 * e);
            }
        }
        if (n < N) {
            // the first word is valid whenever any is, and names the group
#pragma unroll
            for (int j = 0; j < kQWords; j++)
                if (valid[j])
                    qp[n * KW + word + j] = packed[j];
            if (valid[0] && t % LPG == 0)
                scales[n * G + grp] = (uint16_t)sb;
        }
        if (t % LPG == 0)
            zs[rr][gib] = (uint8_t)z;
    }
    if constexpr (SYM)
        return;
    __syncthreads();
    // zero words: GB / 8 per row and block
    constexpr int ZW = GB / 8;
    if (t < kQRows * ZW) {
        const int rr = t / ZW, w = t - rr * ZW;
        const int64_t n = nb * kQRows + rr;
        const int64_t zw = kb * ZW + w;
        if (n < N && zw < GW) {
            uint32_t word32 = 0;
#pragma unroll
            for (int e = 0; e < 8; e++)
                if (zw * 8 + e < G)
                    word32 |= (uint32_t)zs[rr][8 * w + e] << (4 * e);
            zeros[n * GW + zw] = word32;
        }
    }
}

}  // namespace

int launch_quantize(const uint16_t *W, const Geom &geo, uint32_t *qp, uint16_t *scales,
                    uint32_t *zeros, void *stream) {
    const int64_t KB = (geo.K / 8 + kQThreads * kQWords - 1) / (kQThreads * kQWords);
    const dim3 grid((unsigned)((geo.N + kQRows - 1) / kQRows * KB));
    hipStream_t st = (hipStream_t)stream;
    auto go = [&](auto lpg, auto sym) {
        hipLaunchKernelGGL((quantize_kernel<decltype(lpg)::value, decltype(sym)::value>), grid,
                           dim3(kQThreads), 0, st, W, geo.N, geo.K, KB, (int)geo.G, (int)geo.GW,
                           qp, scales, zeros);
    };
    auto by_g = [&](auto sym) {
        switch (geo.g) {
        case 32: go(std::integral_constant<int, 2>{}, sym); break;
        case 64: go(std::integral_constant<int, 4>{}, sym); break;
        case 128: go(std::integral_constant<int, 8>{}, sym); break;
        default: go(std::integral_constant<int, 16>{}, sym); break;
        }
    };
    if (geo.sym)
        by_g(std::true_type{});
    else
        by_g(std::false_type{});
    return (int)hipGetLastError();
}

}  // namespace w4a16
