// The two GEMM kernels of libw4a16 (gfx950), as templates.
//
// Both consume the "tile 16 x 128" device layout: one 1 KiB block per 16 weight
// rows x 128 columns, lane r + 16 i of a wave loading its 16 bytes with one
// 128-bit load; word j of the lane holds row r, columns 32 j + 8 i .. +7.
// That is the B operand of v_mfma_f32_16x16x32_f16 for MFMA step j (lane
// r + 16 i supplies column r, K-slots 8 i .. 8 i + 7), so weights go from HBM
// to the matrix unit without passing through LDS, and each MFMA step covers 32
// consecutive columns -- inside one quantization group for every g >= 32.
//
// Marlin's ideas (the "KPD" Telegram post) carried over, CDNA4 style:
// (1) prefetching -- every weight load of a pass is issued before the first
// MFMA; (2) activations used many times per load -- an activation fragment
// feeds the whole 16-column weight tile, and in the large-M kernel an LDS tile
// feeds 64 columns per wave; (4) dequantization interleaved with MFMA issue;
// (5) the wave/workgroup shape chosen per batch regime.
#pragma once
#include "w4a16_kernels.hpp"

namespace w4a16 {

// Scale bits and zero of row 16 nt + r for the group holding column k.
// Columns past K (ragged last tile) take the last group: their codes are 0 and
// their activations are masked to 0, so they contribute nothing.
__device__ __forceinline__ void group_consts(const GemmArgs &a, int64_t nt, int k, int r,
                                             uint32_t &s_bits, uint32_t &z) {
    int grp = k / a.g;
    grp = grp < a.G ? grp : a.G - 1;
    s_bits = a.sd[(nt * a.G + grp) * 16 + r];
    z = 8u;
    if (!a.sym)
        z = (a.zd[(nt * a.GW + (grp >> 3)) * 16 + r] >> (4 * (grp & 7))) & 0xFu;
}

__device__ __forceinline__ float half_bits_to_float(uint32_t bits) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}

// ---------------------------------------------------------------------------
// Small-M kernel (memory-bound).  One workgroup of W waves computes NB 16-row
// weight tiles (16 NB output columns) for MT 16-row activation tiles, over all
// of K.  Wave w takes the 128-column tiles w, w + W, w + 2W, ... in stages of
// U tiles; a stage is every load it needs (U x NB weight tiles of 1 KiB, the
// activation fragments, the group constants).  The stages are double
// buffered in registers: the loads of stage s + 1 are issued before stage s is
// computed, so each wave keeps up to 2 U NB KiB of weights in flight through
// its whole K range (the prefetching of the Marlin post, done with plain
// 128-bit loads).  One activation fragment feeds NB weight tiles: activation
// bytes per weight byte are M / (4 NB).  The waves' partial 16 x 16 tiles are
// summed in LDS and rounded once to fp16.  The MFMA does the
// multiply-accumulate even at M = 1 (rows past M are zero), leaving the VALU
// only the unpack.
//
// Scales are applied to fp32 group sums: the weight operand is the exact
// integer q - z (fp16) and y = sum_groups s * sum_k (q - z) x.  That is the
// exact product (q - z) * s rather than its fp16 rounding, so y differs from
// the rounded-weight product X . W by at most 2^-11 sum|x w| <= 4.9e-4 ||x||
// ||w|| (a quarter of the error bound), and not at all on exactly
// representable inputs.  JPG = MFMA steps (32 columns each) per group inside
// a tile: 1, 2 or 4 (g = 32, 64, >= 128).
// ---------------------------------------------------------------------------
// Bounds-checked buffer loads: an offset at or past the resource's byte size
// reads 0 without touching memory, so masked lanes and ragged edges need no
// branches, and the loads of a stage stay a straight sequence the compiler
// can keep in flight across the previous stage's MFMAs.
constexpr uint32_t kBufferWord3 = 0x00020000u;  // raw 32-bit buffer, gfx9 family
constexpr uint32_t kOutOfRange = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             (int)kBufferWord3);
}

template <int U, int NB, int MT, int JPG>
struct SmallStage {
    static constexpr int NG = 4 / JPG;  // groups per 128-column tile
    u4_t wq[U][NB];
    uint32_t sb[U][NB][NG], zv[U][NB][NG];
    h8_t xf[U][MT][4];
};

// Buffer resources of one workgroup: its NB weight tiles (with their scales
// and zeros) and its MT x 16 activation rows.
struct SmallRes {
    __amdgpu_buffer_rsrc_t q, s, z, x;
};

template <int W, int U, int NB, int MT, int JPG>
__device__ __forceinline__ void small_load(SmallStage<U, NB, MT, JPG> &st, const GemmArgs &a,
                                           const SmallRes &res, int kt0, int lane, int r, int i) {
    constexpr int NG = 4 / JPG;
    const uint32_t zsym = a.sym ? 8u : 0u;
#pragma unroll
    for (int u = 0; u < U; u++) {
        const int kt = kt0 + u * W;
#pragma unroll
        for (int b = 0; b < NB; b++) {
            const uint32_t qoff = (uint32_t)(((b * a.KT + kt) * 64 + lane) * 16);
            st.wq[u][b] = __builtin_bit_cast(u4_t, __builtin_amdgcn_raw_buffer_load_b128(res.q, qoff, 0, 0));
#pragma unroll
            for (int q = 0; q < NG; q++) {
                int grp = (kt * 128 + 32 * JPG * q) / a.g;
                grp = grp < a.G ? grp : a.G - 1;
                st.sb[u][b][q] = __builtin_amdgcn_raw_buffer_load_b16(
                    res.s, (uint32_t)(((b * a.G + grp) * 16 + r) * 2), 0, 0);
                const uint32_t zw = __builtin_amdgcn_raw_buffer_load_b32(
                    res.z, (uint32_t)(((b * a.GW + (grp >> 3)) * 16 + r) * 4), 0, 0);
                // symmetric: the zero resource is empty (zw == 0) and z = 8
                st.zv[u][b][q] = ((zw >> (4 * (grp & 7))) & 0xFu) + zsym;
            }
        }
#pragma unroll
        for (int t = 0; t < MT; t++)
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const int k = kt * 128 + 32 * j + 8 * i;
                const uint32_t off = (uint32_t)(((t * 16 + r) * a.K + k) * 2);
                st.xf[u][t][j] = __builtin_bit_cast(
                    h8_t, __builtin_amdgcn_raw_buffer_load_b128(res.x, k < a.K ? off : kOutOfRange, 0, 0));
            }
    }
}

template <int W, int U, int NB, int MT, int JPG>
__device__ __forceinline__ void small_compute(const SmallStage<U, NB, MT, JPG> &st,
                                              const GemmArgs &a, int kt0, f4_t (&acc)[NB][MT]) {
    constexpr int NG = 4 / JPG;
#pragma unroll
    for (int u = 0; u < U; u++) {
        if (kt0 + u * W >= a.KT)
            break;
#pragma unroll
        for (int b = 0; b < NB; b++)
#pragma unroll
            for (int q = 0; q < NG; q++) {
                const ZeroPair zp = zero_pair(st.zv[u][b][q]);
                f4_t tmp[MT];
#pragma unroll
                for (int jj = 0; jj < JPG; jj++) {
                    const int j = q * JPG + jj;
                    const h8_t w = unpack_qz(st.wq[u][b][j], zp);
#pragma unroll
                    for (int t = 0; t < MT; t++)
                        tmp[t] = mfma16x16x32(st.xf[u][t][j], w,
                                              jj == 0 ? f4_t{0.f, 0.f, 0.f, 0.f} : tmp[t]);
                }
                const float s = half_bits_to_float(st.sb[u][b][q]);
#pragma unroll
                for (int t = 0; t < MT; t++)
                    acc[b][t] += s * tmp[t];
            }
    }
}

template <int W, int U, int NB, int MT, int JPG>
__global__ __launch_bounds__(W * 64) void gemm_small_m_kernel(GemmArgs a) {
    __shared__ f4_t red[W][NB][MT][64];
    const int nt0 = (int)blockIdx.x * NB;
    const int mb = blockIdx.y;
    // the wave index is uniform across the wave: keep it (and every loop
    // bound derived from it) in scalar registers so the stage branches are
    // scalar and the loads of a stage stay in flight across them
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int r = lane & 15, i = lane >> 4;

    // this workgroup's slices of the weight, scales, zeros and activations
    const int nts = min(NB, a.NT - nt0);
    const int m_base = mb * MT * 16;
    const int rows = min(MT * 16, a.M - m_base);
    SmallRes res;
    res.q = make_rsrc(a.qd + (int64_t)nt0 * a.KT * 64, (uint32_t)(nts * a.KT * 1024));
    res.s = make_rsrc(a.sd + (int64_t)nt0 * a.G * 16, (uint32_t)(nts * a.G * 32));
    res.z = make_rsrc(a.sym ? (const void *)a.sd : (const void *)(a.zd + (int64_t)nt0 * a.GW * 16),
                      a.sym ? 0u : (uint32_t)(nts * a.GW * 64));
    res.x = make_rsrc((const _Float16 *)a.X + (int64_t)m_base * a.K, (uint32_t)(rows * a.K * 2));

    f4_t acc[NB][MT];
#pragma unroll
    for (int b = 0; b < NB; b++)
#pragma unroll
        for (int t = 0; t < MT; t++)
            acc[b][t] = f4_t{0.f, 0.f, 0.f, 0.f};

    // two register stages, W * U column tiles apart
    SmallStage<U, NB, MT, JPG> s0, s1;
    constexpr int STEP = W * U;
    int kt = wave;
    if (kt < a.KT)
        small_load<W>(s0, a, res, kt, lane, r, i);
    for (; kt < a.KT; kt += 2 * STEP) {
        const int kt1 = kt + STEP;
        if (kt1 < a.KT)
            small_load<W>(s1, a, res, kt1, lane, r, i);
        small_compute<W>(s0, a, kt, acc);
        if (kt1 >= a.KT)
            break;
        const int kt2 = kt1 + STEP;
        if (kt2 < a.KT)
            small_load<W>(s0, a, res, kt2, lane, r, i);
        small_compute<W>(s1, a, kt1, acc);
    }

#pragma unroll
    for (int b = 0; b < NB; b++)
#pragma unroll
        for (int t = 0; t < MT; t++)
            red[wave][b][t][lane] = acc[b][t];
    __syncthreads();
    constexpr int SLOTS = NB * MT * 64;
    for (int idx = threadIdx.x; idx < SLOTS; idx += W * 64) {
        const int b = idx / (MT * 64), t = (idx / 64) % MT, l = idx & 63;
        f4_t v = red[0][b][t][l];
#pragma unroll
        for (int w = 1; w < W; w++)
            v += red[w][b][t][l];
        const int n = (nt0 + b) * 16 + (l & 15);
        const int m0 = m_base + t * 16 + 4 * (l >> 4);
        if (n >= a.N)
            continue;
#pragma unroll
        for (int rr = 0; rr < 4; rr++) {
            const int m = m0 + rr;
            if (m < a.M)
                ((_Float16 *)a.Y)[(int64_t)m * a.N + n] = (_Float16)v[rr];
        }
    }
}

}  // namespace w4a16
