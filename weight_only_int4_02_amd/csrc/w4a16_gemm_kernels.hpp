// The small-M GEMM kernel of libw4a16 (gfx950), as a template, and the
// buffer-load helpers both GEMM kernels use.
//
// Both kernels consume the "tile 16 x 128" device layout: one 1 KiB block per
// 16 weight rows x 128 columns, lane r + 16 i of a wave loading its 16 bytes
// with one 128-bit load; word j of the lane holds row r, columns 32 j + 8 i ..
// +7.  That is the B operand of v_mfma_f32_16x16x32_f16 for MFMA step j (lane
// r + 16 i supplies column r, K-slots 8 i .. 8 i + 7), and each MFMA step
// covers 32 consecutive columns -- inside one quantization group for every
// g >= 32.
//
// The Marlin post (the "KPD" Telegram channel) lists the ideas carried over:
// prefetching, asynchronous weight loads, activations used many times per
// load, dequantization interleaved with matrix instructions, and the wave
// configuration tuned per batch regime.
#pragma once
#include <type_traits>

#include "w4a16_kernels.hpp"

namespace w4a16 {

__device__ __forceinline__ float half_bits_to_float(uint32_t bits) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}

// ---------------------------------------------------------------------------
// Bounds-checked buffer loads.  An offset at or past the descriptor's byte
// size reads 0 without touching memory, so masked lanes and ragged edges need
// no branches.
// ---------------------------------------------------------------------------
constexpr uint32_t kBufferWord3 = 0x00020000u;  // raw 32-bit buffer, gfx9 family
constexpr uint32_t kOutOfRange = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             (int)kBufferWord3);
}

// The same descriptor as four scalar words, for inline assembly.
typedef int32_t i4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i4_t make_desc(const void *base, uint32_t bytes) {
    const uint64_t p = (uint64_t)base;
    return i4_t{(int32_t)(uint32_t)p, (int32_t)(uint32_t)(p >> 32), (int32_t)bytes,
                (int32_t)kBufferWord3};
}

// Loads the compiler does not track.  Their completion is the kernel's
// business: it waits with an explicit s_waitcnt whose count it knows (the
// loads it issued after the ones it needs), then "touches" the destination
// registers (reg_fence) so no consumer is scheduled above the wait.  Left to
// the compiler, the waits on loop-carried prefetch registers are
// conservative and drain the prefetch pipeline.
__device__ __forceinline__ uint32_t load_u16_untracked(i4_t desc, uint32_t voffset) {
    uint32_t v;
    asm volatile("buffer_load_ushort %0, %1, %2, 0 offen" : "=v"(v) : "v"(voffset), "s"(desc));
    return v;
}
__device__ __forceinline__ uint32_t load_u32_untracked(i4_t desc, uint32_t voffset) {
    uint32_t v;
    asm volatile("buffer_load_dword %0, %1, %2, 0 offen" : "=v"(v) : "v"(voffset), "s"(desc));
    return v;
}
__device__ __forceinline__ u4_t load_b128_untracked(i4_t desc, uint32_t voffset) {
    u4_t v;
    asm volatile("buffer_load_dwordx4 %0, %1, %2, 0 offen" : "=v"(v) : "v"(voffset), "s"(desc));
    return v;
}
// The same loads with a wave-uniform part of the offset in a scalar register
// and a constant in the instruction: per stage only the scalar changes, so a
// stage's loads cost no vector instructions for their addresses.  The
// per-lane vector offset carries the range check: a lane whose vector offset
// is kOutOfRange (or past the descriptor's size) reads 0.
template <int IMM>
__device__ __forceinline__ uint32_t load_u16_so(i4_t desc, uint32_t voffset, uint32_t soffset) {
    uint32_t v;
    asm volatile("buffer_load_ushort %0, %1, %2, %3 offen offset:%4"
                 : "=v"(v) : "v"(voffset), "s"(desc), "s"(soffset), "n"(IMM));
    return v;
}
template <int IMM>
__device__ __forceinline__ uint32_t load_u32_so(i4_t desc, uint32_t voffset, uint32_t soffset) {
    uint32_t v;
    asm volatile("buffer_load_dword %0, %1, %2, %3 offen offset:%4"
                 : "=v"(v) : "v"(voffset), "s"(desc), "s"(soffset), "n"(IMM));
    return v;
}
template <int IMM>
__device__ __forceinline__ u4_t load_b128_so(i4_t desc, uint32_t voffset, uint32_t soffset) {
    u4_t v;
    asm volatile("buffer_load_dwordx4 %0, %1, %2, %3 offen offset:%4"
                 : "=v"(v) : "v"(voffset), "s"(desc), "s"(soffset), "n"(IMM));
    return v;
}
// Buffer-to-LDS copy of 16 bytes per lane (buffer_load_dwordx4 ... lds):
// lane L's bytes land at lds_wave_base + 16 L.  Out-of-range lanes write 0.
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t rsrc, u4_t *lds_wave_base,
                                          uint32_t voffset) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rsrc, (__attribute__((address_space(3))) void *)lds_wave_base, 16, (int)voffset, 0, 0, 0);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt counts 0..63");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
template <typename T>
__device__ __forceinline__ void reg_fence(T &x) {
    asm volatile("" : "+v"(x));
}

// ---------------------------------------------------------------------------
// Small-M kernel (memory-bound).  One workgroup of W waves computes NB 16-row
// weight tiles (16 NB output columns) for MT 16-row activation tiles over all
// of K.  Wave w takes the 128-column tiles w, w + W, w + 2W, ...; one tile is
// one stage: its NB weight blocks (1 KiB each), the 4 MT activation fragments
// and the group constants, all issued as untracked buffer loads into a ring
// of D register stages.  Stage s + D - 1 is in flight while stage s is
// multiplied, and the wave waits for exactly the loads of stage s (vmcnt =
// the loads issued after them), so up to D - 1 stages of every wave stream
// from HBM at all times.  One activation fragment feeds NB weight tiles:
// activation bytes per weight byte are M / (4 NB).  The waves' partial 16 x 16
// tiles are summed in LDS and rounded once to fp16.  The MFMA does the
// multiply-accumulate even at M = 1 (rows past M read as zeros), leaving the
// VALU only the unpack.
//
// Scales are applied to fp32 group sums: the weight operand is the exact
// integer q - z (fp16) and y = sum_groups s * sum_k (q - z) x.  That is the
// exact product (q - z) * s rather than its fp16 rounding, so y differs from
// the rounded-weight product X . W by at most 2^-11 sum|x w| <= 4.9e-4 ||x||
// ||w|| (a quarter of the error bound), and not at all on exactly
// representable inputs.  JPG = MFMA steps (32 columns each) per group inside
// a tile: 1, 2 or 4 (g = 32, 64, >= 128).  BF: bfloat16 activations, scales
// and output, the same factoring with a 128 + q operand (small_compute).
// ---------------------------------------------------------------------------
template <int NB, int MT, int JPG, bool XL = false>
struct SmallStage {
    static constexpr int NG = 4 / JPG;  // groups per 128-column tile
    // the activation loads are 4 MT fragment loads, or (XL) 4 MT copies
    static constexpr int LOADS = NB + NB * NG + NB + 4 * MT;
    u4_t wq[NB];
    uint32_t sb[NB][NG];  // raw fp16 scale bits
    uint32_t zw[NB];      // packed zero word (the tile's groups share it)
    u4_t xf[XL ? 1 : MT][4];  // activation fragments (8 fp16 each); unused with XL
};

// Activations through LDS (XL).  Each wave copies its stage's activation
// rows (16 MT rows x 128 columns, 4 KiB per 16 rows) into its own slot of a
// ring in LDS with the buffer-to-LDS DMA, four whole rows (8 cache lines) per
// copy, and reads the MFMA fragments from there.  A fragment load straight
// from memory touches 16 half cache lines (one per row) for its 1 KiB, so the
// copies halve the texture unit's cache-line lookups for the activations,
// which bound this kernel from M = 32 on.  In a slot, row q's 16-byte chunk c
// sits at position c ^ (q % 16): a fragment read (16 rows, one chunk each)
// then touches every LDS bank once.  Only the wave that copied a slot reads
// it, after its own wait for the copies, so no barrier is needed.
struct SmallXL {
    __amdgpu_buffer_rsrc_t rx;  // the workgroup's activation rows
    u4_t *ring;                 // this wave's slots: D x MT x 256 u4_t
    uint32_t off[4];            // per-lane part of copy c's offset (by c % 4)
    int col[4];                 // copy c's column inside the tile (by c % 4)
};

struct SmallDesc {
    i4_t q, s, z, x;
};

// Per-lane (vector) parts of the load offsets, fixed for the whole kernel.
template <int NB, int MT>
struct SmallOffs {
    uint32_t q[NB], s[NB], z[NB], x[MT];
};

// Group of column col_in_tile of tile kt, clamped: columns past K take the
// last group; their codes and activations are 0.  The (at most four) groups of
// one tile start at a multiple of 4 and so share one packed zero word.
__device__ __forceinline__ int tile_group(const GemmArgs &a, int kt, int col_in_tile) {
    const int grp = (kt * 128 + col_in_tile) >> a.lg;
    return grp < a.G ? grp : a.G - 1;
}

// Issues the loads of tile kt into a stage.  MASKED: the tile reaches past K
// (the last tile when K % 128 != 0), so activation columns past K read 0.
template <bool MASKED, int NB, int MT, int JPG, bool XL>
__device__ __forceinline__ void small_issue(SmallStage<NB, MT, JPG, XL> &st, const GemmArgs &a,
                                            const SmallDesc &d, const SmallOffs<NB, MT> &o,
                                            int kt, int i, const SmallXL &xl, int xslot) {
    constexpr int NG = 4 / JPG;
    const uint32_t so_q = (uint32_t)kt * 1024u;
#pragma unroll
    for (int b = 0; b < NB; b++)
        st.wq[b] = load_b128_so<0>(d.q, o.q[b], so_q);
    uint32_t so_s[NG];
#pragma unroll
    for (int q = 0; q < NG; q++)
        so_s[q] = (uint32_t)tile_group(a, kt, 32 * JPG * q) * 32u;
    const uint32_t so_z = (uint32_t)(tile_group(a, kt, 0) >> 3) * 64u;
#pragma unroll
    for (int b = 0; b < NB; b++) {
#pragma unroll
        for (int q = 0; q < NG; q++)
            st.sb[b][q] = load_u16_so<0>(d.s, o.s[b], so_s[q]);
        st.zw[b] = load_u32_so<0>(d.z, o.z[b], so_z);
    }
    if constexpr (XL) {
        // copy c: rows 4 c .. 4 c + 3 of the stage, lane L row 4 c + L / 16
        u4_t *slot = xl.ring + xslot * MT * 256;
#pragma unroll
        for (int c = 0; c < 4 * MT; c++) {
            const uint32_t v = xl.off[c & 3] + (uint32_t)((4 * c * a.K + kt * 128) * 2);
            lds_dma16(xl.rx, slot + c * 64,
                      !MASKED || xl.col[c & 3] < a.K - kt * 128 ? v : kOutOfRange);
        }
        return;
    }
    const uint32_t so_x = (uint32_t)kt * 256u;
#pragma unroll
    for (int t = 0; t < MT; t++) {
        if constexpr (MASKED) {
            const int lim = a.K - kt * 128;  // columns of this tile inside K
            st.xf[t][0] = load_b128_so<0>(d.x, 8 * i < lim ? o.x[t] : kOutOfRange, so_x);
            st.xf[t][1] = load_b128_so<64>(d.x, 32 + 8 * i < lim ? o.x[t] : kOutOfRange, so_x);
            st.xf[t][2] = load_b128_so<128>(d.x, 64 + 8 * i < lim ? o.x[t] : kOutOfRange, so_x);
            st.xf[t][3] = load_b128_so<192>(d.x, 96 + 8 * i < lim ? o.x[t] : kOutOfRange, so_x);
        } else {
            st.xf[t][0] = load_b128_so<0>(d.x, o.x[t], so_x);
            st.xf[t][1] = load_b128_so<64>(d.x, o.x[t], so_x);
            st.xf[t][2] = load_b128_so<128>(d.x, o.x[t], so_x);
            st.xf[t][3] = load_b128_so<192>(d.x, o.x[t], so_x);
        }
    }
}

template <int NB, int MT, int JPG, bool XL>
__device__ __forceinline__ void small_fence(SmallStage<NB, MT, JPG, XL> &st) {
    constexpr int NG = 4 / JPG;
#pragma unroll
    for (int b = 0; b < NB; b++) {
        reg_fence(st.wq[b]);
        reg_fence(st.zw[b]);
#pragma unroll
        for (int q = 0; q < NG; q++)
            reg_fence(st.sb[b][q]);
    }
    if constexpr (!XL) {
#pragma unroll
        for (int t = 0; t < MT; t++)
#pragma unroll
            for (int j = 0; j < 4; j++)
                reg_fence(st.xf[t][j]);
    }
}

// magic: 0x64006400 (fp16) or 0x43004300 (bf16) in a vector register.
template <bool BF, int NB, int MT, int JPG, bool XL>
__device__ __forceinline__ void small_compute(const SmallStage<NB, MT, JPG, XL> &st,
                                              const GemmArgs &a, int kt, uint32_t magic,
                                              f4_t (&acc)[NB][MT], const u4_t *xslot, int r, int i) {
    // activation fragment (m-tile t, MFMA step j): from the stage's
    // registers, or (XL) row 16 t + r, chunk 4 j + i of the wave's LDS slot
    auto xfrag = [&](int t, int j) __attribute__((always_inline)) {
        if constexpr (XL)
            return xslot[(t * 16 + r) * 16 + ((4 * j + i) ^ r)];
        else
            return st.xf[t][j];
    };
    constexpr int NG = 4 / JPG;
    // symmetric: the zero descriptor is empty (the words read 0) and z = 8
    const uint32_t zsym = a.sym ? 8u : 0u;
    if constexpr (BF) {
        // bf16 (no packed bf16 arithmetic on gfx950): the weight operand is
        // 128 + q, exact in bf16 (the 0x4300 pattern with the code OR-ed into
        // the low mantissa bits), so the MFMA yields sum (128 + q) x; a second
        // MFMA chain over the same activations with the constant operand
        // 128 + z yields sum (128 + z) x, and the group scale multiplies the
        // difference: y = sum_groups s * (sum (128 + q) x - sum (128 + z) x).
        // That is the exact (q - z) s rather than its bf16 rounding, up to
        // fp32 rounding of the two sums; where q = z throughout a group both
        // chains see identical operands, so a zero weight group adds exactly 0.
#pragma unroll
        for (int q = 0; q < NG; q++) {
            const int zsh = 4 * (tile_group(a, kt, 32 * JPG * q) & 7);
#pragma unroll
            for (int b = 0; b < NB; b++) {
                const float s = bf16_bits_to_float(st.sb[b][q]);
                const uint32_t zpair = (0x4300u + ((st.zw[b] >> zsh) & 0xFu) + zsym) * 0x10001u;
                const bf8_t zop = __builtin_bit_cast(bf8_t, u4_t{zpair, zpair, zpair, zpair});
                f4_t tmp[MT], zx[MT];
#pragma unroll
                for (int jj = 0; jj < JPG; jj++) {
                    const int j = q * JPG + jj;
                    const bf8_t w = unpack_q128_bf16(st.wq[b][j], magic);
#pragma unroll
                    for (int t = 0; t < MT; t++) {
                        const bf8_t xv = __builtin_bit_cast(bf8_t, xfrag(t, j));
                        tmp[t] = mfma16x16x32_bf16(xv, w, jj == 0 ? f4_t{0.f, 0.f, 0.f, 0.f} : tmp[t]);
                        zx[t] = mfma16x16x32_bf16(xv, zop, jj == 0 ? f4_t{0.f, 0.f, 0.f, 0.f} : zx[t]);
                    }
                }
#pragma unroll
                for (int t = 0; t < MT; t++)
#pragma unroll
                    for (int e = 0; e < 4; e++)
                        acc[b][t][e] += s * (tmp[t][e] - zx[t][e]);
            }
        }
        return;
    }
#pragma unroll
    for (int q = 0; q < NG; q++) {
        const int zsh = 4 * (tile_group(a, kt, 32 * JPG * q) & 7);
#pragma unroll
        for (int b = 0; b < NB; b++) {
            const ZeroPair zp = zero_pair(((st.zw[b] >> zsh) & 0xFu) + zsym);
            f4_t tmp[MT];
#pragma unroll
            for (int jj = 0; jj < JPG; jj++) {
                const int j = q * JPG + jj;
                const h8_t w = unpack_qz(st.wq[b][j], zp, magic);
#pragma unroll
                for (int t = 0; t < MT; t++)
                    tmp[t] = mfma16x16x32(__builtin_bit_cast(h8_t, xfrag(t, j)), w,
                                          jj == 0 ? f4_t{0.f, 0.f, 0.f, 0.f} : tmp[t]);
            }
            const float s = half_bits_to_float(st.sb[b][q]);
#pragma unroll
            for (int t = 0; t < MT; t++)
                acc[b][t] += s * tmp[t];
        }
    }
}

// Runs step(s + k, slot k) for k = 0, 1, ... while s + k < S and k < D:
// one pass of a D-stage ring with every slot index a compile-time constant.
template <int D, int K = 0, typename F>
__device__ __forceinline__ void ring_pass(int s, int S, F &&step) {
    if constexpr (K < D) {
        if (s + K < S) {
            step(s + K, std::integral_constant<int, K>{});
            ring_pass<D, K + 1>(s, S, step);
        }
    }
}

// Wait until at most `after` stages of loads (issued after the stage about to
// be used) are outstanding.  vmcnt counts to 63; a smaller count only waits
// longer.
template <int LPS, int D, int K = D - 1>
__device__ __forceinline__ void small_wait(int after) {
    if constexpr (K == 0) {
        wait_vmcnt<0>();
    } else {
        if (after >= K)
            wait_vmcnt<(K * LPS < 63 ? K * LPS : 63)>();
        else
            small_wait<LPS, D, K - 1>(after);
    }
}

template <int W, int NB, int MT, int JPG, int D, bool BF, bool XL = false>
__global__ __launch_bounds__(W * 64) void gemm_small_m_kernel(GemmArgs a) {
    static_assert(D >= 2 && D <= 12, "ring of 2..12 stages");
    using Stage = SmallStage<NB, MT, JPG, XL>;
    constexpr int LPS = Stage::LOADS;
    // Per wave: its part of the cross-wave sum ([NB][MT][64] f4_t, after
    // the last stage) and, with XL, its activation ring (D slots of MT x 4
    // KiB) before that, in the same bytes
    constexpr int RW = NB * MT * 64, XW = XL ? D * MT * 256 : 0;
    constexpr int PW = XW > RW ? XW : RW;  // u4_t per wave
    __shared__ u4_t smem[W * PW];
    const int nt0 = (int)blockIdx.x * NB;
    const int mb = blockIdx.y;
    // the wave index is uniform across the wave: keep it (and every loop
    // bound derived from it) in scalar registers
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int r = lane & 15, i = lane >> 4;

    // this workgroup's slices of the weight, scales, zeros and activations
    const int nts = min(NB, a.NT - nt0);
    const int m_base = mb * MT * 16;
    const int rows = min(MT * 16, a.M - m_base);
    SmallDesc d;
    d.q = make_desc(a.qd + (int64_t)nt0 * a.KT * 64, (uint32_t)(nts * a.KT * 1024));
    d.s = make_desc(a.sd + (int64_t)nt0 * a.G * 16, (uint32_t)(nts * a.G * 32));
    d.z = make_desc(a.sym ? (const void *)a.sd : (const void *)(a.zd + (int64_t)nt0 * a.GW * 16),
                    a.sym ? 0u : (uint32_t)(nts * a.GW * 64));
    d.x = make_desc((const _Float16 *)a.X + (int64_t)m_base * a.K, (uint32_t)(rows * a.K * 2));
    // Vector offsets.  Weight tiles past the last one (b >= nts) and
    // activation rows past M lie beyond their descriptors and read 0.
    SmallOffs<NB, MT> o;
#pragma unroll
    for (int b = 0; b < NB; b++) {
        o.q[b] = (uint32_t)((b * a.KT * 64 + lane) * 16);
        o.s[b] = (uint32_t)((b * a.G * 16 + r) * 2);
        o.z[b] = (uint32_t)((b * a.GW * 16 + r) * 4);
    }
#pragma unroll
    for (int t = 0; t < MT; t++)
        o.x[t] = (uint32_t)(((t * 16 + r) * a.K + 8 * i) * 2);
    // the exponent pattern the codes are OR-ed into: fp16 1024.0 or bf16 128.0
    const uint32_t magic = BF ? bf16_128_pair() : fp16_1024_pair();
    SmallXL xl;
    if constexpr (XL) {
        xl.ring = smem + wave * PW;
        xl.rx = make_rsrc((const _Float16 *)a.X + (int64_t)m_base * a.K, (uint32_t)(rows * a.K * 2));
#pragma unroll
        for (int c = 0; c < 4; c++) {
            // lane L: row 4 c + L / 16 of the copy's four, the chunk its
            // position L % 16 holds
            const int row = 4 * c + (lane >> 4);
            xl.col[c] = 8 * ((lane & 15) ^ (row & 15));
            xl.off[c] = (uint32_t)(((lane >> 4) * a.K + xl.col[c]) * 2);
        }
    }

    f4_t acc[NB][MT];
#pragma unroll
    for (int b = 0; b < NB; b++)
#pragma unroll
        for (int t = 0; t < MT; t++)
            acc[b][t] = f4_t{0.f, 0.f, 0.f, 0.f};

    // This workgroup's slice of K: tiles [kt_lo, kt_hi) (all of K without a
    // split).  The wave's full tiles (all 128 columns inside K) are
    // kt_lo + wave + W s, s < S; a last, partial tile is taken after the ring
    // by the wave it falls to.
    const int kt_lo = (int)blockIdx.z * a.kts;
    const int kt_hi = min(a.KT, kt_lo + a.kts);
    const int KTF = a.K >> 7;
    const int nfull = min(kt_hi, KTF) - kt_lo;
    const int S = nfull > wave ? (nfull - wave + W - 1) / W : 0;
    auto tile = [&](int s) __attribute__((always_inline)) { return kt_lo + wave + W * s; };
    // the wave's LDS activation slot for ring slot k (XL only)
    auto xslot = [&](int k) __attribute__((always_inline)) -> const u4_t * {
        if constexpr (XL)
            return xl.ring + k * MT * 256;
        else
            return nullptr;
    };
    Stage st[D];
#pragma unroll
    for (int p = 0; p < D - 1; p++)
        if (p < S)
            small_issue<false>(st[p], a, d, o, tile(p), i, xl, p);
    auto step = [&](int s, auto slot_c) __attribute__((always_inline)) {
        constexpr int slot = decltype(slot_c)::value;
        if (s + D - 1 < S)
            small_issue<false>(st[(slot + D - 1) % D], a, d, o, tile(s + D - 1), i, xl,
                               (slot + D - 1) % D);
        small_wait<LPS, D>(min(D - 1, S - 1 - s));
        small_fence(st[slot]);
        small_compute<BF>(st[slot], a, tile(s), magic, acc, xslot(slot), r, i);
    };
    for (int s = 0; s < S; s += D)
        ring_pass<D>(s, S, step);
    if (KTF < kt_hi && KTF >= kt_lo && wave == (KTF - kt_lo) % W) {
        small_issue<true>(st[0], a, d, o, KTF, i, xl, 0);
        wait_vmcnt<0>();
        small_fence(st[0]);
        small_compute<BF>(st[0], a, KTF, magic, acc, xslot(0), r, i);
    }

#pragma unroll
    for (int b = 0; b < NB; b++)
#pragma unroll
        for (int t = 0; t < MT; t++)
            ((f4_t *)(smem + wave * PW))[(b * MT + t) * 64 + lane] = acc[b][t];
    __syncthreads();
    constexpr int SLOTS = NB * MT * 64;
    for (int idx = threadIdx.x; idx < SLOTS; idx += W * 64) {
        const int b = idx / (MT * 64), t = (idx / 64) % MT, l = idx & 63;
        f4_t v = ((const f4_t *)smem)[(b * MT + t) * 64 + l];
#pragma unroll
        for (int w = 1; w < W; w++)
            v += ((const f4_t *)(smem + w * PW))[(b * MT + t) * 64 + l];
        const int n = (nt0 + b) * 16 + (l & 15);
        const int m0 = m_base + t * 16 + 4 * (l >> 4);
        if (n >= a.N)
            continue;
        if (a.splits == 1) {
#pragma unroll
            for (int rr = 0; rr < 4; rr++) {
                const int m = m0 + rr;
                if (m < a.M)
                    store_out16<BF>(a.Y + (int64_t)m * a.N + n, v[rr]);
            }
        } else {
            float *part = a.ws + (int64_t)blockIdx.z * a.M * a.N;
#pragma unroll
            for (int rr = 0; rr < 4; rr++) {
                const int m = m0 + rr;
                if (m < a.M)
                    part[(int64_t)m * a.N + n] = v[rr];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Small-M kernel with the activations and group constants in LDS (M <= 16,
// K not split across workgroups; fp16 or bf16 as gemm_small_m_kernel).  At the start the waves copy the
// X rows [M][K] and the scales and zero words of the workgroup's NB weight
// tiles from HBM into LDS with the buffer-to-LDS DMA; from then on a stage's
// only vector-memory loads are its NB weight blocks -- a plain weight stream
// -- and the activation fragments and group constants come from LDS.  Rows
// 16 > r >= M of the MFMA activation operand read row M - 1 (any finite data
// will do: row r of the product only feeds output row r, which is never
// stored).  Otherwise as gemm_small_m_kernel.
// ---------------------------------------------------------------------------
template <int W, int NB, int JPG, int D, bool BF>
__global__ __launch_bounds__(W * 64) void gemm_small_m_lds_kernel(GemmArgs a, int x_chunks,
                                                                  int s_chunks, int z_chunks) {
    static_assert(D >= 2 && D <= 12, "ring of 2..12 stages");
    constexpr int NG = 4 / JPG;
    constexpr int LPS = NB;  // vector-memory loads per stage: the weight blocks
    __shared__ f4_t red[W][NB][64];
    extern __shared__ u4_t lds[];  // 1 KiB chunks: X rows | scales | zero words
    const int nt0 = (int)blockIdx.x * NB;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int r = lane & 15, i = lane >> 4;
    const int nts = min(NB, a.NT - nt0);

    // the copy into LDS: chunk c (1 KiB) of the concatenated image, lane L
    // moving bytes 16 L .. 16 L + 15 of it; bytes past a region's end read 0
    {
        const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.X, (uint32_t)(a.M * a.K * 2));
        const __amdgpu_buffer_rsrc_t rs =
            make_rsrc(a.sd + (int64_t)nt0 * a.G * 16, (uint32_t)(nts * a.G * 32));
        const __amdgpu_buffer_rsrc_t rz = make_rsrc(
            a.sym ? (const void *)a.sd : (const void *)(a.zd + (int64_t)nt0 * a.GW * 16),
            a.sym ? 0u : (uint32_t)(nts * a.GW * 64));
        const int total = x_chunks + s_chunks + z_chunks;
        for (int c = wave; c < total; c += W) {
            if (c < x_chunks)
                lds_dma16(rx, &lds[c * 64], (uint32_t)(c * 1024 + lane * 16));
            else if (c < x_chunks + s_chunks)
                lds_dma16(rs, &lds[c * 64], (uint32_t)((c - x_chunks) * 1024 + lane * 16));
            else
                lds_dma16(rz, &lds[c * 64],
                          (uint32_t)((c - x_chunks - s_chunks) * 1024 + lane * 16));
        }
    }
    const uint16_t *s_lds = (const uint16_t *)&lds[x_chunks * 64];
    const uint32_t *z_lds = (const uint32_t *)&lds[(x_chunks + s_chunks) * 64];
    const int xrow = r < a.M ? r : a.M - 1;
    const u4_t *x_lds = &lds[(xrow * a.K + 8 * i) / 8];  // + (kt * 128 + 32 j) / 8

    const i4_t dq = make_desc(a.qd + (int64_t)nt0 * a.KT * 64, (uint32_t)(nts * a.KT * 1024));
    uint32_t oq[NB];
#pragma unroll
    for (int b = 0; b < NB; b++)
        oq[b] = (uint32_t)((b * a.KT * 64 + lane) * 16);
    const uint32_t magic = BF ? bf16_128_pair() : fp16_1024_pair();
    const uint32_t zsym = a.sym ? 8u : 0u;

    f4_t acc[NB];
#pragma unroll
    for (int b = 0; b < NB; b++)
        acc[b] = f4_t{0.f, 0.f, 0.f, 0.f};

    const int KTF = a.K >> 7;
    const int S = KTF > wave ? (KTF - wave + W - 1) / W : 0;
    auto tile = [&](int s) __attribute__((always_inline)) { return wave + W * s; };
    u4_t wq[D][NB];
    auto issue = [&](u4_t(&w)[NB], int kt) __attribute__((always_inline)) {
        const uint32_t so = (uint32_t)kt * 1024u;
#pragma unroll
        for (int b = 0; b < NB; b++)
            w[b] = load_b128_so<0>(dq, oq[b], so);
    };
    auto compute = [&](const u4_t(&w)[NB], int kt, bool masked) __attribute__((always_inline)) {
        u4_t xf[4];
#pragma unroll
        for (int j = 0; j < 4; j++)
            xf[j] = (masked && kt * 128 + 32 * j + 8 * i >= a.K) ? u4_t{0u, 0u, 0u, 0u}
                                                                 : x_lds[kt * 16 + 4 * j];
#pragma unroll
        for (int q = 0; q < NG; q++) {
            const int grp = tile_group(a, kt, 32 * JPG * q);
#pragma unroll
            for (int b = 0; b < NB; b++) {
                // (symmetric: no zero words were copied; z = 8)
                const uint32_t zw = a.sym ? 0u : z_lds[(b * a.GW + (grp >> 3)) * 16 + r];
                const uint32_t z = ((zw >> (4 * (grp & 7))) & 0xFu) + zsym;
                const uint32_t sbits = s_lds[(b * a.G + grp) * 16 + r];
                f4_t tmp;
                if constexpr (BF) {
                    // as in gemm_small_m_kernel: s * (sum (128 + q) x - sum (128 + z) x)
                    const uint32_t zpair = (0x4300u + z) * 0x10001u;
                    const bf8_t zop = __builtin_bit_cast(bf8_t, u4_t{zpair, zpair, zpair, zpair});
                    f4_t zx;
#pragma unroll
                    for (int jj = 0; jj < JPG; jj++) {
                        const int j = q * JPG + jj;
                        const bf8_t xv = __builtin_bit_cast(bf8_t, xf[j]);
                        const f4_t c0 = jj == 0 ? f4_t{0.f, 0.f, 0.f, 0.f} : tmp;
                        const f4_t c1 = jj == 0 ? f4_t{0.f, 0.f, 0.f, 0.f} : zx;
                        tmp = mfma16x16x32_bf16(xv, unpack_q128_bf16(w[b][j], magic), c0);
                        zx = mfma16x16x32_bf16(xv, zop, c1);
                    }
                    acc[b] += bf16_bits_to_float(sbits) * (tmp - zx);
                } else {
                    const ZeroPair zp = zero_pair(z);
#pragma unroll
                    for (int jj = 0; jj < JPG; jj++) {
                        const int j = q * JPG + jj;
                        tmp = mfma16x16x32(__builtin_bit_cast(h8_t, xf[j]),
                                           unpack_qz(w[b][j], zp, magic),
                                           jj == 0 ? f4_t{0.f, 0.f, 0.f, 0.f} : tmp);
                    }
                    acc[b] += half_bits_to_float(sbits) * tmp;
                }
            }
        }
    };

#pragma unroll
    for (int p = 0; p < D - 1; p++)
        if (p < S)
            issue(wq[p], tile(p));
    // the LDS image is complete once every wave's copies have landed: wait
    // for the copies (issued before the stage loads above), then a bare
    // barrier (__syncthreads would also wait for the stage loads)
    if (S >= D - 1)
        wait_vmcnt<(LPS * (D - 1) < 63 ? LPS * (D - 1) : 63)>();
    else
        wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");  // no LDS read moves above the barrier

    auto step = [&](int s, auto slot_c) __attribute__((always_inline)) {
        constexpr int slot = decltype(slot_c)::value;
        if (s + D - 1 < S)
            issue(wq[(slot + D - 1) % D], tile(s + D - 1));
        small_wait<LPS, D>(min(D - 1, S - 1 - s));
#pragma unroll
        for (int b = 0; b < NB; b++)
            reg_fence(wq[slot][b]);
        compute(wq[slot], tile(s), false);
    };
    for (int s = 0; s < S; s += D)
        ring_pass<D>(s, S, step);
    if (KTF < a.KT && wave == KTF % W) {
        issue(wq[0], KTF);
        wait_vmcnt<0>();
#pragma unroll
        for (int b = 0; b < NB; b++)
            reg_fence(wq[0][b]);
        compute(wq[0], KTF, true);
    }

#pragma unroll
    for (int b = 0; b < NB; b++)
        red[wave][b][lane] = acc[b];
    __syncthreads();
    for (int idx = threadIdx.x; idx < NB * 64; idx += W * 64) {
        const int b = idx / 64, l = idx & 63;
        f4_t v = red[0][b][l];
#pragma unroll
        for (int w = 1; w < W; w++)
            v += red[w][b][l];
        const int n = (nt0 + b) * 16 + (l & 15);
        const int m0 = 4 * (l >> 4);
        if (n >= a.N)
            continue;
#pragma unroll
        for (int rr = 0; rr < 4; rr++)
            if (m0 + rr < a.M)
                store_out16<BF>(a.Y + (int64_t)(m0 + rr) * a.N + n, v[rr]);
    }
}

}  // namespace w4a16
