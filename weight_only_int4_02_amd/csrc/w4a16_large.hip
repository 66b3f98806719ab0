// Large-M kernel of libw4a16 (compute-bound): fp16 MFMA tiles with fp32
// accumulation, the int4 weight dequantized in registers.
//
// The Marlin post ("KPD" Telegram channel) describes large-batch int4 GEMM as
// compute-bound: the matrix units must be kept busy while weights are
// dequantized, with weights prefetched and loaded asynchronously and each
// activation tile used many times.  Here, for CDNA4:
//   * workgroup = WM x WN waves; wave tile (16 TM) x 64 outputs, TM x 4 tiles
//     of v_mfma_f32_16x16x32_f16 with fp32 accumulators;
//   * each 128-column step of K is one stage: the activation tile (BM rows)
//     and the packed weight tile (BN rows, 4 bits each) are copied HBM -> LDS
//     by the buffer-to-LDS DMA of gfx950 (buffer_load_dwordx4 ... lds), with
//     no register round trip, into a ring of NBUF stages -- stage kt + NBUF - 1
//     is in flight while stage kt is multiplied (one barrier per stage);
//   * in LDS both operands are kept in MFMA fragment order: a 1 KiB block per
//     (16-row tile, 32-column step), lane L's 16 bytes at L * 16, which is
//     exactly what lane L feeds the MFMA -- every LDS read is one conflict-free
//     ds_read_b128, with no padding;
//   * each wave dequantizes its 64 weight columns from LDS into B operands
//     (w = RNE_fp16((q - z) * s), bit-exact), group constants prefetched one
//     stage ahead;
//   * workgroups are ordered so that neighbouring output tiles of one column
//     block run on the same XCD (one L2 each on MI355X).
// All global reads are bounds-checked buffer loads (out-of-range offsets read
// zeros), so ragged M, N and K edges need no branches.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "w4a16_gemm_kernels.hpp"
#include "w4a16_kernels.hpp"

namespace w4a16 {

namespace {

constexpr int kXcds = 8;  // MI355X: 8 XCDs, workgroups dealt round-robin

// s_waitcnt immediate that waits for vmcnt <= N only (gfx9 encoding: vmcnt in
// bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima).
template <int N>
constexpr int kVmcnt = (N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8);

__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rsrc, u4_t *lds_wave_base,
                                      uint32_t voffset) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rsrc, (__attribute__((address_space(3))) void *)lds_wave_base, 16, (int)voffset, 0, 0, 0);
}

template <int WM, int WN, int TM, int JPG, int NBUF>
__global__ __launch_bounds__(WM *WN * 64) void gemm_large_m_kernel(GemmArgs a, int tiles_m,
                                                                    int tiles_n) {
    constexpr int NW = WM * WN;
    constexpr int TN = 4;  // 16-row weight tiles per wave
    constexpr int NG = 4 / JPG;
    constexpr int BM = WM * TM * 16, BN = WN * TN * 16;
    constexpr int AFR = BM / 16 * 4;  // activation fragments (1 KiB) per stage
    constexpr int BFR = BN / 16;      // packed weight tiles (1 KiB) per stage
    constexpr int FR = AFR + BFR;
    __shared__ u4_t lds[NBUF][FR * 64];

    // XCD-aware order: launch slot b runs on XCD b % 8; each XCD gets a
    // contiguous range of output tiles, M-blocks fastest, so the workgroups
    // of one XCD share weight columns in its L2.
    const int per_xcd = (int)gridDim.x / kXcds;
    const int logical = ((int)blockIdx.x % kXcds) * per_xcd + (int)blockIdx.x / kXcds;
    if (logical >= tiles_m * tiles_n)
        return;
    const int mb = logical % tiles_m, nb = logical / tiles_m;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int r = lane & 15, i = lane >> 4;
    const int wm = wave % WM, wn = wave / WM;
    const int m0 = mb * BM;
    const int ntw = nb * BFR;          // first weight tile of the workgroup
    const int nt0 = ntw + wn * TN;     // first weight tile of this wave

    // buffer resources: the workgroup's activation rows and weight tiles,
    // the wave's scales and zeros
    const int rows = min(BM, a.M - m0);
    const __amdgpu_buffer_rsrc_t rx =
        make_rsrc((const _Float16 *)a.X + (int64_t)m0 * a.K, (uint32_t)(rows * a.K * 2));
    const int ntsw = min(BFR, a.NT - ntw);
    const __amdgpu_buffer_rsrc_t rq =
        make_rsrc(a.qd + (int64_t)ntw * a.KT * 64, (uint32_t)(ntsw * a.KT * 1024));
    // (per workgroup, so the resources stay uniform; a wave's tiles are
    // addressed by offset)
    const i4_t rs = make_desc(a.sd + (int64_t)ntw * a.G * 16, (uint32_t)(ntsw * a.G * 32));
    const i4_t rz =
        make_desc(a.sym ? (const void *)a.sd : (const void *)(a.zd + (int64_t)ntw * a.GW * 16),
                  a.sym ? 0u : (uint32_t)(ntsw * a.GW * 64));
    const uint32_t zsym = a.sym ? 8u : 0u;

    // (every helper lambda below is force-inlined: left out of line, the
    // accumulators and the prefetch ring would stay in scratch memory)
    // Stage copy: fragment f < AFR is activation block (16-row tile f / 4,
    // step f % 4); f >= AFR is packed weight tile f - AFR.  Wave w issues the
    // fragments w, w + NW, ...; one 64-lane DMA instruction per fragment.
    // (AFR and BFR are multiples of NW for every shape: no branches)
    static_assert(AFR % NW == 0 && BFR % NW == 0, "fragments split evenly over waves");
    auto issue = [&](int kt, int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int k = 0; k < AFR / NW; k++) {
            const int f = wave + NW * k;
            const int row = (f >> 2) * 16 + r;
            const int col = kt * 128 + 32 * (f & 3) + 8 * i;
            dma16(rx, &lds[buf][f * 64],
                  col < a.K ? (uint32_t)((row * a.K + col) * 2) : kOutOfRange);
        }
#pragma unroll
        for (int k = 0; k < BFR / NW; k++) {
            const int t = wave + NW * k;
            dma16(rq, &lds[buf][(AFR + t) * 64], (uint32_t)(((t * a.KT + kt) * 64 + lane) * 16));
        }
    };

    // group constants of the wave's weight tiles for one stage: raw scale
    // bits and the packed zero word, decoded only where they are used so
    // the loads stay in flight
    struct Meta {
        uint32_t sb[TN][NG], zw[TN];
        int zsh[NG];  // nibble shift of each group's zero in zw
    };
    // (the groups of one 128-column tile share one packed zero word: at most
    // four consecutive groups starting at a multiple of 4, clamped to G - 1)
    auto load_meta = [&](Meta &mt, int kt) __attribute__((always_inline)) {
#pragma unroll
        for (int t = 0; t < TN; t++) {
            int grp[NG];
#pragma unroll
            for (int q = 0; q < NG; q++) {
                grp[q] = (kt * 128 + 32 * JPG * q) / a.g;
                grp[q] = grp[q] < a.G ? grp[q] : a.G - 1;
                mt.sb[t][q] = load_u16_untracked(
                    rs, (uint32_t)((((wn * TN + t) * a.G + grp[q]) * 16 + r) * 2));
            }
            mt.zw[t] = load_u32_untracked(
                rz, (uint32_t)((((wn * TN + t) * a.GW + (grp[0] >> 3)) * 16 + r) * 4));
#pragma unroll
            for (int q = 0; q < NG; q++)
                mt.zsh[q] = 4 * (grp[q] & 7);
        }
    };

    f4_t acc[TM][TN];
#pragma unroll
    for (int x = 0; x < TM; x++)
#pragma unroll
        for (int y = 0; y < TN; y++)
            acc[x][y] = f4_t{0.f, 0.f, 0.f, 0.f};

    const uint32_t magic = fp16_1024_pair();
    auto compute = [&](const u4_t *st, const Meta &mt) __attribute__((always_inline)) {
        u4_t bw[TN];
#pragma unroll
        for (int t = 0; t < TN; t++)
            bw[t] = st[(AFR + wn * TN + t) * 64 + lane];
#pragma unroll
        for (int j = 0; j < 4; j++) {
            h8_t xa[TM];
#pragma unroll
            for (int mi = 0; mi < TM; mi++)
                xa[mi] = __builtin_bit_cast(h8_t, st[((wm * TM + mi) * 4 + j) * 64 + lane]);
#pragma unroll
            for (int t = 0; t < TN; t++) {
                const uint32_t z = ((mt.zw[t] >> mt.zsh[j / JPG]) & 0xFu) + zsym;
                const h8_t b = dequant_word(bw[t][j], zero_pair(z), scale_pair(mt.sb[t][j / JPG]),
                                            magic);
#pragma unroll
                for (int mi = 0; mi < TM; mi++)
                    acc[mi][t] = mfma16x16x32(xa[mi], b, acc[mi][t]);
            }
        }
    };

    // Ring of NBUF stages.  Per stage every wave issues MQ group-constant
    // loads and then DQ DMA copies (FR is a multiple of NW for every shape);
    // stage kt + NBUF - 1 is issued while stage kt is multiplied.  Before the
    // barrier of stage kt a wave waits until only the loads it issued after
    // its own copies of stage kt are outstanding: (NBUF - 2) stages of them.
    constexpr int DQ = FR / NW;
    constexpr int MQ = TN * (NG + 1);
    static_assert(FR % NW == 0, "every wave issues the same number of copies");
    // vmcnt counts up to 63; waiting for fewer outstanding loads than issued
    // after stage kt is merely conservative
    constexpr int AHEAD = (NBUF - 2) * (MQ + DQ) < 63 ? (NBUF - 2) * (MQ + DQ) : 63;
    // this workgroup's slice of K (all of it without a split): U stages,
    // stage u is 128-column tile kt0 + u
    const int kt0 = (int)blockIdx.z * a.kts;
    const int U = max(0, min(a.KT, kt0 + a.kts) - kt0);
    Meta meta[NBUF];
#pragma unroll
    for (int p = 0; p < NBUF - 1; p++)
        if (p < U) {
            load_meta(meta[p], kt0 + p);
            __builtin_amdgcn_sched_barrier(0);
            issue(kt0 + p, p);
            __builtin_amdgcn_sched_barrier(0);
        }

    // stage u lives in ring slot u % NBUF; the loop is unrolled NBUF times
    // so every slot index is a compile-time constant
    auto step = [&](int u, auto slot_c) __attribute__((always_inline)) {
        constexpr int slot = decltype(slot_c)::value;
        constexpr int next = (slot + NBUF - 1) % NBUF;
        __builtin_amdgcn_sched_barrier(0);
        if (u + NBUF - 2 < U)
            __builtin_amdgcn_s_waitcnt(kVmcnt<AHEAD>);
        else
            __builtin_amdgcn_s_waitcnt(kVmcnt<0>);
        // Stage u is in LDS (every wave waited above for its own copies)
        // and every wave is done reading stage u - 1 (its LDS reads fed its
        // MFMAs).  A bare s_barrier: __syncthreads() would add a workgroup
        // release fence, which waits for all outstanding LDS-DMA copies --
        // the later stages too -- and drains the ring.
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        if (u + NBUF - 1 < U) {
            load_meta(meta[next], kt0 + u + NBUF - 1);
            __builtin_amdgcn_sched_barrier(0);
            issue(kt0 + u + NBUF - 1, next);
        }
        __builtin_amdgcn_sched_barrier(0);
        compute(lds[slot], meta[slot]);
    };
    for (int u = 0; u < U; u += NBUF) {
        step(u, std::integral_constant<int, 0>{});
        if (u + 1 < U)
            step(u + 1, std::integral_constant<int, 1 % NBUF>{});
        if constexpr (NBUF > 2) {
            if (u + 2 < U)
                step(u + 2, std::integral_constant<int, 2 % NBUF>{});
        }
        if constexpr (NBUF > 3) {
            if (u + 3 < U)
                step(u + 3, std::integral_constant<int, 3 % NBUF>{});
        }
    }

    // epilogue: one RNE rounding to fp16, or with K split across
    // workgroups the fp32 partial sums of this slice (summed and rounded by
    // the reduce kernel)
    float *part = a.ws + (int64_t)blockIdx.z * a.M * a.N;
#pragma unroll
    for (int t = 0; t < TN; t++) {
        const int n = (nt0 + t) * 16 + r;
        if (n >= a.N)
            continue;
#pragma unroll
        for (int mi = 0; mi < TM; mi++)
#pragma unroll
            for (int rr = 0; rr < 4; rr++) {
                const int m = m0 + wm * TM * 16 + mi * 16 + 4 * i + rr;
                if (m >= a.M)
                    continue;
                if (a.splits == 1)
                    ((_Float16 *)a.Y)[(int64_t)m * a.N + n] = (_Float16)acc[mi][t][rr];
                else
                    part[(int64_t)m * a.N + n] = acc[mi][t][rr];
            }
    }
}

template <int WM, int WN, int TM, int NBUF, int JPG>
int launch_large_inst(const GemmArgs &a, hipStream_t st) {
    constexpr int BM = WM * TM * 16, BN = WN * 64;
    const int tiles_m = (a.M + BM - 1) / BM;
    const int tiles_n = (a.N + BN - 1) / BN;
    const int tiles = tiles_m * tiles_n;
    const int grid = (tiles + kXcds - 1) / kXcds * kXcds;
    hipLaunchKernelGGL((gemm_large_m_kernel<WM, WN, TM, JPG, NBUF>),
                       dim3((unsigned)grid, 1, (unsigned)a.splits), dim3(WM * WN * 64), 0, st, a,
                       tiles_m, tiles_n);
    return (int)hipGetLastError();
}

template <int WM, int WN, int TM, int NBUF>
int launch_large_jpg(const GemmArgs &a, hipStream_t st) {
    if (a.g == 32)
        return launch_large_inst<WM, WN, TM, NBUF, 1>(a, st);
    if (a.g == 64)
        return launch_large_inst<WM, WN, TM, NBUF, 2>(a, st);
    return launch_large_inst<WM, WN, TM, NBUF, 4>(a, st);
}

}  // namespace

int launch_large_m(const GemmArgs &a, const LargePlan &p, hipStream_t st) {
    int e;
    switch (p.shape) {
    case 0: e = launch_large_jpg<2, 2, 4, 3>(a, st); break;   // 128 x 128, 4 waves, 3 stages
    case 1: e = launch_large_jpg<2, 2, 8, 2>(a, st); break;   // 256 x 128, 4 waves, 2 stages
    case 2: e = launch_large_jpg<1, 4, 8, 3>(a, st); break;   // 128 x 256, 4 waves, 3 stages
    case 3: e = launch_large_jpg<2, 4, 4, 3>(a, st); break;   // 128 x 256, 8 waves, 3 stages
    case 4: e = launch_large_jpg<1, 2, 4, 4>(a, st); break;   //  64 x 128, 2 waves, 4 stages
    case 5: e = launch_large_jpg<1, 4, 4, 4>(a, st); break;   //  64 x 256, 4 waves, 4 stages
    case 7: e = launch_large_jpg<1, 4, 2, 3>(a, st); break;   //  32 x 256, 4 waves, 3 stages
    case 8: e = launch_large_jpg<1, 2, 2, 4>(a, st); break;   //  32 x 128, 2 waves, 4 stages
    case 9: e = launch_large_jpg<2, 2, 2, 4>(a, st); break;   //  64 x 128, 4 waves, 4 stages
    default: e = launch_large_jpg<2, 1, 4, 4>(a, st); break;  // 128 x  64, 2 waves, 4 stages
    }
    if (e || a.splits == 1)
        return e;
    return launch_splitk_reduce(a, st);
}

}  // namespace w4a16
