// Large-M kernel of libw4a16 (compute-bound): fp16 MFMA tiles with fp32
// accumulation, the int4 weight dequantized in registers.
//
// The Marlin post ("KPD" Telegram channel) describes large-batch int4 GEMM as
// compute-bound: the matrix units must be kept busy while weights are
// dequantized, with prefetched, asynchronously loaded weights and activations
// reused many times.  Here, for CDNA4:
//   * workgroup = WM x WN waves, wave tile (16 TM) x 64 outputs
//     (TM x 4 tiles of v_mfma_f32_16x16x32_f16, fp32 accumulators);
//   * activation stages of 64 columns (two MFMA steps) are copied
//     global -> registers -> LDS, double buffered: the copy of stage s + 1 is
//     in flight while stage s is multiplied, one barrier per stage;
//   * weights are not staged: each wave loads the 16-byte lane chunks of its
//     four 16-row weight tiles for the next 128-column tile while the current
//     one is multiplied, and dequantizes them into MFMA B operands
//     (w = RNE_fp16((q - z) * s), bit-exact);
//   * workgroups are ordered so that neighbouring output tiles of one column
//     block run on the same XCD (one L2 each on MI355X).
// Loads are bounds-checked buffer loads (out-of-range offsets read 0): ragged
// M, N and K edges need no branches.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "w4a16_gemm_kernels.hpp"
#include "w4a16_kernels.hpp"

namespace w4a16 {

namespace {

constexpr int kXcds = 8;     // MI355X: 8 XCDs, workgroups dealt round-robin
constexpr int KS = 64;       // activation columns per LDS stage
constexpr int LDA = KS + 8;  // LDS row pitch in halves (16-byte pad)

template <int WM, int WN, int TM, int JPG>
__global__ __launch_bounds__(WM *WN * 64) void gemm_large_m_kernel(GemmArgs a, int tiles_m,
                                                                    int tiles_n) {
    constexpr int NW = WM * WN, NTHR = NW * 64;
    constexpr int TN = 4;  // 16-row weight tiles per wave
    constexpr int NG = 4 / JPG;
    constexpr int BM = WM * TM * 16, BN = WN * TN * 16;
    constexpr int CHUNKS = BM * KS / 8;  // 16-byte activation chunks per stage
    static_assert(CHUNKS % NTHR == 0, "stage copy must split evenly");
    constexpr int CPT = CHUNKS / NTHR;
    __shared__ _Float16 sa[2][BM * LDA];

    // XCD-aware order: launch slot b runs on XCD b % 8; give each XCD a
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
    const int nt0 = nb * (BN / 16) + wn * TN;  // first weight tile of this wave

    // buffer resources: the workgroup's activation rows, the wave's weight
    // tiles with their scales and zeros
    const int rows = min(BM, a.M - m0);
    const __amdgpu_buffer_rsrc_t rx =
        make_rsrc((const _Float16 *)a.X + (int64_t)m0 * a.K, (uint32_t)(rows * a.K * 2));
    const int nts = max(0, min(TN, a.NT - nt0));
    const __amdgpu_buffer_rsrc_t rq =
        make_rsrc(a.qd + (int64_t)min(nt0, a.NT - 1) * a.KT * 64, (uint32_t)(nts * a.KT * 1024));
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(a.sd + (int64_t)min(nt0, a.NT - 1) * a.G * 16, (uint32_t)(nts * a.G * 32));
    const __amdgpu_buffer_rsrc_t rz =
        make_rsrc(a.sym ? (const void *)a.sd
                        : (const void *)(a.zd + (int64_t)min(nt0, a.NT - 1) * a.GW * 16),
                  a.sym ? 0u : (uint32_t)(nts * a.GW * 64));
    const uint32_t zsym = a.sym ? 8u : 0u;

    // activation stage copy: chunk c = row c / 8, 8-column group c % 8
    h8_t ra[CPT];
    auto load_a = [&](int s) {
#pragma unroll
        for (int c = 0; c < CPT; c++) {
            const int chunk = c * NTHR + tid;
            const int row = chunk >> 3, col = s * KS + (chunk & 7) * 8;
            const uint32_t off = (uint32_t)((row * a.K + col) * 2);
            ra[c] = __builtin_bit_cast(
                h8_t, __builtin_amdgcn_raw_buffer_load_b128(rx, col < a.K ? off : kOutOfRange, 0, 0));
        }
    };
    auto store_a = [&](int buf) {
#pragma unroll
        for (int c = 0; c < CPT; c++) {
            const int chunk = c * NTHR + tid;
            const int row = chunk >> 3, col = (chunk & 7) * 8;
            *(h8_t *)(&sa[buf][row * LDA + col]) = ra[c];
        }
    };

    // weights and group constants of one 128-column tile
    struct BTile {
        u4_t w[TN];
        uint32_t sb[TN][NG], zv[TN][NG];
    };
    auto load_b = [&](BTile &bt, int kt) {
#pragma unroll
        for (int t = 0; t < TN; t++) {
            bt.w[t] = __builtin_bit_cast(
                u4_t, __builtin_amdgcn_raw_buffer_load_b128(
                          rq, (uint32_t)(((t * a.KT + kt) * 64 + lane) * 16), 0, 0));
#pragma unroll
            for (int q = 0; q < NG; q++) {
                int grp = (kt * 128 + 32 * JPG * q) / a.g;
                grp = grp < a.G ? grp : a.G - 1;
                bt.sb[t][q] = __builtin_amdgcn_raw_buffer_load_b16(
                    rs, (uint32_t)(((t * a.G + grp) * 16 + r) * 2), 0, 0);
                const uint32_t zw = __builtin_amdgcn_raw_buffer_load_b32(
                    rz, (uint32_t)(((t * a.GW + (grp >> 3)) * 16 + r) * 4), 0, 0);
                bt.zv[t][q] = ((zw >> (4 * (grp & 7))) & 0xFu) + zsym;
            }
        }
    };

    f4_t acc[TM][TN];
#pragma unroll
    for (int x = 0; x < TM; x++)
#pragma unroll
        for (int y = 0; y < TN; y++)
            acc[x][y] = f4_t{0.f, 0.f, 0.f, 0.f};

    const int S = (a.K + KS - 1) / KS;  // activation stages
    BTile bcur, bnext;
    load_a(0);
    load_b(bcur, 0);
    store_a(0);
    if (S > 1)
        load_a(1);
    __syncthreads();

    // one activation stage: half h of 128-column tile kt (compile-time h so
    // every register index below is static)
    auto stage = [&](int s, auto hc) {
        constexpr int h = decltype(hc)::value;
        const int kt = s >> 1;
        if (h == 0 && kt + 1 < a.KT)
            load_b(bnext, kt + 1);
        const _Float16 *abuf = sa[s & 1] + (wm * TM * 16 + r) * LDA + 8 * i;
#pragma unroll
        for (int jj = 0; jj < 2; jj++) {
            constexpr int j0 = 2 * h;
            const int j = j0 + jj;  // MFMA step inside the 128-column tile
            h8_t xa[TM];
#pragma unroll
            for (int mi = 0; mi < TM; mi++)
                xa[mi] = *(const h8_t *)(abuf + mi * 16 * LDA + 32 * jj);
#pragma unroll
            for (int t = 0; t < TN; t++) {
                const int q = j / JPG;
                const h8_t b = dequant_word(bcur.w[t][j], zero_pair(bcur.zv[t][q]),
                                            scale_pair(bcur.sb[t][q]));
#pragma unroll
                for (int mi = 0; mi < TM; mi++)
                    acc[mi][t] = mfma16x16x32(xa[mi], b, acc[mi][t]);
            }
        }
        if (s + 1 < S)
            store_a((s + 1) & 1);
        if (s + 2 < S)
            load_a(s + 2);
        if (h == 1)
            bcur = bnext;
        __syncthreads();
    };
    for (int s = 0; s < S; s += 2) {
        stage(s, std::integral_constant<int, 0>{});
        if (s + 1 < S)
            stage(s + 1, std::integral_constant<int, 1>{});
    }

    // epilogue: one RNE rounding to fp16
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
                if (m < a.M)
                    ((_Float16 *)a.Y)[(int64_t)m * a.N + n] = (_Float16)acc[mi][t][rr];
            }
    }
}

template <int WM, int WN, int TM, int JPG>
int launch_large_inst(const GemmArgs &a, hipStream_t st) {
    constexpr int BM = WM * TM * 16, BN = WN * 64;
    const int tiles_m = (a.M + BM - 1) / BM;
    const int tiles_n = (a.N + BN - 1) / BN;
    const int tiles = tiles_m * tiles_n;
    const int grid = (tiles + kXcds - 1) / kXcds * kXcds;
    hipLaunchKernelGGL((gemm_large_m_kernel<WM, WN, TM, JPG>), dim3((unsigned)grid),
                       dim3(WM * WN * 64), 0, st, a, tiles_m, tiles_n);
    return (int)hipGetLastError();
}

template <int WM, int WN, int TM>
int launch_large_jpg(const GemmArgs &a, hipStream_t st) {
    if (a.g == 32)
        return launch_large_inst<WM, WN, TM, 1>(a, st);
    if (a.g == 64)
        return launch_large_inst<WM, WN, TM, 2>(a, st);
    return launch_large_inst<WM, WN, TM, 4>(a, st);
}

}  // namespace

int launch_large_m(const GemmArgs &a, const LargePlan &p, hipStream_t st) {
    switch (p.shape) {
    case 0: return launch_large_jpg<2, 2, 4>(a, st);   // 128 x 128, 4 waves
    case 1: return launch_large_jpg<2, 2, 8>(a, st);   // 256 x 128, 4 waves
    case 2: return launch_large_jpg<1, 4, 8>(a, st);   // 128 x 256, 4 waves
    case 3: return launch_large_jpg<2, 4, 4>(a, st);   // 128 x 256, 8 waves
    case 4: return launch_large_jpg<1, 2, 4>(a, st);   //  64 x 128, 2 waves
    case 5: return launch_large_jpg<1, 4, 4>(a, st);   //  64 x 256, 4 waves
    default: return launch_large_jpg<2, 1, 4>(a, st);  // 128 x  64, 2 waves
    }
}

}  // namespace w4a16
