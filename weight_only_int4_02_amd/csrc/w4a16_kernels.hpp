// Arguments and launchers of the GEMM kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "w4a16_device.hpp"

namespace w4a16 {

struct GemmArgs {
    const uint16_t *X;     // fp16 [M][K]
    const u4_t *qd;        // weight, device layout, [NT][KT][64] x 16 bytes
    const uint16_t *sd;    // fp16 scales [NT][G][16]
    const uint32_t *zd;    // packed zeros [NT][GW][16] (unused when sym)
    uint16_t *Y;           // fp16 [M][N]
    int M, N, K, g, G, GW, KT, NT, sym;
    int lg;                // log2(g)
    int bf16;              // X, scales and Y are bfloat16 (else fp16)
    // split of K across workgroups (small-M kernel): `splits` slices of `kts`
    // 128-column tiles each; with splits > 1 every slice writes fp32 partial
    // sums to ws [splits][M][N] and a reduce kernel forms Y
    float *ws;
    int splits, kts;
};

// Shape of one small-M launch (see gemm_small_m_kernel).
struct SmallPlan {
    int waves;    // waves per workgroup: 4, 8 or 16
    int nb;       // 16-row weight tiles per workgroup: 1, 2, 4 or 8
    int depth;    // register stages in each wave's prefetch ring: 2, 3 or 4
    int mtiles;   // 16-row activation tiles per workgroup: 1 or 2
    int splits;   // workgroups along K (1: no reduce kernel)
    int lds;      // activations and group constants staged in LDS (M <= 16,
                  // no split): gemm_small_m_lds_kernel
    int xl;       // each wave's activation stages copied through LDS (the
                  // XL form of gemm_small_m_kernel)
};


int launch_small_m(const GemmArgs &a, const SmallPlan &p, hipStream_t stream);
// Y = RNE_fp16(sum of the a.splits fp32 partial-sum slices in a.ws).
int launch_splitk_reduce(const GemmArgs &a, hipStream_t stream);
int launch_small_m_jpg1(const GemmArgs &a, const SmallPlan &p, hipStream_t st);
int launch_small_m_jpg2(const GemmArgs &a, const SmallPlan &p, hipStream_t st);
int launch_small_m_jpg4(const GemmArgs &a, const SmallPlan &p, hipStream_t st);
int launch_small_m_jpg1_bf16(const GemmArgs &a, const SmallPlan &p, hipStream_t st);
int launch_small_m_jpg2_bf16(const GemmArgs &a, const SmallPlan &p, hipStream_t st);
int launch_small_m_jpg4_bf16(const GemmArgs &a, const SmallPlan &p, hipStream_t st);
// Shape of one large-M launch (output tile per workgroup, compute waves, plus
// loader waves): 0 = 128x128 (2x2 waves), 3 = 128x256 (2x4),
// 4 = 64x128 (1x2), 5 = 64x256 (1x4), 6 = 128x64 (2x1), 7 = 32x256 (1x4),
// 8 = 32x128 (1x2), 9 = 64x128 (2x2), 12 = 128x256 from four 128x64 waves
// (1x4; g >= 128, else it runs shape 3), 14 = 256x256 from eight 128x64
// waves (2x4, no loader waves; g >= 128, else shape 3), 17 = 128x192 from
// four 128x48 waves (1x4; fp16 with g >= 128, else shape 3).  K is split across a.splits
// workgroups when a.splits > 1 (partial sums in a.ws, then the reduce kernel).
struct LargePlan {
    int shape;
};

int launch_large_m(const GemmArgs &a, const LargePlan &p, hipStream_t stream);
int launch_large_m_bf16(const GemmArgs &a, const LargePlan &p, hipStream_t stream);

}  // namespace w4a16
