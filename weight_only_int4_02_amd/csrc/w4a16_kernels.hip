// gfx950 kernels of libw4a16: pack, repack, dequant and the two GEMM paths.
//
// Source of the method: lmdeploy PR "[Feature] Blazing fast W4A16 inference"
// (4-bit AWQ-format weights, group size 128, fp16 activations, a load-time
// conversion into the runtime's layout) and the Marlin post on the "KPD"
// Telegram channel (small batch is memory-bound, the ideal int4 gain is 4x;
// large batch is compute-bound and needs the matrix units; the kernel
// prefetches weights, reuses each activation tile many times, and interleaves
// dequantization with matrix instructions).  The designs named there target
// NVIDIA Ampere; the tiling below is built for CDNA4 instead: 64-lane waves,
// v_mfma_f32_16x16x32_f16, 160 KiB of LDS per CU and 256 CUs.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "w4a16_device.hpp"
#include "w4a16_internal.hpp"
#include "w4a16_kernels.hpp"

namespace w4a16 {

// ---------------------------------------------------------------------------
// pack: codes uint8 [R][C] -> uint32 [R][ceil(C/8)], low nibble first
// ---------------------------------------------------------------------------
__global__ void pack_kernel(const uint8_t *__restrict__ codes, int64_t R, int64_t C,
                            uint32_t *__restrict__ out) {
    const int64_t CW = (C + 7) / 8;
    const int64_t total = R * CW;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = idx / CW, j = idx - r * CW;
        const uint8_t *src = codes + r * C + 8 * j;
        const int64_t left = C - 8 * j;
        uint32_t w = 0;
#pragma unroll
        for (int i = 0; i < 8; i++)
            if (i < left)
                w |= (uint32_t)(src[i] & 0xF) << (4 * i);
        out[idx] = w;
    }
}

static unsigned grid_for(int64_t total, int block) {
    int64_t grid = (total + block - 1) / block;
    if (grid > 65536)
        grid = 65536;
    if (grid < 1)
        grid = 1;
    return (unsigned)grid;
}

int launch_pack(const uint8_t *codes, int64_t rows, int64_t cols, uint32_t *out,
                void *stream) {
    const int64_t total = rows * ((cols + 7) / 8);
    hipLaunchKernelGGL(pack_kernel, dim3(grid_for(total, 256)), dim3(256), 0,
                       (hipStream_t)stream, codes, rows, cols, out);
    return (int)hipGetLastError();
}

// ---------------------------------------------------------------------------
// repack: canonical -> "tile 16 x 128" device layout (see w4a16.h)
// ---------------------------------------------------------------------------
// Element e of a canonical word moves to nibble (e >> 1) + 4 (e & 1).
__device__ __forceinline__ uint32_t interleave_nibbles(uint32_t w) {
    uint32_t o = 0;
#pragma unroll
    for (int e = 0; e < 8; e++)
        o |= ((w >> (4 * e)) & 0xFu) << (4 * ((e >> 1) + 4 * (e & 1)));
    return o;
}

// Output word [nt][kt][lane = r + 16 i][j] holds row 16 nt + r, columns
// 128 kt + 32 j + 8 i .. +7: MFMA step j of a tile reads word j of every lane
// and so covers the 32 consecutive columns 128 kt + 32 j .. +31.
__global__ void repack_q_kernel(const uint32_t *__restrict__ qp, int64_t N, int64_t K,
                                int64_t KT, int64_t total, uint32_t *__restrict__ qd) {
    const int64_t KW = K / 8;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int j = (int)(idx & 3);
        const int lane = (int)((idx >> 2) & 63);
        const int64_t tile = idx >> 8;  // nt * KT + kt
        const int64_t nt = tile / KT, kt = tile - nt * KT;
        const int64_t n = nt * 16 + (lane & 15);
        const int64_t k = kt * 128 + 32 * j + 8 * (lane >> 4);
        uint32_t w = 0;
        if (n < N && k < K)
            w = interleave_nibbles(qp[n * KW + k / 8]);
        qd[idx] = w;
    }
}

__global__ void repack_meta_kernel(const uint16_t *__restrict__ scales,
                                   const uint32_t *__restrict__ zp, int64_t N,
                                   int64_t G, int64_t GW, int64_t NT, int sym,
                                   uint16_t *__restrict__ sd, uint32_t *__restrict__ zd) {
    const int64_t ns = NT * G * 16;
    const int64_t nz = sym ? 0 : NT * GW * 16;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < ns + nz;
         idx += (int64_t)gridDim.x * blockDim.x) {
        if (idx < ns) {
            const int r = (int)(idx & 15);
            const int64_t t = idx >> 4, nt = t / G, j = t - nt * G;
            const int64_t n = nt * 16 + r;
            sd[idx] = (n < N) ? scales[n * G + j] : (uint16_t)0;
        } else {
            const int64_t zi = idx - ns;
            const int r = (int)(zi & 15);
            const int64_t t = zi >> 4, nt = t / GW, w = t - nt * GW;
            const int64_t n = nt * 16 + r;
            zd[zi] = (n < N) ? zp[n * GW + w] : 0u;
        }
    }
}

int launch_repack(const uint32_t *qp, const uint16_t *scales, const uint32_t *zp,
                  const Geom &geo, void *q_dev, void *s_dev, void *z_dev, void *stream) {
    hipStream_t st = (hipStream_t)stream;
    const int64_t total_q = geo.NT * geo.KT * 256;
    hipLaunchKernelGGL(repack_q_kernel, dim3(grid_for(total_q, 256)), dim3(256), 0, st, qp,
                       geo.N, geo.K, geo.KT, total_q, (uint32_t *)q_dev);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return (int)e;
    const int64_t total_m = geo.NT * geo.G * 16 + (geo.sym ? 0 : geo.NT * geo.GW * 16);
    hipLaunchKernelGGL(repack_meta_kernel, dim3(grid_for(total_m, 256)), dim3(256), 0, st,
                       scales, zp, geo.N, geo.G, geo.GW, geo.NT, geo.sym ? 1 : 0,
                       (uint16_t *)s_dev, (uint32_t *)z_dev);
    return (int)hipGetLastError();
}

// ---------------------------------------------------------------------------
// dequant: canonical formats -> W fp16 [N][K]
// ---------------------------------------------------------------------------
// One thread per canonical word (8 weights; K % 8 == 0 and g % 8 == 0, so the
// 8 weights share one group).  The word is put in device nibble order and
// dequantized with the same packed arithmetic as the GEMM kernels.
template <bool BF>
__global__ void dequant_kernel(const uint32_t *__restrict__ qp,
                               const uint16_t *__restrict__ scales,
                               const uint32_t *__restrict__ zp, int64_t N, int64_t K,
                               int g, int64_t G, int64_t GW, int sym,
                               uint16_t *__restrict__ W) {
    const int64_t KW = K / 8;
    const int64_t total = N * KW;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int64_t n = idx / KW, jw = idx - n * KW;
        const int64_t grp = (8 * jw) / g;
        const uint32_t z = sym ? 8u : (zp[n * GW + grp / 8] >> (4 * (grp % 8))) & 0xFu;
        if constexpr (BF) {
            const float s = bf16_bits_to_float(scales[n * G + grp]);
            *(bf8_t *)(W + idx * 8) = dequant_word_bf16(interleave_nibbles(qp[idx]), s, (float)z);
        } else {
            *(h8_t *)(W + idx * 8) = dequant_word(interleave_nibbles(qp[idx]), zero_pair(z),
                                                  scale_pair(scales[n * G + grp]));
        }
    }
}

int launch_dequant(const uint32_t *qp, const uint16_t *scales, const uint32_t *zp,
                   const Geom &geo, uint16_t *W, void *stream) {
    const int64_t total = geo.N * (geo.K / 8);
    if (geo.bf16)
        hipLaunchKernelGGL(dequant_kernel<true>, dim3(grid_for(total, 256)), dim3(256), 0,
                           (hipStream_t)stream, qp, scales, zp, geo.N, geo.K, geo.g, geo.G,
                           geo.GW, geo.sym ? 1 : 0, W);
    else
        hipLaunchKernelGGL(dequant_kernel<false>, dim3(grid_for(total, 256)), dim3(256), 0,
                           (hipStream_t)stream, qp, scales, zp, geo.N, geo.K, geo.g, geo.G,
                           geo.GW, geo.sym ? 1 : 0, W);
    return (int)hipGetLastError();
}

// ---------------------------------------------------------------------------
// GEMM dispatch
// ---------------------------------------------------------------------------
int launch_gemm(const uint16_t *X, const void *q_dev, const void *s_dev,
                const void *z_dev, const Geom &geo, const GemmPlan &plan, uint16_t *Y,
                void *workspace, void *stream) {
    GemmArgs a;
    a.X = X;
    a.qd = (const u4_t *)q_dev;
    a.sd = (const uint16_t *)s_dev;
    a.zd = (const uint32_t *)z_dev;
    a.Y = Y;
    a.M = (int)geo.M;
    a.N = (int)geo.N;
    a.K = (int)geo.K;
    a.g = geo.g;
    a.G = (int)geo.G;
    a.GW = (int)geo.GW;
    a.KT = (int)geo.KT;
    a.NT = (int)geo.NT;
    a.sym = geo.sym ? 1 : 0;
    a.lg = __builtin_ctz((unsigned)geo.g);
    a.bf16 = geo.bf16 ? 1 : 0;
    hipStream_t st = (hipStream_t)stream;
    a.ws = (float *)workspace;
    a.splits = 1;
    a.kts = a.KT;
    if (plan.path == PATH_SMALL) {
        SmallPlan sp;
        sp.waves = plan.waves;
        sp.nb = plan.nb;
        sp.depth = plan.depth;
        sp.mtiles = plan.mtiles;
        sp.splits = plan.splits;
        sp.lds = plan.lds;
        sp.xl = plan.xl;
        a.splits = plan.splits;
        a.kts = (a.KT + plan.splits - 1) / plan.splits;
        return launch_small_m(a, sp, st);
    }
    LargePlan lp;
    lp.shape = plan.large_shape;
    a.splits = plan.splits;
    a.kts = (a.KT + plan.splits - 1) / plan.splits;
    return a.bf16 ? launch_large_m_bf16(a, lp, st) : launch_large_m(a, lp, st);
}

}  // namespace w4a16
