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

int launch_pack(const uint8_t *codes, int64_t rows, int64_t cols, uint32_t *out,
                void *stream) {
    const int64_t total = rows * ((cols + 7) / 8);
    const int block = 256;
    int64_t grid = (total + block - 1) / block;
    if (grid > 65536)
        grid = 65536;
    hipLaunchKernelGGL(pack_kernel, dim3((unsigned)grid), dim3(block), 0,
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
        const int64_t k = kt * 128 + 32 * (lane >> 4) + 8 * j;
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

static unsigned grid_for(int64_t total, int block) {
    int64_t grid = (total + block - 1) / block;
    if (grid > 65536)
        grid = 65536;
    if (grid < 1)
        grid = 1;
    return (unsigned)grid;
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
// 8 weights share one group).  Canonical nibbles i and i + 4 hold elements i
// and i + 4.
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
        const h2_t zz = zero_pair(z);
        const h2_t ss = scale_pair(scales[n * G + grp]);
        const uint32_t w = qp[idx];
        uint32_t p[4];
#pragma unroll
        for (int i = 0; i < 4; i++)
            p[i] = dq_pair(w, 4 * i, zz, ss);  // (element i, element i + 4)
        u4_t o;
        o.x = (p[0] & 0xFFFFu) | (p[1] << 16);
        o.y = (p[2] & 0xFFFFu) | (p[3] << 16);
        o.z = (p[0] >> 16) | (p[1] & 0xFFFF0000u);
        o.w = (p[2] >> 16) | (p[3] & 0xFFFF0000u);
        *(u4_t *)(W + idx * 8) = o;
    }
}

int launch_dequant(const uint32_t *qp, const uint16_t *scales, const uint32_t *zp,
                   const Geom &geo, uint16_t *W, void *stream) {
    const int64_t total = geo.N * (geo.K / 8);
    hipLaunchKernelGGL(dequant_kernel, dim3(grid_for(total, 256)), dim3(256), 0,
                       (hipStream_t)stream, qp, scales, zp, geo.N, geo.K, geo.g, geo.G,
                       geo.GW, geo.sym ? 1 : 0, W);
    return (int)hipGetLastError();
}

// ---------------------------------------------------------------------------
// Per-lane group metadata of one 16 x 128 weight tile
// ---------------------------------------------------------------------------
// Lane (r, i) owns columns [128 kt + 32 i, +32) of row 16 nt + r; with g a
// multiple of 32 these lie in one group.  Chunks past K (ragged last tile)
// take the last group: their codes are 0 and their activations are masked to
// 0, so any finite (q - z) * s contributes nothing.
struct GroupMeta {
    h2_t zz, ss;
};

__device__ __forceinline__ GroupMeta load_meta(const uint16_t *__restrict__ sd,
                                               const uint32_t *__restrict__ zd,
                                               int64_t nt, int kbase, int g, int G,
                                               int GW, int r, int sym) {
    int grp = kbase / g;
    grp = grp < G ? grp : G - 1;
    GroupMeta gm;
    gm.ss = scale_pair(sd[(nt * G + grp) * 16 + r]);
    uint32_t z = 8u;
    if (!sym)
        z = (zd[(nt * GW + (grp >> 3)) * 16 + r] >> (4 * (grp & 7))) & 0xFu;
    gm.zz = zero_pair(z);
    return gm;
}

// ---------------------------------------------------------------------------
// Small-M path (memory-bound): one workgroup per (16-row weight tile, 16-row
// activation tile); its waves split K; partial 16 x 16 tiles are summed in LDS.
// ---------------------------------------------------------------------------
// The matrix unit does the multiply-accumulate even at M = 1 (rows past M are
// zero): the VALU then only unpacks and dequantizes, which keeps it off the
// critical path of the weight stream.
template <int WAVES>
__global__ __launch_bounds__(WAVES * 64) void gemm_small_m_kernel(
    const uint16_t *__restrict__ X, int M, int K, const u4_t *__restrict__ qd,
    const uint16_t *__restrict__ sd, const uint32_t *__restrict__ zd, int N, int g,
    int G, int GW, int KT, int sym, uint16_t *__restrict__ Y) {
    __shared__ f4_t red[WAVES][64];
    const int nt = blockIdx.x, mt = blockIdx.y;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int r = lane & 15, i = lane >> 4;
    const int m = mt * 16 + r;
    const bool mok = m < M;
    const _Float16 *xrow = (const _Float16 *)X + (int64_t)(mok ? m : 0) * K;
    const u4_t *qtile = qd + (int64_t)nt * KT * 64 + lane;

    f4_t acc = {0.f, 0.f, 0.f, 0.f};
    for (int kt = wave; kt < KT; kt += WAVES) {
        const u4_t wq = qtile[(int64_t)kt * 64];
        const int kbase = kt * 128 + 32 * i;
        const GroupMeta gm = load_meta(sd, zd, nt, kbase, g, G, GW, r, sym);
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const int k = kbase + 8 * j;
            h8_t a = {};
            if (mok && k < K)
                a = *(const h8_t *)(xrow + k);
            const h8_t b = dq_dev_word(wq[j], gm.zz, gm.ss);
            acc = mfma16x16x32(a, b, acc);
        }
    }
    red[wave][lane] = acc;
    __syncthreads();
    if (wave == 0) {
        f4_t s = red[0][lane];
#pragma unroll
        for (int w = 1; w < WAVES; w++)
            s += red[w][lane];
        const int n = nt * 16 + r;
        if (n < N) {
#pragma unroll
            for (int rr = 0; rr < 4; rr++) {
                const int mo = mt * 16 + 4 * i + rr;
                if (mo < M)
                    ((_Float16 *)Y)[(int64_t)mo * N + n] = (_Float16)s[rr];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Large-M path (compute-bound): 128 x 128 output tile per workgroup of four
// waves (2 x 2, 64 x 64 each).  The activation tile (128 rows x 128 columns)
// is staged in LDS and read by both waves of a row; each wave loads and
// dequantizes its own 64 weight columns straight into MFMA operand registers.
// ---------------------------------------------------------------------------
constexpr int LBM = 128, LBN_TILES = 8, LDX = 128 + 8;

__global__ __launch_bounds__(256) void gemm_large_m_kernel(
    const uint16_t *__restrict__ X, int M, int K, const u4_t *__restrict__ qd,
    const uint16_t *__restrict__ sd, const uint32_t *__restrict__ zd, int N, int g,
    int G, int GW, int KT, int NT, int sym, uint16_t *__restrict__ Y) {
    __shared__ _Float16 sx[LBM * LDX];
    // 1-D grid, M-blocks fastest: workgroups that read the same weight columns
    // run side by side and share them through L2.
    const int MB = (M + LBM - 1) / LBM;
    const int mb = (int)(blockIdx.x % (unsigned)MB), nb = (int)(blockIdx.x / (unsigned)MB);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int r = lane & 15, i = lane >> 4;
    const int wm = wave & 1, wn = wave >> 1;
    const int m0 = mb * LBM;
    const _Float16 *Xh = (const _Float16 *)X;

    f4_t acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; a++)
#pragma unroll
        for (int b = 0; b < 4; b++)
            acc[a][b] = f4_t{0.f, 0.f, 0.f, 0.f};

    for (int kt = 0; kt < KT; kt++) {
        __syncthreads();
#pragma unroll
        for (int it = 0; it < 8; it++) {
            const int idx = it * 256 + tid;
            const int row = idx >> 4, c = idx & 15;
            const int gm = m0 + row, gk = kt * 128 + c * 8;
            h8_t v = {};
            if (gm < M && gk < K)
                v = *(const h8_t *)(Xh + (int64_t)gm * K + gk);
            *(h8_t *)(sx + row * LDX + c * 8) = v;
        }
        u4_t wq[4];
        GroupMeta gmeta[4];
        const int kbase = kt * 128 + 32 * i;
#pragma unroll
        for (int t = 0; t < 4; t++) {
            const int nt = nb * LBN_TILES + wn * 4 + t;
            if (nt < NT) {
                wq[t] = qd[((int64_t)nt * KT + kt) * 64 + lane];
                gmeta[t] = load_meta(sd, zd, nt, kbase, g, G, GW, r, sym);
            } else {
                wq[t] = u4_t{0u, 0u, 0u, 0u};
                gmeta[t].zz = zero_pair(0);
                gmeta[t].ss = scale_pair(0);
            }
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < 4; j++) {
            h8_t a[4];
#pragma unroll
            for (int mi = 0; mi < 4; mi++)
                a[mi] = *(const h8_t *)(sx + (wm * 64 + mi * 16 + r) * LDX + 32 * i + 8 * j);
#pragma unroll
            for (int t = 0; t < 4; t++) {
                const h8_t b = dq_dev_word(wq[t][j], gmeta[t].zz, gmeta[t].ss);
#pragma unroll
                for (int mi = 0; mi < 4; mi++)
                    acc[mi][t] = mfma16x16x32(a[mi], b, acc[mi][t]);
            }
        }
    }

#pragma unroll
    for (int t = 0; t < 4; t++) {
        const int n = (nb * LBN_TILES + wn * 4 + t) * 16 + r;
        if (n >= N)
            continue;
#pragma unroll
        for (int mi = 0; mi < 4; mi++)
#pragma unroll
            for (int rr = 0; rr < 4; rr++) {
                const int m = m0 + wm * 64 + mi * 16 + 4 * i + rr;
                if (m < M)
                    ((_Float16 *)Y)[(int64_t)m * N + n] = (_Float16)acc[mi][t][rr];
            }
    }
}

int launch_gemm(const uint16_t *X, const void *q_dev, const void *s_dev,
                const void *z_dev, const Geom &geo, const GemmPlan &plan, uint16_t *Y,
                void *workspace, void *stream) {
    hipStream_t st = (hipStream_t)stream;
    const u4_t *qd = (const u4_t *)q_dev;
    const uint16_t *sd = (const uint16_t *)s_dev;
    const uint32_t *zd = (const uint32_t *)z_dev;
    const int sym = geo.sym ? 1 : 0;
    (void)workspace;
    if (plan.path == PATH_SMALL) {
        dim3 grid((unsigned)geo.NT, (unsigned)((geo.M + 15) / 16));
        hipLaunchKernelGGL(gemm_small_m_kernel<8>, grid, dim3(512), 0, st, X, (int)geo.M,
                           (int)geo.K, qd, sd, zd, (int)geo.N, geo.g, (int)geo.G,
                           (int)geo.GW, (int)geo.KT, sym, Y);
    } else {
        dim3 grid((unsigned)(((geo.M + LBM - 1) / LBM) *
                             ((geo.NT + LBN_TILES - 1) / LBN_TILES)));
        hipLaunchKernelGGL(gemm_large_m_kernel, grid, dim3(256), 0, st, X, (int)geo.M,
                           (int)geo.K, qd, sd, zd, (int)geo.N, geo.g, (int)geo.G,
                           (int)geo.GW, (int)geo.KT, (int)geo.NT, sym, Y);
    }
    return (int)hipGetLastError();
}

}  // namespace w4a16
