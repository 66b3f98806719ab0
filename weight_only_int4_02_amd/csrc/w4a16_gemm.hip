// Small-M launcher: dispatch by group-size class.
#include <hip/hip_runtime.h>

#include "w4a16_gemm_kernels.hpp"
#include "w4a16_kernels.hpp"

namespace w4a16 {

namespace {

// Y = RNE(sum over the K slices of the fp32 partial sums), slices summed in
// order, rounded to the output's 16-bit format.  ws is [splits][M][N] fp32, Y [M][N] fp16, both flat; four
// consecutive elements per thread when M N is a multiple of 4.  The partial
// sums are a few MiB at most and the kernel is latency-bound: each thread
// issues the loads of B slices at once (indices past the last slice re-read
// the last one, whose extra copies are not added) before adding them in slice
// order, so the sum is the same as one load and add at a time; blocks of one
// wave spread the threads over all compute units.
constexpr int kReduceThreads = 64;

template <bool BF, int B>
__global__ __launch_bounds__(kReduceThreads) void splitk_reduce_kernel(const float *__restrict__ ws,
                                                                       int splits, int64_t MN,
                                                                       uint16_t *__restrict__ Y) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    if ((MN & 3) == 0) {
        const int64_t n4 = MN >> 2;
        const float4 *ws4 = (const float4 *)ws;
        for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
            float4 acc = {0.f, 0.f, 0.f, 0.f};
            for (int sp0 = 0; sp0 < splits; sp0 += B) {
                float4 v[B];
#pragma unroll
                for (int b = 0; b < B; b++)
                    v[b] = ws4[(int64_t)min(sp0 + b, splits - 1) * n4 + i];
#pragma unroll
                for (int b = 0; b < B; b++) {
                    if (sp0 + b == 0) {
                        acc = v[0];
                    } else if (sp0 + b < splits) {
                        acc.x += v[b].x;
                        acc.y += v[b].y;
                        acc.z += v[b].z;
                        acc.w += v[b].w;
                    }
                }
            }
            if constexpr (BF) {
                typedef __bf16 b4_t __attribute__((ext_vector_type(4)));
                const b4_t h = {(__bf16)acc.x, (__bf16)acc.y, (__bf16)acc.z, (__bf16)acc.w};
                ((b4_t *)Y)[i] = h;
            } else {
                typedef _Float16 h4_t __attribute__((ext_vector_type(4)));
                const h4_t h = {(_Float16)acc.x, (_Float16)acc.y, (_Float16)acc.z,
                                (_Float16)acc.w};
                ((h4_t *)Y)[i] = h;
            }
        }
    } else {
        for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < MN; i += stride) {
            float acc = 0.f;
            for (int sp0 = 0; sp0 < splits; sp0 += B) {
                float v[B];
#pragma unroll
                for (int b = 0; b < B; b++)
                    v[b] = ws[(int64_t)min(sp0 + b, splits - 1) * MN + i];
#pragma unroll
                for (int b = 0; b < B; b++) {
                    if (sp0 + b == 0)
                        acc = v[0];
                    else if (sp0 + b < splits)
                        acc += v[b];
                }
            }
            store_out16<BF>(Y + i, acc);
        }
    }
}

template <bool BF>
void launch_reduce(const GemmArgs &a, int64_t MN, unsigned blocks, hipStream_t stream) {
    if (a.splits <= 2)
        hipLaunchKernelGGL((splitk_reduce_kernel<BF, 2>), dim3(blocks), dim3(kReduceThreads), 0,
                           stream, a.ws, a.splits, MN, a.Y);
    else if (a.splits <= 4)
        hipLaunchKernelGGL((splitk_reduce_kernel<BF, 4>), dim3(blocks), dim3(kReduceThreads), 0,
                           stream, a.ws, a.splits, MN, a.Y);
    else
        hipLaunchKernelGGL((splitk_reduce_kernel<BF, 8>), dim3(blocks), dim3(kReduceThreads), 0,
                           stream, a.ws, a.splits, MN, a.Y);
}

}  // namespace

int launch_small_m(const GemmArgs &a, const SmallPlan &p, hipStream_t stream) {
    int e;
    if (a.g == 32)
        e = a.bf16 ? launch_small_m_jpg1_bf16(a, p, stream) : launch_small_m_jpg1(a, p, stream);
    else if (a.g == 64)
        e = a.bf16 ? launch_small_m_jpg2_bf16(a, p, stream) : launch_small_m_jpg2(a, p, stream);
    else
        e = a.bf16 ? launch_small_m_jpg4_bf16(a, p, stream) : launch_small_m_jpg4(a, p, stream);
    if (e || a.splits == 1)
        return e;
    return launch_splitk_reduce(a, stream);
}

int launch_splitk_reduce(const GemmArgs &a, hipStream_t stream) {
    const int64_t MN = (int64_t)a.M * a.N;
    const int64_t work = (MN & 3) == 0 ? MN >> 2 : MN;
    int64_t blocks = (work + kReduceThreads - 1) / kReduceThreads;
    if (blocks > 16384)
        blocks = 16384;
    if (a.bf16)
        launch_reduce<true>(a, MN, (unsigned)blocks, stream);
    else
        launch_reduce<false>(a, MN, (unsigned)blocks, stream);
    return (int)hipGetLastError();
}

}  // namespace w4a16
