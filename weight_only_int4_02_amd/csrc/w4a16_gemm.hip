// Small-M launcher: dispatch by group-size class.
#include <hip/hip_runtime.h>

#include "w4a16_gemm_kernels.hpp"
#include "w4a16_kernels.hpp"

namespace w4a16 {

namespace {

// Y = RNE(sum over the K slices of the fp32 partial sums), slices summed in
// order, rounded to the output's 16-bit format.  ws is [splits][M][N] fp32, Y [M][N] fp16, both flat; four
// consecutive elements per thread when M N is a multiple of 4.
template <bool BF>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float *__restrict__ ws,
                                                            int splits, int64_t MN,
                                                            uint16_t *__restrict__ Y) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    if ((MN & 3) == 0) {
        const int64_t n4 = MN >> 2;
        for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
            float4 acc = ((const float4 *)ws)[i];
            for (int sp = 1; sp < splits; sp++) {
                const float4 v = ((const float4 *)(ws + sp * MN))[i];
                acc.x += v.x;
                acc.y += v.y;
                acc.z += v.z;
                acc.w += v.w;
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
            float acc = ws[i];
            for (int sp = 1; sp < splits; sp++)
                acc += ws[sp * MN + i];
            store_out16<BF>(Y + i, acc);
        }
    }
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
    int64_t blocks = (work + 255) / 256;
    if (blocks > 4096)
        blocks = 4096;
    if (a.bf16)
        hipLaunchKernelGGL(splitk_reduce_kernel<true>, dim3((unsigned)blocks), dim3(256), 0,
                           stream, a.ws, a.splits, MN, a.Y);
    else
        hipLaunchKernelGGL(splitk_reduce_kernel<false>, dim3((unsigned)blocks), dim3(256), 0,
                           stream, a.ws, a.splits, MN, a.Y);
    return (int)hipGetLastError();
}

}  // namespace w4a16
