// Small-M launcher: dispatch by group-size class.
#include <hip/hip_runtime.h>

#include "w4a16_gemm_kernels.hpp"
#include "w4a16_kernels.hpp"

namespace w4a16 {

int launch_small_m(const GemmArgs &a, const SmallPlan &p, hipStream_t stream) {
    if (a.g == 32)
        return launch_small_m_jpg1(a, p, stream);
    if (a.g == 64)
        return launch_small_m_jpg2(a, p, stream);
    return launch_small_m_jpg4(a, p, stream);
}

}  // namespace w4a16
