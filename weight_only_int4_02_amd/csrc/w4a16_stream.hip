// A plain streaming read, for measurement only: it reads up to three byte
// ranges once, 16 bytes per lane, and keeps nothing.  Timing it over the
// bytes a GEMM call must move gives the read rate the chip reaches with no
// arithmetic at all -- the practical ceiling the weight stream of the small-M
// kernel is compared with.  It is not a step of the method.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "w4a16_device.hpp"
#include "w4a16_internal.hpp"

namespace w4a16 {

namespace {

constexpr int kStreamThreads = 256;
constexpr int kStreamUnroll = 2;   // 16-byte loads in flight per lane

// The three ranges as one index space of 16-byte units: unit i is in a while
// i < na, then in b, then in c.  One grid-stride pass over all of them, so
// the loads of every range are in flight together (measured on MI355X over
// 8-244 MB: two loads per lane with no cap on the grid is the fastest of
// 2, 4 or 8 loads per lane, capped or not).
__device__ __forceinline__ const u4_t *unit_ptr(const u4_t *a, int64_t na, const u4_t *b,
                                                int64_t nb, const u4_t *c, int64_t i) {
    return i < na ? a + i : (i < na + nb ? b + (i - na) : c + (i - na - nb));
}

__global__ __launch_bounds__(kStreamThreads) void stream_read_kernel(
    const u4_t *__restrict__ a, int64_t na, const u4_t *__restrict__ b, int64_t nb,
    const u4_t *__restrict__ c, int64_t nc, uint32_t key, uint32_t *__restrict__ sink) {
    const int64_t n = na + nb + nc;
    const int64_t stride = (int64_t)gridDim.x * kStreamThreads;
    uint32_t acc = 0;
    for (int64_t i = (int64_t)blockIdx.x * kStreamThreads + threadIdx.x; i < n;
         i += kStreamUnroll * stride) {
        u4_t v[kStreamUnroll];
#pragma unroll
        for (int u = 0; u < kStreamUnroll; u++) {
            const int64_t j = i + u * stride;
            v[u] = j < n ? __builtin_nontemporal_load(unit_ptr(a, na, b, nb, c, j))
                         : u4_t{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kStreamUnroll; u++)
            acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    // the loads must not be dropped: their xor decides a store that the
    // caller's key makes (practically) never happen
    if (acc == key)
        sink[0] = acc;
}

}  // namespace

int launch_stream_read(const void *a, size_t a_bytes, const void *b, size_t b_bytes,
                       const void *c, size_t c_bytes, uint32_t key, uint32_t *sink,
                       void *stream) {
    const int64_t na = (int64_t)(a_bytes / 16), nb = (int64_t)(b_bytes / 16),
                  nc = (int64_t)(c_bytes / 16);
    int64_t grid = (na + nb + nc + kStreamThreads * kStreamUnroll - 1) /
                   (kStreamThreads * kStreamUnroll);
    if (grid > (int64_t(1) << 30))
        grid = int64_t(1) << 30;
    if (grid < 1)
        grid = 1;
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)grid), dim3(kStreamThreads), 0,
                       (hipStream_t)stream, (const u4_t *)a, na, (const u4_t *)b, nb,
                       (const u4_t *)c, nc, key, sink);
    return (int)hipGetLastError();
}

}  // namespace w4a16
