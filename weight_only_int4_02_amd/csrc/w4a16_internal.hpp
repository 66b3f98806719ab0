// Internal host-side interface between the C ABI (w4a16_api.hip), the pure
// host checks (w4a16_host.cpp) and the kernel launchers (w4a16_kernels.hip).
#pragma once
#include <stddef.h>
#include <stdint.h>

namespace w4a16 {

// Problem geometry shared by repack and the GEMM kernels.
struct Geom {
    int64_t M, N, K;
    int32_t g;
    int64_t NT;  // ceil(N / 16)   row tiles
    int64_t KT;  // ceil(K / 128)  column tiles
    int64_t G;   // ceil(K / g)    groups per row
    int64_t GW;  // ceil(G / 8)    packed zero words per row
    bool sym;
    bool bf16;   // activations, scales, outputs in bfloat16
};
Geom make_geom(int64_t M, int64_t N, int64_t K, int32_t g, uint32_t flags);

enum Path { PATH_SMALL = 0, PATH_LARGE = 1 };

// How one w4a16_gemm call is executed; chosen on the host from the shape.
struct GemmPlan {
    Path path;
    // small-M kernel shape (see gemm_small_m_kernel)
    int waves;          // waves per workgroup
    int nb;             // 16-row weight tiles per workgroup
    int depth;          // register stages in each wave's prefetch ring
    int mtiles;         // 16-row activation tiles per workgroup
    int splits;         // small-M kernel: workgroups along K (1 = no split)
    int lds;            // small-M kernel: X and group constants staged in LDS
    int xl;             // small-M kernel: activation stages copied through LDS
    int large_shape;    // large-M kernel: output tile shape (see LargePlan)
    size_t ws_bytes;    // workspace bytes needed (split-K partial sums)
};
GemmPlan plan_gemm(const Geom &geo, uint32_t flags);

// Dynamic LDS bytes of the LDS-staged small-M kernel: 1 KiB chunks of the X
// rows, the nb weight tiles' scales and their zero words.
inline size_t small_lds_bytes(int64_t M, int64_t K, int64_t G, int64_t GW, int nb, bool sym) {
    const int64_t x = (M * K * 2 + 1023) / 1024, s = (nb * G * 32 + 1023) / 1024,
                  z = sym ? 0 : (nb * GW * 64 + 1023) / 1024;
    return (size_t)((x + s + z) * 1024);
}

// Small-M kernel shapes (waves, weight tiles nb, activation tiles mt) whose
// instances keep every value in registers, for the group-size class jpg (MFMA
// steps per group inside a 128-column tile: 1, 2, 4 for g = 32, 64, >= 128)
// and the 16-bit format.  The kernel's loads are untracked (their results are
// waited for explicitly), so a register spilled between a load and its wait
// would be saved before the data lands: only these shapes are instantiated,
// the build rejects any kernel that uses scratch, and the host plan moves any
// other shape to fewer waves (four waves fit every shape it asks for; 3 or 6
// tiles only at four waves, 6 tiles of two activation tiles only for fp16
// with g >= 128).
constexpr bool small_shape_fits(int jpg, bool bf16, int waves, int nb, int mt) {
    if (nb == 8)
        return waves <= 8 && !bf16 && jpg == 4;
    if (nb == 3 || nb == 6)
        return waves <= 4 && (nb == 3 || mt == 1 || (jpg == 4 && !bf16));
    if (waves <= 4)
        return true;
    if (waves == 8)
        return !bf16 || nb < 4 || jpg == 4 || (jpg == 2 && mt == 1);
    return waves == 16 && nb == 4 && mt == 1 && !bf16 && jpg == 4;
}

// Largest M the small-M kernel is chosen for automatically (two 16-row
// activation tiles per workgroup, the weight read once per 32 rows), and
// the larger limit for narrow weights (at most 256 row tiles, N <= 4096),
// where it stays ahead of the large-M kernel (measured at N = 4096:
// M = 128 12.1 against 16.3 us for K = 4096, 27.1 against 28.1-30.4 us for
// K = 11008; even at M = 192..256).
constexpr int64_t kSmallMMax = 64;
constexpr int64_t kSmallMMaxNarrow = 128;
// And up to M = 384 for narrow fp16 weights with K <= 4096 (g >= 128), the
// eight-wave shape that copies its activation stages through LDS: Llama-2 7B
// o_proj at M = 160 21.3 -> 19.2 us, 192 23.1 -> 19.7, 256 23.4 -> 18.6, 384
// 30.8 -> 26.1 against the large-M kernel; at M = 512 the large-M kernel is
// ahead (31.3 against 32.6), and down (K = 11008) stays ahead on it from
// M = 192 (41 against 47-53 us).
constexpr int64_t kSmallMMaxNarrowShortK = 384;

// Launchers (w4a16_kernels.hip).  Return a hipError_t as int.
int launch_pack(const uint8_t *codes, int64_t rows, int64_t cols, uint32_t *out,
                void *stream);
int launch_repack(const uint32_t *qp, const uint16_t *scales, const uint32_t *zp,
                  const Geom &geo, void *q_dev, void *s_dev, void *z_dev,
                  void *stream);
int launch_dequant(const uint32_t *qp, const uint16_t *scales, const uint32_t *zp,
                   const Geom &geo, uint16_t *W, void *stream);
int launch_gemm(const uint16_t *X, const void *q_dev, const void *s_dev,
                const void *z_dev, const Geom &geo, const GemmPlan &plan,
                uint16_t *Y, void *workspace, void *stream);
// w4a16_stream.hip
int launch_stream_read(const void *a, size_t a_bytes, const void *b, size_t b_bytes,
                       const void *c, size_t c_bytes, uint32_t key, uint32_t *sink,
                       void *stream);
// w4a16_quantize.hip
int launch_quantize(const uint16_t *W, const Geom &geo, uint32_t *qp, uint16_t *scales,
                    uint32_t *zeros, void *stream);

}  // namespace w4a16
