/*
 * w4a16.h -- C ABI of the MI355X (gfx950) W4A16 group-quantized GEMM library
 * (libw4a16.so).
 *
 *     Y[M][N] = X[M][K] . dequant(Q)[N][K]^T,   dequant: w = (q - z) * s
 *
 * X are fp16 activations; Q holds 4-bit weight codes quantized in groups of g
 * consecutive K elements, each group with one fp16 scale s and one 4-bit zero
 * z.  Sources (the pages this library implements):
 *   - lmdeploy PR "[Feature] Blazing fast W4A16 inference": W4A16 inference,
 *     AWQ-format weights with group size 128, converted once offline into the
 *     runtime's own layout before serving (its deploy command);
 *   - the Marlin post on the "KPD" Telegram channel: an fp16 x int4 kernel,
 *     memory-bound at small batch, compute-bound at large batch;
 *   - torchchat issue "linear:int4 quantization regression testing": group
 *     size 256 against a 288 x 288 weight; a shape that is not a multiple of
 *     the group size is either rejected or served by a groupwise GEMM whose
 *     last group is partial (option 2);
 *   - AutoAWQ issue "Add unit/integration testing": the kernel is gated on the
 *     GPU architecture whose matrix instructions it uses.
 *
 * Conventions common to every entry point
 *   - fp16 values are passed as uint16_t bit patterns (IEEE binary16); with
 *     W4A16_BF16 the same arguments carry bfloat16 bit patterns instead.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Device work is enqueued on it; no call synchronizes.
 *   - Device pointers (everything except the *_size / check / status
 *     functions' arguments) must be device memory of the current HIP device
 *     and 16-byte aligned, except `codes` of w4a16_pack (any alignment).
 *   - The caller allocates and owns every buffer, the workspace included.
 *     The library allocates no device memory and keeps no pointer after a call
 *     returns.  Inputs are read only; outputs are fully overwritten.
 *   - Arguments are checked on the host before anything is launched; a
 *     non-zero status means nothing was enqueued (except W4A16_ERR_HIP, which
 *     reports a failed launch; w4a16_last_hip_error() then names it).
 *
 * Canonical (library-neutral) formats
 *   codes    uint8  [R][C], values 0..15 (higher bits are ignored by pack).
 *   packed   uint32 [R][ceil(C/8)]: word j holds codes 8j..8j+7 of its row,
 *            code 8j+i in bits 4i..4i+3 (lowest nibble = lowest index);
 *            nibbles past column C are 0.
 *   qpacked  packed weight codes, R = N, C = K.
 *   scales   fp16 [N][G], G = ceil(K / g): scale of row n, group j.
 *   zeros    packed zeros, R = N, C = G: zero of row n, group j is nibble
 *            (j % 8) of word [n][j / 8].  Unused when W4A16_SYMMETRIC (z = 8).
 *   X        fp16 [M][K] row-major;  Y  fp16 [M][N] row-major.
 */
#ifndef W4A16_H
#define W4A16_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define W4A16_OK             0
#define W4A16_ERR_NULL      (-1) /* a required pointer is NULL */
#define W4A16_ERR_SHAPE     (-2) /* M, N or K <= 0, or K % 8 != 0 (pack: R, C <= 0) */
#define W4A16_ERR_GROUP     (-3) /* g not in {32, 64, 128, 256}, or K % g != 0
                                    without W4A16_PARTIAL_LAST_GROUP */
#define W4A16_ERR_ALIGN     (-4) /* a device pointer is not 16-byte aligned */
#define W4A16_ERR_WORKSPACE (-5) /* workspace smaller than w4a16_gemm_workspace_size */
#define W4A16_ERR_ARCH      (-6) /* the current device is not gfx950 */
#define W4A16_ERR_HIP       (-7) /* a HIP call or launch failed */
#define W4A16_ERR_FLAGS     (-8) /* unknown flag bits, or both path bits set */

/* ---- flags ------------------------------------------------------------- */
/* Symmetric quantization: z = 8 for every group; `zeros` / `z_dev` may be NULL
 * and are not read.  Bit-identical to passing all-8 zeros without the flag. */
#define W4A16_SYMMETRIC          0x1u
/* Allow K % g != 0: G = ceil(K/g) and the last group holds the K - (G-1)*g
 * remaining columns (torchchat issue, option 2). */
#define W4A16_PARTIAL_LAST_GROUP 0x2u
/* bfloat16 instead of fp16 for every 16-bit value of the call: activations
 * X, scales, the output Y (w4a16_gemm) and the dequantized W
 * (w4a16_dequant); the weight becomes RNE_bf16((q - z) * s).  The bf16
 * variant torchchat's int4 linear layers run with.  Not for w4a16_quantize
 * (W4A16_ERR_FLAGS). */
#define W4A16_BF16               0x4u
/* w4a16_gemm only: force the small-M (memory-bound) or the MFMA tile
 * (compute-bound) kernel instead of choosing by M.  Any M is accepted by
 * either; used to run both kernels on the same inputs. */
#define W4A16_PATH_SMALL_M       0x10u
#define W4A16_PATH_LARGE_M       0x20u

/* ---- status ------------------------------------------------------------ */
/* Static, human-readable name of a status code ("unknown status" otherwise).
 * Passage: torchchat issue "linear:int4 quantization regression testing",
 * the opening post's log, where a weight whose shape does not fit the group
 * size is skipped with only a printed message; here every refusal is a
 * status the caller sees and decides on.  Pure host, never fails. */
const char *w4a16_status_str(int32_t status);
/* Text of the last HIP error seen by a call on this host thread ("" if none).
 * Passage: lmdeploy PR "[Feature] Blazing fast W4A16 inference", the comment
 * reporting a library that failed to load over an undefined GemmS4F16
 * symbol: a failure carries its cause.  Every symbol this header declares is
 * a plain extern "C" function of libw4a16.so.  Pure host, never fails. */
const char *w4a16_last_hip_error(void);
/* Architecture gate: W4A16_OK if the current HIP device is gfx950, else
 * W4A16_ERR_ARCH (or W4A16_ERR_HIP if no device can be queried).  The result
 * is cached per device.  Every launching entry point applies it.
 * Passage: AutoAWQ issue "Add unit/integration testing", the comment that
 * the kernel's .m16n8k16 matrix instruction ties it to sm_80 and later: a
 * kernel written for one generation's matrix instructions is refused
 * elsewhere with an explicit status instead of a failed launch. */
int32_t w4a16_device_check(void);

/* ---- pack -------------------------------------------------------------- */
/* Packs a 4-bit code matrix: codes uint8 [rows][cols] (device) ->
 * packed uint32 [rows][ceil(cols/8)] (device), low nibble first, keeping the
 * low 4 bits of each code.  Used for weight codes (rows = N, cols = K) and for
 * zeros (rows = N, cols = G).  Bit-exact.
 * Passage: lmdeploy PR "[Feature] Blazing fast W4A16 inference", the
 * conversion command (deploy.py ... --model_format awq --group_size 128):
 * 4-bit AWQ weights stored as packed codes.
 * Errors: W4A16_ERR_NULL (codes or packed NULL), W4A16_ERR_SHAPE (rows or
 * cols <= 0, or rows * cols > 2^34), W4A16_ERR_ALIGN (packed not 16-byte
 * aligned), W4A16_ERR_ARCH, W4A16_ERR_HIP.  The caller owns both buffers. */
int32_t w4a16_pack(const uint8_t *codes, int64_t rows, int64_t cols,
                   uint32_t *packed, void *stream);
int32_t w4a16_check_pack_args(const uint8_t *codes, int64_t rows, int64_t cols,
                              const uint32_t *packed);

/* ---- repack (load-time layout conversion) ------------------------------ */
/* Passage: lmdeploy PR "[Feature] Blazing fast W4A16 inference", the
 * conversion command (deploy.py ... --model_format awq --group_size 128
 * --dst-path ...): AWQ weights are converted once, offline, into the
 * runtime's own layout before serving.  w4a16_repack_size is pure host;
 * w4a16_repack enqueues the conversion.
 * Errors: W4A16_ERR_NULL (a required pointer NULL; zeros and z_dev may be
 * NULL only with W4A16_SYMMETRIC), W4A16_ERR_SHAPE (N, K <= 0, K % 8 != 0,
 * N > 2^26, K >= 2^22 or N K > 2^34), W4A16_ERR_GROUP, W4A16_ERR_FLAGS,
 * W4A16_ERR_ALIGN, W4A16_ERR_ARCH, W4A16_ERR_HIP.
 * Device layout "tile 16 x 128" (version 1).  NT = ceil(N/16),
 * KT = ceil(K/128), G = ceil(K/g), GW = ceil(G/8).
 *   q_dev uint32 [NT][KT][64][4]: weight (n, k), n = 16 nt + r,
 *         k = 128 kt + 32 j + 8 i + e (r < 16, i < 4, j < 4, e < 8), is in
 *         word [nt][kt][r + 16 i][j] at nibble (e >> 1) + 4 (e & 1): even
 *         elements in nibbles 0..3, odd ones in nibbles 4..7.  One 1 KiB
 *         block is a 16-row x 128-column tile; word j of its 64 lanes is the
 *         16-row x 32-column slice 32 j .. 32 j + 31.  Padding rows / columns
 *         hold code 0.
 *   s_dev fp16   [NT][G][16]:  s_dev[nt][j][r] = scales[16 nt + r][j].
 *   z_dev uint32 [NT][GW][16]: z_dev[nt][w][r] = zeros[16 nt + r][w]
 *         (canonical zero words); 0 bytes when W4A16_SYMMETRIC.
 * Padding rows hold scale 0 and zero word 0.  Bit-exact, invertible. */
int32_t w4a16_repack_size(int64_t N, int64_t K, int32_t g, uint32_t flags,
                          size_t *q_bytes, size_t *s_bytes, size_t *z_bytes);
int32_t w4a16_repack(const uint32_t *qpacked, const uint16_t *scales,
                     const uint32_t *zeros, int64_t N, int64_t K, int32_t g,
                     uint32_t flags, void *q_dev, void *s_dev, void *z_dev,
                     void *stream);
int32_t w4a16_check_repack_args(const uint32_t *qpacked, const uint16_t *scales,
                                const uint32_t *zeros, int64_t N, int64_t K,
                                int32_t g, uint32_t flags, const void *q_dev,
                                const void *s_dev, const void *z_dev);

/* ---- dequant ----------------------------------------------------------- */
/* W fp16 [N][K] = RNE_fp16((q - z) * s) from the canonical formats (one
 * rounding; the subtraction is exact).  Bit-exact.
 * Passage: lmdeploy PR "[Feature] Blazing fast W4A16 inference", title and
 * conversion command: 4-bit weights with 16-bit activations, one scale and
 * zero per group of --group_size 128 columns; the formula itself is a
 * reading (the pages print none).
 * Errors: as w4a16_repack (W replaces the device outputs). */
int32_t w4a16_dequant(const uint32_t *qpacked, const uint16_t *scales,
                      const uint32_t *zeros, int64_t N, int64_t K, int32_t g,
                      uint32_t flags, uint16_t *W, void *stream);
int32_t w4a16_check_dequant_args(const uint32_t *qpacked, const uint16_t *scales,
                                 const uint32_t *zeros, int64_t N, int64_t K,
                                 int32_t g, uint32_t flags, const uint16_t *W);

/* ---- quantize ---------------------------------------------------------- */
/* Round-to-nearest group quantization of an fp16 weight W [N][K] into the
 * canonical formats above: qpacked [N][K/8], scales [N][G], zeros
 * [N][ceil(G/8)] (not written, and may be NULL, with W4A16_SYMMETRIC).
 * Passage: torchchat issue "linear:int4 quantization regression testing",
 * the padding discussion and option 2 (a groupwise GEMM whose last group is
 * not full): with W4A16_PARTIAL_LAST_GROUP a K that is not a multiple of g
 * gets a partial last group, which yields the same codes, scales and zeros
 * as padding K with zero columns (option 1).  The output is the group-wise
 * format of the lmdeploy PR's AWQ conversion.  The rule is a reading.
 * Per row and group, in fp32 with every operation rounded to nearest-even:
 *   asymmetric: lo = min(0, min w), hi = max(0, max w) ([-1, 1] if both 0);
 *     s = smallest fp16 >= (hi - lo) / 15;  z = clamp(rint(-lo / s), 0, 15);
 *   symmetric: s = smallest fp16 >= max|w| / 7 (max|w| = 1 if 0);  z = 8;
 *   q = clamp(rint(w / s) + z, 0, 15)   (rint: half to even; the quotients
 *   correctly rounded, so exact ties w / s = k + 1/2 go to the even k).
 * Then |(q - z) s - w| <= s / 2.  W must be finite.  Bit-exact (integer
 * results decided in the stated precision).
 * Errors: W4A16_ERR_NULL, W4A16_ERR_SHAPE, W4A16_ERR_GROUP (K % g != 0
 * without W4A16_PARTIAL_LAST_GROUP), W4A16_ERR_FLAGS (W4A16_BF16 or a path
 * bit), W4A16_ERR_ALIGN, W4A16_ERR_ARCH, W4A16_ERR_HIP. */
int32_t w4a16_quantize(const uint16_t *W, int64_t N, int64_t K, int32_t g,
                       uint32_t flags, uint32_t *qpacked, uint16_t *scales,
                       uint32_t *zeros, void *stream);
int32_t w4a16_check_quantize_args(const uint16_t *W, int64_t N, int64_t K,
                                  int32_t g, uint32_t flags,
                                  const uint32_t *qpacked,
                                  const uint16_t *scales,
                                  const uint32_t *zeros);

/* ---- GEMM -------------------------------------------------------------- */
/* Bytes of workspace w4a16_gemm needs for this problem (the same M, N, K, g
 * and flags, path flags included).  Pure host.
 * Passage: the Marlin post on the "KPD" channel, the paragraph on small
 * batches being memory-bound: a small-M call is spread over the whole chip
 * by splitting K across workgroups, whose fp32 partial sums need this
 * caller-owned scratch.  Errors: W4A16_ERR_NULL (bytes NULL), W4A16_ERR_SHAPE
 * (M <= 0 or M > 2^20, or the weight shape), W4A16_ERR_GROUP, W4A16_ERR_FLAGS.  0 when the chosen kernel
 * covers all of K in one workgroup; S * M * N * 4 when it splits K across S
 * workgroups (S fp32 partial sums of Y, summed in order and rounded once by
 * a second kernel).  S depends only on the shape. */
int32_t w4a16_gemm_workspace_size(int64_t M, int64_t N, int64_t K, int32_t g,
                                  uint32_t flags, size_t *bytes);
/* Which kernel w4a16_gemm runs for this problem (the same arguments and
 * flags, path flags included) and across how many workgroups it splits K.
 * Passage: the Marlin post on the "KPD" channel: memory-bound at small batch,
 * compute-bound as the batch grows, and feature 5 (the thread-group
 * configuration tuned per case).
 * Pure host; the same checks and status codes as
 * w4a16_gemm_workspace_size.  *path = W4A16_KERNEL_SMALL_M or
 * W4A16_KERNEL_LARGE_M; *splits = S >= 1 (S > 1: S fp32 partial sums and
 * the reduce kernel after the main one).  Without a path flag the small-M
 * kernel runs for M <= 64, up to M = 128 when N <= 4096, and for fp16 up to
 * M = 384 when also K <= 4096 and g >= 128. */
#define W4A16_KERNEL_SMALL_M 0
#define W4A16_KERNEL_LARGE_M 1
int32_t w4a16_gemm_kernel(int64_t M, int64_t N, int64_t K, int32_t g,
                          uint32_t flags, int32_t *path, int32_t *splits);
/* Y = X . dequant(Q)^T with the weight in the repacked device layout.
 * Passages: lmdeploy PR "[Feature] Blazing fast W4A16 inference" (W4A16
 * inference on AWQ weights with group size 128; its benchmark table is the
 * Llama-2-7B decode workload this serves) and the Marlin post on the "KPD"
 * channel (an FP16 x INT4 kernel for batched LLM inference).
 * Errors: those of w4a16_check_gemm_args, then W4A16_ERR_ARCH and
 * W4A16_ERR_HIP.  Nothing is enqueued when the status is not W4A16_OK
 * (W4A16_ERR_HIP: a launch failed).
 * fp16: products in fp16 x fp16 with fp32 accumulation, one RNE rounding to
 * fp16 at the end; |y| beyond the fp16 range becomes +-inf.  The large-M
 * kernel multiplies by the dequantized weight RNE_fp16((q - z) * s) defined
 * above.  The small-M kernel (see w4a16_gemm_kernel) applies each group's scale
 * to the fp32 sum of (q - z) x over the group, i.e. it uses the exact product
 * (q - z) * s; its result differs from the product with the rounded weight by
 * at most 2^-11 sum_k |x_k w_k|.
 * W4A16_BF16: the same with bf16 X, scales and Y and one RNE rounding to
 * bf16.  The large-M kernel multiplies by RNE_bf16((q - z) * s); the small-M
 * kernel forms the exact (q - z) * s per group as s * (sum (128 + q) x -
 * sum (128 + z) x) of two fp32 MFMA sums, which differs from the product with
 * the rounded weight by at most 2^-9 sum_k |x_k w_k| plus the fp32 rounding
 * of those sums, and is exactly 0 for a group whose weights are all 0.
 * X and Y must not overlap (W4A16_ERR_SHAPE).  The workspace (at least
 * w4a16_gemm_workspace_size bytes, else W4A16_ERR_WORKSPACE) is caller-owned
 * scratch, overwritten by the call; two calls that may run at the same time
 * must not share it. */
int32_t w4a16_gemm(const uint16_t *X, int64_t M, int64_t K, const void *q_dev,
                   const void *s_dev, const void *z_dev, int64_t N, int32_t g,
                   uint32_t flags, uint16_t *Y, void *workspace,
                   size_t workspace_bytes, void *stream);
/* The host-side checks of w4a16_gemm alone (no HIP call).
 * Passage: torchchat issue "linear:int4 quantization regression testing",
 * the skip message for a 288 x 288 weight "not compatible with group_size
 * 256" and option 2: a K that is not a multiple of g is W4A16_ERR_GROUP
 * unless W4A16_PARTIAL_LAST_GROUP asks for a partial last group.
 * Errors: W4A16_ERR_FLAGS (unknown bits, or both path bits), W4A16_ERR_NULL
 * (X, q_dev, s_dev or Y NULL; z_dev NULL without W4A16_SYMMETRIC; workspace
 * NULL when w4a16_gemm_workspace_size is not 0), W4A16_ERR_SHAPE (M <= 0,
 * M > 2^20, M K or M N > 2^34, the weight shape of w4a16_repack, or X and Y
 * overlapping), W4A16_ERR_GROUP, W4A16_ERR_ALIGN (a device pointer not
 * 16-byte aligned), W4A16_ERR_WORKSPACE (workspace_bytes too small). */
int32_t w4a16_check_gemm_args(const uint16_t *X, int64_t M, int64_t K,
                              const void *q_dev, const void *s_dev,
                              const void *z_dev, int64_t N, int32_t g,
                              uint32_t flags, const uint16_t *Y,
                              const void *workspace, size_t workspace_bytes);

/* ---- GEMM without allocation ------------------------------------------- */
/* For callers that cannot allocate device memory at call time -- code being
 * captured into a HIP graph, tight serving loops, harnesses that forbid
 * hipMalloc: w4a16_gemm with the split-K workspace replaced by a static
 * scratch array inside the library (W4A16_NOALLOC_SCRATCH_BYTES per GPU,
 * held from the first call on that GPU until the process ends).  The caller
 * still passes X, the weight and Y; the call allocates nothing (no hipMalloc,
 * hipFree or allocating library routine) and computes exactly what w4a16_gemm
 * computes with the same arguments (same plan, same kernels, bit for bit).
 * Every call on one GPU shares that GPU's scratch, which keeps the last
 * call's partial sums (each call overwrites what it reads, so nothing needs
 * clearing): calls that may overlap on one GPU -- other streams, other host
 * threads -- race on it and must be ordered by the caller.
 * The scratch is as large as the largest split-K workspace the library's plan
 * makes (256 workgroups, each with one 128 x 256 fp32 partial tile: 32 MiB),
 * so every call fits.
 * Errors: those of w4a16_gemm; W4A16_ERR_WORKSPACE if a call's plan ever
 * needed more split-K scratch than W4A16_NOALLOC_SCRATCH_BYTES
 * (w4a16_last_hip_error then states both sizes), checked before anything is
 * enqueued. */
#define W4A16_NOALLOC_SCRATCH_BYTES (32u << 20)
int32_t w4a16_gemm_noalloc(const uint16_t *X, int64_t M, int64_t K, const void *q_dev,
                           const void *s_dev, const void *z_dev, int64_t N, int32_t g,
                           uint32_t flags, uint16_t *Y, void *stream);

/* ---- measurement ------------------------------------------------------- */
/* Reads the byte ranges [a, a + a_bytes), [b, ...), [c, ...) once (16 bytes
 * per lane, no arithmetic) and writes *sink only if the xor of everything
 * read equals `key` (pick a key that is practically never met; the store
 * keeps the loads from being dropped).  Not a step of the method: a plain
 * streaming read of the bytes a call must move, timed beside it as the read
 * rate the chip reaches without any arithmetic.
 * Passage: bigcode-inference-benchmark issue "Inference tasks and
 * milestones", the profiling task (basic profiling in the benchmarking code).
 * Errors: W4A16_ERR_NULL (sink NULL, or a range NULL with bytes > 0),
 * W4A16_ERR_SHAPE (a size not a multiple of 16, or all sizes 0),
 * W4A16_ERR_ALIGN (a range not 16-byte aligned), W4A16_ERR_ARCH,
 * W4A16_ERR_HIP.  Device pointers; the caller owns them. */
int32_t w4a16_stream_read(const void *a, size_t a_bytes, const void *b, size_t b_bytes,
                          const void *c, size_t c_bytes, uint32_t key, uint32_t *sink,
                          void *stream);

#ifdef __cplusplus
}
#endif
#endif /* W4A16_H */
