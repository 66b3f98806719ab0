/*
 * CPU oracle for the W4A16 group-quantized GEMM  Y = X . dequant(Q)^T.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is compiled into liboracle_w4a16.so,
 * which only the tests, the smoke check and the CPU-baseline leg of the
 * benchmark load.  The GPU library never links, includes or calls it, and
 * this file includes nothing from the GPU side.
 *
 * Plain, slow, obviously-correct C.  Floating point is fp64 throughout; the
 * only fp16 rounding is the one the method defines for the dequantized
 * weight.  Every function names the passage of the source pages it follows:
 *
 *   [W4A16]   lmdeploy PR "[Feature] Blazing fast W4A16 inference" -- 4-bit
 *             weights with 16-bit activations; the AWQ-format conversion
 *             command (--model_format awq --group_size 128) fixes group-wise
 *             quantization with 128 consecutive weights per group.
 *   [FP16xINT4] the Marlin post (channel "KPD", Telegram) -- an fp16 x int4
 *             mixed-precision linear layer for LLM inference.
 *   [PARTIAL] torchchat issue "linear:int4 quantization regression testing"
 *             -- a 288x288 weight is not compatible with group size 256;
 *             option 2 in the discussion is a groupwise GEMM whose last group
 *             is not a full group.
 *
 * The pages do not write the dequantization formula, the bit order of the
 * packing, the zero-point storage or the scale layout down.  The readings
 * taken here (affine w = (q - z) * s with one RNE rounding to fp16; eight
 * 4-bit codes per uint32, lowest nibble = lowest index; zeros packed the same
 * way along the group index; scales fp16 [N][G]) are the plainest ones and
 * are listed with their reasons in the design notes.
 *
 * Every function below is pinned by a CPU test against something other than
 * itself (closed forms, a hand-worked example, exact integer arithmetic,
 * numpy's float64->float16 cast over the whole finite fp16 domain, and a
 * brute-force numpy matmul).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------ */
/* fp16 <-> fp64, written out from the IEEE 754 binary16 definition.   */
/* ------------------------------------------------------------------ */

/* Decode an IEEE binary16 bit pattern exactly into a double.
 * sign(1) exponent(5, bias 15) fraction(10).  Exponent 0 = subnormal
 * (fraction * 2^-24); exponent 31 = inf / NaN. */
double o_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int ex = (h >> 10) & 0x1F;
    int fr = h & 0x3FF;
    double v;
    if (ex == 0)
        v = ldexp((double)fr, -24);
    else if (ex == 31)
        v = fr ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + fr), ex - 25);
    return sign ? -v : v;
}

/* Round a double to the nearest binary16 value, ties to even, and encode it.
 * Magnitudes that round to 2^16 or more become infinity (IEEE overflow under
 * round-to-nearest); NaN stays NaN. */
uint16_t o_f64_to_f16_rne(double v)
{
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (isnan(v))
        return 0x7E00;
    if (isinf(a))
        return sign | 0x7C00;
    if (a == 0.0)
        return sign;
    /* a = f * 2^e2 with f in [0.5, 1): the leading bit has weight 2^(e2-1). */
    int e2;
    frexp(a, &e2);
    int lead = e2 - 1;
    /* Spacing of binary16 values around a: 2^(lead-10) for normal numbers,
     * the fixed subnormal quantum 2^-24 below 2^-14. */
    int qexp = (lead < -14) ? -24 : lead - 10;
    double n = ldexp(a, -qexp); /* exact: scaling by a power of two */
    double r = rint(n);         /* default rounding mode: nearest, ties to even */
    double R = ldexp(r, qexp);  /* the rounded magnitude, exact */
    if (R >= 65536.0)
        return sign | 0x7C00;
    if (R < ldexp(1.0, -14)) {
        /* subnormal (or the smallest normal when r == 1024): the bit
         * pattern is the integer multiple of 2^-24 itself */
        return sign | (uint16_t)r;
    }
    int f2;
    frexp(R, &f2);
    int L = f2 - 1;                                 /* 2^L <= R < 2^(L+1) */
    int frac = (int)(ldexp(R, 10 - L) - 1024.0);   /* exact integer 0..1023 */
    return sign | (uint16_t)((L + 15) << 10) | (uint16_t)frac;
}

/* bfloat16 (the upper half of an IEEE binary32): sign(1) exponent(8, bias
 * 127) fraction(7).  Exponent 0 = subnormal (fraction * 2^-133); exponent
 * 255 = inf / NaN.  The 16-bit format of the bf16 variant of the method
 * (torchchat runs its int4 linear layers with bf16 activations). */
double o_bf16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int ex = (h >> 7) & 0xFF;
    int fr = h & 0x7F;
    double v;
    if (ex == 0)
        v = ldexp((double)fr, -133);
    else if (ex == 255)
        v = fr ? NAN : INFINITY;
    else
        v = ldexp((double)(128 + fr), ex - 134);
    return sign ? -v : v;
}

/* Round a double to the nearest bfloat16, ties to even (same construction as
 * the binary16 rounding above: 8 significant bits, quantum 2^-133 below the
 * smallest normal 2^-126, infinity from 2^128 on). */
uint16_t o_f64_to_bf16_rne(double v)
{
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (isnan(v))
        return 0x7FC0;
    if (isinf(a))
        return sign | 0x7F80;
    if (a == 0.0)
        return sign;
    int e2;
    frexp(a, &e2);
    int lead = e2 - 1;
    int qexp = (lead < -126) ? -133 : lead - 7;
    double r = rint(ldexp(a, -qexp));
    double R = ldexp(r, qexp);
    if (R >= ldexp(1.0, 128))
        return sign | 0x7F80;
    if (R < ldexp(1.0, -126))
        return sign | (uint16_t)r;  /* subnormal: the multiple of 2^-133 */
    int f2;
    frexp(R, &f2);
    int L = f2 - 1;
    int frac = (int)(ldexp(R, 7 - L) - 128.0);
    return sign | (uint16_t)((L + 127) << 7) | (uint16_t)frac;
}

/* Element-wise o_f64_to_bf16_rne / o_f64_to_f16_rne over an array (the
 * encodings of whole outputs). */
void o_f64_to_16_array(const double *v, int64_t n, int bf16, uint16_t *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++)
        out[i] = bf16 ? o_f64_to_bf16_rne(v[i]) : o_f64_to_f16_rne(v[i]);
}

/* The 16-bit format of activations, scales, weights and outputs: 0 = IEEE
 * binary16, 1 = bfloat16. */
static double h2d(uint16_t h, int bf16) { return bf16 ? o_bf16_to_f64(h) : o_f16_to_f64(h); }
static uint16_t d2h(double v, int bf16) { return bf16 ? o_f64_to_bf16_rne(v) : o_f64_to_f16_rne(v); }

/* ------------------------------------------------------------------ */
/* Packing: eight 4-bit codes per uint32, lowest nibble = lowest index. */
/* ------------------------------------------------------------------ */

/* codes uint8 [R][C] -> words uint32 [R][ceil(C/8)].
 * word[r][j] = sum_i (codes[r][8j+i] & 0xF) << 4i; nibbles past column C
 * are 0.  Only the low 4 bits of each code are kept. [W4A16] */
void o_pack(const uint8_t *codes, int64_t R, int64_t C, uint32_t *words)
{
    int64_t CW = (C + 7) / 8;
    for (int64_t r = 0; r < R; r++)
        for (int64_t j = 0; j < CW; j++) {
            uint32_t w = 0;
            for (int i = 0; i < 8; i++) {
                int64_t c = 8 * j + i;
                if (c < C)
                    w |= (uint32_t)(codes[r * C + c] & 0xF) << (4 * i);
            }
            words[r * CW + j] = w;
        }
}

/* Inverse of o_pack: words uint32 [R][ceil(C/8)] -> codes uint8 [R][C]. */
void o_unpack(const uint32_t *words, int64_t R, int64_t C, uint8_t *codes)
{
    int64_t CW = (C + 7) / 8;
    for (int64_t r = 0; r < R; r++)
        for (int64_t c = 0; c < C; c++)
            codes[r * C + c] = (words[r * CW + c / 8] >> (4 * (c % 8))) & 0xF;
}

/* Nibble c of row r in a packed [R][ceil(C/8)] matrix. */
static int nib(const uint32_t *words, int64_t CW, int64_t r, int64_t c)
{
    return (words[r * CW + c / 8] >> (4 * (c % 8))) & 0xF;
}

/* ------------------------------------------------------------------ */
/* Dequantization  [W4A16] [FP16xINT4] [PARTIAL]                       */
/* ------------------------------------------------------------------ */

/* One row of the dequantized weight.
 *   q = code of (n, k);  j = floor(k / g) its group;  z = zero of (n, j)
 *   (8 when symmetric);  s = fp16 scale of (n, j).
 *   W[n][k] = RNE_fp16((q - z) * s), the product taken in fp64, where it is
 *   exact (a 5-bit integer times an 11-bit significand).
 * G = ceil(K / g): with a partial last group the last group simply holds the
 * K - (G-1)*g remaining columns. */
static void dequant_row(const uint32_t *qp, const uint16_t *scales,
                        const uint32_t *zp, int64_t K, int32_t g,
                        int symmetric, int bf16, int64_t n, uint16_t *wrow)
{
    int64_t KW = (K + 7) / 8;
    int64_t G = (K + g - 1) / g;
    int64_t GW = (G + 7) / 8;
    for (int64_t k = 0; k < K; k++) {
        int64_t j = k / g;
        int q = nib(qp, KW, n, k);
        int z = symmetric ? 8 : nib(zp, GW, n, j);
        double s = h2d(scales[n * G + j], bf16);
        wrow[k] = d2h((double)(q - z) * s, bf16);
    }
}

/* Whole dequantized weight W [N][K] in the 16-bit format `bf16` selects
 * (scales in the same format; for bfloat16 the product of the 5-bit integer
 * and the 8-bit significand is again exact in fp64 and rounds once). */
void o_dequant_fmt(const uint32_t *qp, const uint16_t *scales, const uint32_t *zp,
                   int64_t N, int64_t K, int32_t g, int symmetric, int bf16, uint16_t *W)
{
    for (int64_t n = 0; n < N; n++)
        dequant_row(qp, scales, zp, K, g, symmetric, bf16, n, W + n * K);
}

/* Whole dequantized weight W fp16 [N][K]. */
void o_dequant(const uint32_t *qp, const uint16_t *scales, const uint32_t *zp,
               int64_t N, int64_t K, int32_t g, int symmetric, uint16_t *W)
{
    o_dequant_fmt(qp, scales, zp, N, K, g, symmetric, 0, W);
}

/* ------------------------------------------------------------------ */
/* GEMM  Y[m][n] = sum_k X[m][k] * W[n][k]   [W4A16] [FP16xINT4]        */
/* ------------------------------------------------------------------ */

/* For each selected weight row rows[t] (0 <= t < nrows), every m:
 *   y[m * nrows + t] = sum over k = 0..K-1, in that order, of
 *                      (double)X[m][k] * (double)W[rows[t]][k]
 * where W is the dequantized weight above, X and W in the 16-bit format
 * `bf16` selects.  Each 16-bit x 16-bit product is exact in fp64; the sum is
 * a plain sequential fp64 sum.  wnorm2[t] receives
 * sum_k W[rows[t]][k]^2 (fp64) for the error bound.
 * Passing rows = 0..N-1 gives the whole Y.  OpenMP spreads rows over threads
 * (the result does not depend on the thread count). */
void o_gemm_rows_fmt(const uint16_t *X, int64_t M, int64_t K, const uint32_t *qp,
                     const uint16_t *scales, const uint32_t *zp, int32_t g,
                     int symmetric, int bf16, const int64_t *rows, int64_t nrows,
                     double *y, double *wnorm2)
{
    double *xd = (double *)malloc(sizeof(double) * (size_t)(M * K));
    for (int64_t i = 0; i < M * K; i++)
        xd[i] = h2d(X[i], bf16);
#pragma omp parallel
    {
        uint16_t *wrow = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)K);
        double *wd = (double *)malloc(sizeof(double) * (size_t)K);
#pragma omp for schedule(dynamic, 4)
        for (int64_t t = 0; t < nrows; t++) {
            dequant_row(qp, scales, zp, K, g, symmetric, bf16, rows[t], wrow);
            double nn = 0.0;
            for (int64_t k = 0; k < K; k++) {
                wd[k] = h2d(wrow[k], bf16);
                nn += wd[k] * wd[k];
            }
            if (wnorm2)
                wnorm2[t] = nn;
            for (int64_t m = 0; m < M; m++) {
                double acc = 0.0;
                const double *xr = xd + m * K;
                for (int64_t k = 0; k < K; k++)
                    acc += xr[k] * wd[k];
                y[m * nrows + t] = acc;
            }
        }
        free(wd);
        free(wrow);
    }
    free(xd);
}

/* The fp16 GEMM (activations, scales and weights in binary16). */
void o_gemm_rows(const uint16_t *X, int64_t M, int64_t K, const uint32_t *qp,
                 const uint16_t *scales, const uint32_t *zp, int32_t g,
                 int symmetric, const int64_t *rows, int64_t nrows, double *y,
                 double *wnorm2)
{
    o_gemm_rows_fmt(X, M, K, qp, scales, zp, g, symmetric, 0, rows, nrows, y, wnorm2);
}

/* Number of threads the OpenMP loops above use. */
int o_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Sets that number (used to time the oracle on one thread). */
void o_set_num_threads(int n)
{
#ifdef _OPENMP
    omp_set_num_threads(n > 0 ? n : 1);
#else
    (void)n;
#endif
}

/* ------------------------------------------------------------------ */
/* Device layout (the load-time conversion of the packed weight, the   */
/* counterpart of the offline AWQ -> device conversion step in [W4A16]) */
/* ------------------------------------------------------------------ */
/*
 * Layout "tile 16 x 128", written out from its definition:
 *   NT = ceil(N/16), KT = ceil(K/128), G = ceil(K/g), GW = ceil(G/8).
 *   q_dev: uint32 [NT][KT][64][4].  Weight (n, k) with n = 16*nt + r and
 *     k = 128*kt + 32*j + 8*i + e  (r < 16, i < 4, j < 4, e < 8) lives in
 *     word [nt][kt][r + 16*i][j], at nibble position (e >> 1) + 4*(e & 1)
 *     (even elements in nibbles 0..3, odd elements in nibbles 4..7).
 *     Rows n >= N and columns k >= K hold code 0.
 *   s_dev: fp16 [NT][G][16]:  s_dev[nt][j][r] = scales[16*nt + r][j]
 *     (0 for rows >= N).
 *   z_dev: uint32 [NT][GW][16]: z_dev[nt][w][r] = zeros[16*nt + r][w]
 *     (0 for rows >= N); absent when symmetric.
 */
void o_repack(const uint32_t *qp, const uint16_t *scales, const uint32_t *zp,
              int64_t N, int64_t K, int32_t g, int symmetric, uint32_t *q_dev,
              uint16_t *s_dev, uint32_t *z_dev)
{
    int64_t NT = (N + 15) / 16, KT = (K + 127) / 128;
    int64_t KW = (K + 7) / 8, G = (K + g - 1) / g, GW = (G + 7) / 8;
    memset(q_dev, 0, sizeof(uint32_t) * (size_t)(NT * KT * 256));
    for (int64_t n = 0; n < NT * 16; n++)
        for (int64_t k = 0; k < KT * 128; k++) {
            int code = (n < N && k < K) ? nib(qp, KW, n, k) : 0;
            int64_t nt = n / 16, r = n % 16;
            int64_t kt = k / 128, j = (k % 128) / 32, i = (k % 32) / 8, e = k % 8;
            int64_t word = ((nt * KT + kt) * 64 + (r + 16 * i)) * 4 + j;
            int pos = (int)((e >> 1) + 4 * (e & 1));
            q_dev[word] |= (uint32_t)code << (4 * pos);
        }
    for (int64_t nt = 0; nt < NT; nt++)
        for (int64_t jg = 0; jg < G; jg++)
            for (int64_t r = 0; r < 16; r++) {
                int64_t n = 16 * nt + r;
                s_dev[(nt * G + jg) * 16 + r] = (n < N) ? scales[n * G + jg] : 0;
            }
    if (!symmetric)
        for (int64_t nt = 0; nt < NT; nt++)
            for (int64_t w = 0; w < GW; w++)
                for (int64_t r = 0; r < 16; r++) {
                    int64_t n = 16 * nt + r;
                    z_dev[(nt * GW + w) * 16 + r] = (n < N) ? zp[n * GW + w] : 0;
                }
}

/* Inverse of the weight part of o_repack: q_dev -> canonical packed words. */
void o_unrepack_q(const uint32_t *q_dev, int64_t N, int64_t K, uint32_t *qp)
{
    int64_t KT = (K + 127) / 128, KW = (K + 7) / 8;
    memset(qp, 0, sizeof(uint32_t) * (size_t)(N * KW));
    for (int64_t n = 0; n < N; n++)
        for (int64_t k = 0; k < K; k++) {
            int64_t nt = n / 16, r = n % 16;
            int64_t kt = k / 128, j = (k % 128) / 32, i = (k % 32) / 8, e = k % 8;
            int64_t word = ((nt * KT + kt) * 64 + (r + 16 * i)) * 4 + j;
            int pos = (int)((e >> 1) + 4 * (e & 1));
            int code = (q_dev[word] >> (4 * pos)) & 0xF;
            qp[n * KW + k / 8] |= (uint32_t)code << (4 * (k % 8));
        }
}

/* ------------------------------------------------------------------ */
/* Round-to-nearest group quantizer: fp16 W -> codes, scales, zeros.    */
/* ------------------------------------------------------------------ */

/* The step upstream of the GEMM: turning an fp16 weight into the 4-bit codes
 * with one scale and one zero per group that the AWQ-format conversion
 * produces [W4A16], for a K that is a multiple of the group size or, as in
 * the torchchat discussion, with a last group that is not full [PARTIAL]
 * (padding K with zero columns gives the same codes, scales and zeros for
 * the real columns, because 0 is always inside a group's range).
 *
 * The pages fix no quantizer.  The reading taken is plain round-to-nearest
 * over each group's range, and since floating point decides an integer (the
 * code), the precision is fixed too: fp32, every operation rounded to
 * nearest-even (the quotients w / s correctly rounded, rint half to even),
 * no fused operations (gcc's ISO C mode does not contract).
 * For row n, group j (columns j*g .. min((j+1)*g, K) - 1), with w the exact
 * fp16 values:
 *
 *   asymmetric: lo = min(0, min w), hi = max(0, max w); lo = -1, hi = 1 if
 *     both are 0.  t = (hi - lo) / 15; s = the smallest fp16 >= t;
 *     z = clamp(rint(-lo / s), 0, 15);  q = clamp(rint(w / s) + z, 0, 15).
 *   symmetric (z = 8): a = max |w| (a = 1 if 0); t = a / 7;
 *     s = the smallest fp16 >= t;  q = clamp(rint(w / s) + 8, 0, 15).
 *
 * With w and s both fp16 and |w / s| < 2^5, the fp32 quotient lands on a
 * half-integer only where the exact quotient is that half-integer, and never
 * crosses one, so rint of it is the nearest integer to the exact w / s with
 * exact ties going to the even neighbour.
 *
 * Rounding t up keeps (hi - lo) / s <= 15 (a / s <= 7), so no code is
 * clipped by more than half a step: |(q - z) s - w| <= s/2 up to the fp32
 * rounding of t.  W must be finite; a group whose values come within s/2 of
 * the fp16 maximum can have grid points past it, which the fp16
 * dequantization turns into +-inf.
 * codes uint8 [N][K], scales fp16 bits [N][G], zeros uint8 [N][G] (8s when
 * symmetric). */
static uint16_t f16_round_up(float t)
{
    uint16_t h = o_f64_to_f16_rne((double)t); /* t >= 0 */
    if (o_f16_to_f64(h) < (double)t)
        h = (uint16_t)(h + 1); /* next fp16 up (positive, below infinity) */
    return h;
}

void o_quantize(const uint16_t *W, int64_t N, int64_t K, int32_t g, int symmetric,
                uint8_t *codes, uint16_t *scales, uint8_t *zeros)
{
    int64_t G = (K + g - 1) / g;
    for (int64_t n = 0; n < N; n++)
        for (int64_t j = 0; j < G; j++) {
            int64_t k0 = j * g, k1 = (j + 1) * g < K ? (j + 1) * g : K;
            float lo = 0.0f, hi = 0.0f, amax = 0.0f;
            for (int64_t k = k0; k < k1; k++) {
                float w = (float)o_f16_to_f64(W[n * K + k]); /* exact */
                if (w < lo)
                    lo = w;
                if (w > hi)
                    hi = w;
                if (fabsf(w) > amax)
                    amax = fabsf(w);
            }
            uint16_t sb;
            int z;
            if (symmetric) {
                if (amax == 0.0f)
                    amax = 1.0f;
                sb = f16_round_up(amax / 7.0f);
                z = 8;
            } else {
                if (hi == lo) {
                    lo = -1.0f;
                    hi = 1.0f;
                }
                float t = (hi - lo) / 15.0f;
                sb = f16_round_up(t);
                float zr = rintf(-lo / (float)o_f16_to_f64(sb));
                z = zr < 0.0f ? 0 : (zr > 15.0f ? 15 : (int)zr);
            }
            float s = (float)o_f16_to_f64(sb); /* exact */
            scales[n * G + j] = sb;
            zeros[n * G + j] = (uint8_t)z;
            for (int64_t k = k0; k < k1; k++) {
                float w = (float)o_f16_to_f64(W[n * K + k]);
                int q = (int)rintf(w / s) + z;
                codes[n * K + k] = (uint8_t)(q < 0 ? 0 : (q > 15 ? 15 : q));
            }
        }
}
