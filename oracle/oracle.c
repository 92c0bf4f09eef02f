/*
 * CPU oracle for the per-output-channel INT8 quantized linear.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product library may include,
 * link, load or call this file: only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark use it. It shares no header, helper,
 * table or constant with the HIP library; it is compiled by gcc from this
 * file alone.
 *
 * Build: gcc -std=c11 -O2 -ffp-contract=off -fno-fast-math -fopenmp -fPIC
 *        -shared (see build.py in this directory). -ffp-contract=off keeps
 *        every float multiply and add separately rounded; x86-64 SSE gives
 *        FLT_EVAL_METHOD == 0 and no flush-to-zero, so each float operation
 *        below is one correctly rounded IEEE binary32 operation.
 *
 * Plain and slow on purpose: every function is the definition on the pages
 * written out in loops, in the order the pages state it. OpenMP splits only
 * independent outputs (rows, or the (row, column) pairs of the linears), and
 * every sum runs whole inside one thread, so no result depends on the thread
 * count (the SmolVLM recipe's RefSDPA note: sums whose order follows the
 * thread split change from run to run). Integer sums are int64; float references are
 * fp64 sums of exact products.
 *
 * Citations name the page and the section on it:
 *   [SmolVLM q8 recipe]  SmolVLM-500M-Instruct ExecuTorch WebGPU, the 8-bit
 *                        building blocks (module docstring, weight_int8,
 *                        act_observer/qparams, fake_quant, Q8Linear)
 *   [Ming INT8 linear]   Ming-Image-0.1-Design-ROCm-INT8 int8_linear
 *                        (QUANT_RULE, quantize_weight, Int8Linear.forward)
 *   [tiny-llm quant]     tiny-llm quant module (Step 4.6 docstring,
 *                        quantize_per_channel, dequantize, Int8Linear)
 *   [ExecuTorch PR 8da4w] ExecuTorch WebGPU PR "Add linear_dq8ca_q4gsw +
 *                        choose_qparams_affine (8da4w)", the Impl paragraph
 */
#include <math.h>
#include <omp.h>
#include <float.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_BAD (-1)

/* ------------------------------------------------------------------ helpers */

/* Clamp a float to [lo, hi] in float, as torch.clamp does before the cast. */
static float clampf_(float v, float lo, float hi)
{
    if (v < lo) return lo;
    if (v > hi) return hi;
    return v;
}

/* bf16 bit pattern -> float: the 16 bits are the top half of a binary32. */
static float bf16_to_float_(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* ------------------------------------------------ weight quantization (int8) */

/*
 * Per-output-channel symmetric int8 weight quantization.
 *
 * mode 0 (SYM127), [Ming INT8 linear] QUANT_RULE / quantize_weight and
 * [tiny-llm quant] quantize_per_channel: scale = absmax(row) / 127,
 * q = clamp(round(w / scale), -127, 127).
 * mode 1 (SYM127_5), [SmolVLM q8 recipe] weight_int8: the per-channel
 * symmetric observer scale amax / 127.5, q = clamp(round(w / scale), -128, 127).
 *
 * All-zero row, both modes: scale 1.0 and q 0 (the Ming QUANT_RULE
 * convention: no division by zero). round() is round-half-to-even (rintf
 * under the default rounding mode), the division is IEEE binary32 w / scale
 * exactly as all three pages write it. wsum[n] = sum_k q[n,k], the
 * weight_sums the q8ta_q8csw op takes ([SmolVLM q8 recipe] fix_q8ta_fake
 * signature); wsum may be NULL.
 */
int orc_quantize_weight_int8(const float *w, int64_t N, int64_t K, int mode,
                             int8_t *q, float *scale, int32_t *wsum)
{
    if (N < 0 || K < 0 || (mode != 0 && mode != 1)) return ORC_BAD;
    const float den = (mode == 0) ? 127.0f : 127.5f;
    const float lo = (mode == 0) ? -127.0f : -128.0f;
    const float hi = 127.0f;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        const float *row = w + n * K;
        float amax = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float a = fabsf(row[k]);
            if (a > amax) amax = a;
        }
        int64_t sum = 0;
        if (amax == 0.0f) {
            scale[n] = 1.0f;
            for (int64_t k = 0; k < K; ++k) q[n * K + k] = 0;
        } else {
            float s = amax / den;
            scale[n] = s;
            for (int64_t k = 0; k < K; ++k) {
                float t = row[k] / s;
                float r = clampf_(rintf(t), lo, hi);
                int8_t c = (int8_t)(int)r;
                q[n * K + k] = c;
                sum += c;
            }
        }
        if (wsum) wsum[n] = (int32_t)sum;
    }
    return ORC_OK;
}

/* ---------------------------------------- 4-bit group-symmetric weights (q4gsw) */

/*
 * q4gsw weights for the 8da4w linear ([ExecuTorch PR 8da4w]: "4-bit group
 * weights" consumed by the q4gsw GEMM; the page prints no layout or scale
 * rule, so both are readings): per output channel n and group g of `group`
 * consecutive k, gs = amax_g / 7.5 (the symmetric observer rule of
 * [SmolVLM q8 recipe] weight_int8, amax / ((qmax - qmin) / 2), with the int4
 * range [-8, 7]); q4 = clamp(round(w / gs), -8, 7); an all-zero group gets
 * gs = 1, q4 = 0. Packing: byte n*K/2 + k/2 holds k even in its low nibble
 * and k odd in its high nibble, two's complement. gsum[n, g] = sum of the
 * group's codes (the per-group weight_sums).
 */
int orc_quantize_weight_q4gsw(const float *w, int64_t N, int64_t K,
                              int64_t group, uint8_t *q4, float *gs,
                              int32_t *gsum)
{
    if (N < 0 || K < 0 || group <= 0 || (group % 2) != 0 || (K % group) != 0)
        return ORC_BAD;
    const int64_t G = K / group;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t g = 0; g < G; ++g) {
            const float *src = w + n * K + g * group;
            float amax = 0.0f;
            for (int64_t j = 0; j < group; ++j) {
                float a = fabsf(src[j]);
                if (a > amax) amax = a;
            }
            float s = (amax == 0.0f) ? 1.0f : amax / 7.5f;
            gs[n * G + g] = s;
            int64_t sum = 0;
            for (int64_t j = 0; j < group; ++j) {
                int c = 0;
                if (amax != 0.0f) c = (int)clampf_(rintf(src[j] / s), -8.0f, 7.0f);
                sum += c;
                int64_t k = g * group + j;
                uint8_t *byte = q4 + n * (K / 2) + k / 2;
                uint8_t nib = (uint8_t)(c & 0xF);
                if ((k & 1) == 0)
                    *byte = (uint8_t)((*byte & 0xF0) | nib);
                else
                    *byte = (uint8_t)((*byte & 0x0F) | (nib << 4));
            }
            gsum[n * G + g] = (int32_t)sum;
        }
    }
    return ORC_OK;
}

/* Decode one packed signed nibble (the layout above). */
static int q4_at_(const uint8_t *q4, int64_t K, int64_t n, int64_t k)
{
    uint8_t b = q4[n * (K / 2) + k / 2];
    int v = (k & 1) ? (b >> 4) : (b & 0xF);
    return v >= 8 ? v - 16 : v;
}

/* ------------------------------------------------- activation quantization */

/*
 * Static per-tensor affine int8 quantization of activations,
 * [SmolVLM q8 recipe] fake_quant and Q8Linear.forward:
 * xq = clamp(round(x * (1/s)) + z, -128, 127). The reciprocal is one
 * binary32 division 1/s; the product, the rounding and the add of z are
 * each a binary32 operation and the clamp happens in float before the cast.
 *
 * With two_pass, the second pass quantizes the first pass's rounding error:
 * r = x - (xq1 - z1) * s1 (the residual "written with plain ops": one
 * rounded multiply, then one rounded subtract, no fused multiply-add), and
 * xq2 = clamp(round(r * (1/s2)) + z2, -128, 127). xq2 may be NULL when
 * two_pass is 0.
 */
int orc_quantize_act_per_tensor(const float *x, int64_t count, float s1,
                                int32_t z1, int two_pass, float s2, int32_t z2,
                                int8_t *xq1, int8_t *xq2)
{
    if (count < 0 || !(s1 > 0.0f) || (two_pass && !(s2 > 0.0f))) return ORC_BAD;
    const float inv1 = 1.0f / s1;
    const float inv2 = two_pass ? 1.0f / s2 : 0.0f;
    const float fz1 = (float)z1, fz2 = (float)z2;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i) {
        float v = x[i];
        float p = v * inv1;
        float c1 = clampf_(rintf(p) + fz1, -128.0f, 127.0f);
        xq1[i] = (int8_t)(int)c1;
        if (two_pass) {
            float t = (c1 - fz1) * s1;
            float r = v - t;
            float p2 = r * inv2;
            float c2 = clampf_(rintf(p2) + fz2, -128.0f, 127.0f);
            xq2[i] = (int8_t)(int)c2;
        }
    }
    return ORC_OK;
}

/*
 * Per-row asymmetric int8 activation qparams, [ExecuTorch PR 8da4w]
 * choose_qparams_affine: a per-row min/max, then calculate_scale_and_zero_point.
 * The page prints no formula; the affine min/max rule that the recipe's
 * MinMaxObserver uses ([SmolVLM q8 recipe] act_observer, qparams) is the
 * reading: mn = min(min_k x, 0), mx = max(max_k x, 0),
 * s = max((mx - mn) / 255, FLT_EPSILON), zp = clamp(-128 - round(mn / s),
 * -128, 127). If xq is not NULL the row is also quantized with (s, zp) by
 * the fake_quant rule above.
 */
int orc_choose_qparams_rows(const float *x, int64_t M, int64_t K, float *scale,
                            int32_t *zp, int8_t *xq)
{
    if (M < 0 || K <= 0) return ORC_BAD;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        const float *row = x + m * K;
        float mn = row[0], mx = row[0];
        for (int64_t k = 1; k < K; ++k) {
            if (row[k] < mn) mn = row[k];
            if (row[k] > mx) mx = row[k];
        }
        if (mn > 0.0f) mn = 0.0f;
        if (mx < 0.0f) mx = 0.0f;
        float s = (mx - mn) / 255.0f;
        if (s < FLT_EPSILON) s = FLT_EPSILON;
        float zf = -128.0f - rintf(mn / s);
        zf = clampf_(zf, -128.0f, 127.0f);
        int32_t z = (int32_t)zf;
        scale[m] = s;
        zp[m] = z;
        if (xq) {
            const float inv = 1.0f / s;
            const float fz = (float)z;
            for (int64_t k = 0; k < K; ++k) {
                float c = clampf_(rintf(row[k] * inv) + fz, -128.0f, 127.0f);
                xq[m * K + k] = (int8_t)(int)c;
            }
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------- integer contraction */

/*
 * c[m, n] = sum_k a[m, k] * b[n, k], exact in int64: the integer core of
 * the q8ta_q8csw and dq8ca linears (int8 activations times int8 weights
 * stored [out, in]).
 */
int orc_gemm_i8_i64(const int8_t *a, const int8_t *b, int64_t M, int64_t N,
                    int64_t K, int64_t *c)
{
    if (M < 0 || N < 0 || K < 0) return ORC_BAD;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            int64_t acc = 0;
            for (int64_t k = 0; k < K; ++k)
                acc += (int64_t)a[m * K + k] * (int64_t)b[n * K + k];
            c[m * N + n] = acc;
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------- W8A16 */

/*
 * Weight-only linear, [tiny-llm quant] Step 4.6 docstring: the per-channel
 * scale factors out of the matmul exactly,
 *     y[m, n] = s[n] * sum_k x[m, k] * q[n, k]   (+ bias[n])
 * x and bias are bf16 bit patterns, read exactly as float; the sum is fp64
 * of exact products, the bias ([Ming INT8 linear] Int8Linear keeps one)
 * is added once. tol[m, n] (may be NULL) receives the sum of the addends'
 * magnitudes, |s[n]| * sum_k |x q| + |bias[n]|, the scale of the rounding
 * error a correct fp32 kernel can make.
 */
int orc_linear_w8a16(const uint16_t *x, int64_t M, int64_t K, const int8_t *q,
                     const float *scale, const uint16_t *bias, int64_t N,
                     double *y, double *tol)
{
    if (M < 0 || N < 0 || K < 0) return ORC_BAD;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0, mag = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double p = (double)bf16_to_float_(x[m * K + k]) * (double)q[n * K + k];
                acc += p;
                mag += fabs(p);
            }
            double b = bias ? (double)bf16_to_float_(bias[n]) : 0.0;
            y[m * N + n] = (double)scale[n] * acc + b;
            if (tol) tol[m * N + n] = fabs((double)scale[n]) * mag + fabs(b);
        }
    }
    return ORC_OK;
}

/*
 * The other side of the factorization, [Ming INT8 linear] Int8Linear.forward
 * and [tiny-llm quant] dequantize: w = q * s[n] first, then the linear.
 * Here in fp64 (the products q * s are exact in fp64), so this and
 * orc_linear_w8a16 agree to fp64 rounding; used to pin the identity.
 */
int orc_linear_w8a16_dequant_first(const uint16_t *x, int64_t M, int64_t K,
                                   const int8_t *q, const float *scale,
                                   const uint16_t *bias, int64_t N, double *y)
{
    if (M < 0 || N < 0 || K < 0) return ORC_BAD;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double wdq = (double)q[n * K + k] * (double)scale[n];
                acc += (double)bf16_to_float_(x[m * K + k]) * wdq;
            }
            y[m * N + n] = acc + (bias ? (double)bf16_to_float_(bias[n]) : 0.0);
        }
    }
    return ORC_OK;
}

/* ----------------------------------------------- W8A8, static per-tensor act */

/*
 * linear_q8ta_q8csw, one or two passes, [SmolVLM q8 recipe] module
 * docstring and Q8Linear.forward: y = W8 . dq(q(x, s1)) + W8 . dq(q(r, s2)),
 * r = x - dq(q(x, s1)), the same int8 weight in both passes, bias once.
 * With dq(v) = (v - z) * s and the weight dequantized per channel
 * (q[n, k] * ws[n]), each pass is ws[n] * s_p * sum_k (xq_p - z_p) q, and
 * sum_k (xq - z) q = acc - z * wsum[n] with acc = sum_k xq q (the fold that
 * the op's weight_sums argument exists for). In fp64:
 *     y = ws[n] * (s1 * A1 + s2 * A2) + bias[n],  A_p = acc_p - z_p * wsum[n]
 * wsum is recomputed here from q (not taken from the caller), xq1/xq2 come
 * from orc_quantize_act_per_tensor. Optional outputs (NULL to skip): xq1,
 * xq2 [M, K], acc1, acc2 [M, N] (int64), tol [M, N] = |ws| * (s1 sum|xq1 - z1||q|
 * + s2 sum|xq2 - z2||q|) + |bias|.
 */
int orc_linear_q8ta_q8csw(const float *x, int64_t M, int64_t K, float s1,
                          int32_t z1, int two_pass, float s2, int32_t z2,
                          const int8_t *q, const float *wscale,
                          const float *bias, int64_t N, double *y,
                          int8_t *xq1_out, int8_t *xq2_out, int64_t *acc1_out,
                          int64_t *acc2_out, double *tol)
{
    if (M < 0 || N < 0 || K < 0) return ORC_BAD;
    int8_t *xq1 = (int8_t *)malloc((size_t)(M * K > 0 ? M * K : 1));
    int8_t *xq2 = (int8_t *)malloc((size_t)(M * K > 0 ? M * K : 1));
    if (!xq1 || !xq2) { free(xq1); free(xq2); return ORC_BAD; }
    int rc = orc_quantize_act_per_tensor(x, M * K, s1, z1, two_pass, s2, z2, xq1,
                                         two_pass ? xq2 : NULL);
    if (rc != ORC_OK) { free(xq1); free(xq2); return rc; }
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            int64_t acc1 = 0, acc2 = 0, ws = 0;
            double mag1 = 0.0, mag2 = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                int64_t w = q[n * K + k];
                ws += w;
                acc1 += (int64_t)xq1[m * K + k] * w;
                mag1 += fabs((double)((int64_t)xq1[m * K + k] - z1) * (double)w);
                if (two_pass) {
                    acc2 += (int64_t)xq2[m * K + k] * w;
                    mag2 += fabs((double)((int64_t)xq2[m * K + k] - z2) * (double)w);
                }
            }
            int64_t A1 = acc1 - (int64_t)z1 * ws;
            int64_t A2 = two_pass ? acc2 - (int64_t)z2 * ws : 0;
            double b = bias ? (double)bias[n] : 0.0;
            double inner = (double)s1 * (double)A1 + (two_pass ? (double)s2 * (double)A2 : 0.0);
            y[m * N + n] = (double)wscale[n] * inner + b;
            if (acc1_out) acc1_out[m * N + n] = acc1;
            if (acc2_out && two_pass) acc2_out[m * N + n] = acc2;
            if (tol)
                tol[m * N + n] = fabs((double)wscale[n]) *
                                     ((double)s1 * mag1 + (two_pass ? (double)s2 * mag2 : 0.0)) +
                                 fabs(b);
        }
    }
    if (xq1_out) memcpy(xq1_out, xq1, (size_t)(M * K));
    if (xq2_out && two_pass) memcpy(xq2_out, xq2, (size_t)(M * K));
    free(xq1);
    free(xq2);
    return ORC_OK;
}

/*
 * Q8Linear.forward of [SmolVLM q8 recipe] as printed, in fp64: dequantize
 * the weight per channel, dequantize the (re)quantized activations per
 * tensor, linear of each pass, bias in the first. Takes the codes xq1/xq2
 * (from orc_quantize_act_per_tensor) so that the factorized form above can
 * be checked against it.
 */
int orc_linear_q8ta_dequant_first(const int8_t *xq1, const int8_t *xq2,
                                  int64_t M, int64_t K, float s1, int32_t z1,
                                  int two_pass, float s2, int32_t z2,
                                  const int8_t *q, const float *wscale,
                                  const float *bias, int64_t N, double *y)
{
    if (M < 0 || N < 0 || K < 0) return ORC_BAD;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            double y1 = 0.0, y2 = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double w = (double)q[n * K + k] * (double)wscale[n];
                y1 += ((double)xq1[m * K + k] - (double)z1) * (double)s1 * w;
                if (two_pass)
                    y2 += ((double)xq2[m * K + k] - (double)z2) * (double)s2 * w;
            }
            y[m * N + n] = y1 + (bias ? (double)bias[n] : 0.0) + y2;
        }
    }
    return ORC_OK;
}

/* --------------------------------------------------- W8A8, dynamic per-row act */

/*
 * linear_dq8ca, [ExecuTorch PR 8da4w]: choose_qparams_affine per row, then
 * out[m, n] = s[m] * sum_k (xq[m, k] - z[m]) * dequant(w)[n, k] (+ bias[n]).
 *
 * wfmt 0 (int8 per-channel weights, group 0): dequant(w) = q[n, k] * ws[n], so
 *     y = s[m] * ws[n] * (acc - z[m] * wsum[n]) + bias[n].
 * wfmt 1 (q4gsw, group g): dequant(w) = q4[n, k] * gs[n, k / g], so per group
 *     A_g = sum_{k in g} xq q4 - z[m] * gsum[n, g]   (exact integers)
 *     y = s[m] * sum_g gs[n, g] * A_g + bias[n]      (fp64)
 * wsum/gsum are recomputed here from the codes. Optional outputs (NULL to
 * skip): x_scale [M], x_zp [M], xq [M, K], tol [M, N] (the sum of the
 * addends' magnitudes, s[m] * sum |gs| |xq - z| |q| + |bias|).
 */
int orc_linear_dq8ca(const float *x, int64_t M, int64_t K, int wfmt,
                     const void *wq, const float *wscale, int64_t group,
                     const float *bias, int64_t N, double *y, float *x_scale,
                     int32_t *x_zp, int8_t *xq_out, double *tol)
{
    if (M < 0 || N < 0 || K <= 0) return ORC_BAD;
    if (wfmt == 0 && group != 0) return ORC_BAD;
    if (wfmt == 1 && (group <= 0 || K % group != 0 || group % 2 != 0)) return ORC_BAD;
    if (wfmt != 0 && wfmt != 1) return ORC_BAD;
    float *s = (float *)malloc((size_t)(M > 0 ? M : 1) * sizeof(float));
    int32_t *z = (int32_t *)malloc((size_t)(M > 0 ? M : 1) * sizeof(int32_t));
    int8_t *xq = (int8_t *)malloc((size_t)(M * K > 0 ? M * K : 1));
    if (!s || !z || !xq) { free(s); free(z); free(xq); return ORC_BAD; }
    orc_choose_qparams_rows(x, M, K, s, z, xq);
    const int64_t G = (wfmt == 1) ? K / group : 1;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0, mag = 0.0;
            if (wfmt == 0) {
                const int8_t *q = (const int8_t *)wq;
                int64_t dot = 0, ws = 0;
                for (int64_t k = 0; k < K; ++k) {
                    int64_t w = q[n * K + k];
                    dot += (int64_t)xq[m * K + k] * w;
                    ws += w;
                    mag += fabs((double)((int64_t)xq[m * K + k] - z[m]) * (double)w);
                }
                int64_t A = dot - (int64_t)z[m] * ws;
                acc = (double)wscale[n] * (double)A;
                mag *= fabs((double)wscale[n]);
            } else {
                const uint8_t *q4 = (const uint8_t *)wq;
                for (int64_t g = 0; g < G; ++g) {
                    int64_t dot = 0, gsm = 0;
                    double gmag = 0.0;
                    for (int64_t j = 0; j < group; ++j) {
                        int64_t k = g * group + j;
                        int64_t w = q4_at_(q4, K, n, k);
                        dot += (int64_t)xq[m * K + k] * w;
                        gsm += w;
                        gmag += fabs((double)((int64_t)xq[m * K + k] - z[m]) * (double)w);
                    }
                    int64_t A = dot - (int64_t)z[m] * gsm;
                    acc += (double)wscale[n * G + g] * (double)A;
                    mag += fabs((double)wscale[n * G + g]) * gmag;
                }
            }
            double b = bias ? (double)bias[n] : 0.0;
            y[m * N + n] = (double)s[m] * acc + b;
            if (tol) tol[m * N + n] = fabs((double)s[m]) * mag + fabs(b);
        }
    }
    if (x_scale) memcpy(x_scale, s, (size_t)M * sizeof(float));
    if (x_zp) memcpy(x_zp, z, (size_t)M * sizeof(int32_t));
    if (xq_out) memcpy(xq_out, xq, (size_t)(M * K));
    free(s);
    free(z);
    free(xq);
    return ORC_OK;
}

/*
 * The printed form of the 8da4w fold, in fp64: out[m, n] = s[m] *
 * sum_k (xq[m, k] - z[m]) * dequant(w)[n, k], with dequant(w) the float
 * weight (q * ws[n] or q4 * gs[n, k / g]) formed first. Takes xq, s, z as
 * inputs so the grouped integer form above can be checked against it.
 */
int orc_linear_dq8ca_dequant_first(const int8_t *xq, const float *xs,
                                   const int32_t *xz, int64_t M, int64_t K,
                                   int wfmt, const void *wq,
                                   const float *wscale, int64_t group,
                                   const float *bias, int64_t N, double *y)
{
    if (M < 0 || N < 0 || K <= 0) return ORC_BAD;
    const int64_t G = (wfmt == 1) ? K / group : 1;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double wdq;
                if (wfmt == 0)
                    wdq = (double)((const int8_t *)wq)[n * K + k] * (double)wscale[n];
                else
                    wdq = (double)q4_at_((const uint8_t *)wq, K, n, k) *
                          (double)wscale[n * G + k / group];
                acc += ((double)xq[m * K + k] - (double)xz[m]) * wdq;
            }
            y[m * N + n] = (double)xs[m] * acc + (bias ? (double)bias[n] : 0.0);
        }
    }
    return ORC_OK;
}

/* ---------------------------------------------------- static calibration */

/*
 * Running per-tensor (min, max) of a static activation observer,
 * [SmolVLM q8 recipe] act_observer / Recorder / calibrate: state = {min, max},
 * (+inf, -inf) before anything is observed, folded with every element fed.
 * x is [rows, cols]; with seq > 0 the row at position 0 of every sequence of
 * seq rows (r % seq == 0, the attention-sink position the Recorder drops) is
 * skipped. residual != 0 observes the two-pass recipe's second run instead:
 * r = x - fake_quant(x, s1, z1), fake_quant = (clamp(round(x * (1/s1)) + z1,
 * -128, 127) - z1) * s1, each binary32 operation rounded on its own (the same
 * residual the per-tensor activation quantizer above forms).
 */
int orc_minmax_observe(const float *x, int64_t rows, int64_t cols, int64_t seq,
                       int residual, float s1, int32_t z1, float *state)
{
    if (rows < 0 || cols < 0 || seq < 0 || (residual && !(s1 > 0.0f))) return ORC_BAD;
    const float inv1 = residual ? 1.0f / s1 : 0.0f;
    const float fz1 = (float)z1;
    float mn = state[0], mx = state[1];
    for (int64_t r = 0; r < rows; ++r) {
        if (seq > 0 && r % seq == 0) continue;
        for (int64_t c = 0; c < cols; ++c) {
            float v = x[r * cols + c];
            if (residual) {
                float q = clampf_(rintf(v * inv1) + fz1, -128.0f, 127.0f);
                float t = (q - fz1) * s1;
                v = v - t;
            }
            if (v < mn) mn = v;
            if (v > mx) mx = v;
        }
    }
    state[0] = mn;
    state[1] = mx;
    return ORC_OK;
}

/*
 * Per-tensor affine int8 qparams of an observer's (min, max),
 * [SmolVLM q8 recipe] qparams (MinMaxObserver.calculate_qparams):
 * mn = min(min, 0), mx = max(max, 0), s = max((mx - mn) / 255, FLT_EPSILON),
 * z = clamp(-128 - round(mn / s), -128, 127), in binary32. An observer that
 * saw nothing (min > max) gives the observer's defaults s = 1, z = 0.
 */
int orc_minmax_qparams(const float *state, float *scale, int32_t *zp)
{
    if (!(state[0] <= state[1])) {
        *scale = 1.0f;
        *zp = 0;
        return ORC_OK;
    }
    float mn = state[0] < 0.0f ? state[0] : 0.0f;
    float mx = state[1] > 0.0f ? state[1] : 0.0f;
    float s = (mx - mn) / 255.0f;
    if (s < FLT_EPSILON) s = FLT_EPSILON;
    float zf = clampf_(-128.0f - rintf(mn / s), -128.0f, 127.0f);
    *scale = s;
    *zp = (int32_t)zf;
    return ORC_OK;
}

/* ------------------------------------------------------------------- GPTQ */

/*
 * GPTQ for the int8 weight grid, [SmolVLM q8 recipe] gptq_int8 (Frantar et al.),
 * in binary64 throughout. The page leaves the order of its library reductions
 * (Cholesky, the inverse, the block product, the diagonal mean) to LAPACK/BLAS;
 * the reading here fixes each to a plain ascending sum that starts at 0 and is
 * subtracted (or used) once complete, with every multiply and add rounded on
 * its own:
 *
 *   chol(A) = L lower, column by column: L[j][j] = sqrt(A[j][j] - sum_{k<j}
 *     L[j][k]^2), L[i][j] = (A[i][j] - sum_{k<j} L[i][k] L[j][k]) / L[j][j];
 *   X = L^-1 row by row: X[j][j] = 1 / L[j][j], X[i][j] = -(sum_{k=j}^{i-1}
 *     L[i][k] X[k][j]) / L[i][i];
 *   A^-1 = X^T X: (A^-1)[i][j] = sum_{k>=max(i,j)} X[k][i] X[k][j];
 *   hinv = chol(H^-1)^T (upper, hinv^T hinv = H^-1).
 *
 * Matrices are row-major double; L, X, A^-1 are K x K. Returns ORC_BAD if a
 * pivot is not positive (H not positive definite after damping).
 */
static int chol_lower_(const double *A, int64_t K, double *L)
{
    for (int64_t i = 0; i < K * K; ++i) L[i] = 0.0;
    for (int64_t j = 0; j < K; ++j) {
        double acc = 0.0;
        for (int64_t k = 0; k < j; ++k) acc = acc + L[j * K + k] * L[j * K + k];
        const double d = A[j * K + j] - acc;
        if (!(d > 0.0)) return ORC_BAD;
        const double ljj = sqrt(d);
        L[j * K + j] = ljj;
#pragma omp parallel for schedule(static)
        for (int64_t i = j + 1; i < K; ++i) {
            double a = 0.0;
            for (int64_t k = 0; k < j; ++k) a = a + L[i * K + k] * L[j * K + k];
            L[i * K + j] = (A[i * K + j] - a) / ljj;
        }
    }
    return ORC_OK;
}

/* hinv (upper, row-major) of the damped Hessian Hd: chol(chol_inverse(chol(Hd)))^T. */
int orc_gptq_hinv(const double *Hd, int64_t K, double *hinv)
{
    if (K <= 0) return ORC_BAD;
    double *L = malloc(sizeof(double) * K * K);
    double *X = malloc(sizeof(double) * K * K);
    double *Ai = malloc(sizeof(double) * K * K);
    int rc = ORC_BAD;
    if (!L || !X || !Ai) goto out;
    if (chol_lower_(Hd, K, L) != ORC_OK) goto out;
    for (int64_t i = 0; i < K * K; ++i) X[i] = 0.0;
    for (int64_t i = 0; i < K; ++i) {
        X[i * K + i] = 1.0 / L[i * K + i];
#pragma omp parallel for schedule(static)
        for (int64_t j = 0; j < i; ++j) {
            double a = 0.0;
            for (int64_t k = j; k < i; ++k) a = a + L[i * K + k] * X[k * K + j];
            X[i * K + j] = -a / L[i * K + i];
        }
    }
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < K; ++i)
        for (int64_t j = 0; j < K; ++j) {
            const int64_t k0 = i > j ? i : j;
            double a = 0.0;
            for (int64_t k = k0; k < K; ++k) a = a + X[k * K + i] * X[k * K + j];
            Ai[i * K + j] = a;
        }
    if (chol_lower_(Ai, K, L) != ORC_OK) goto out;
    for (int64_t i = 0; i < K; ++i)
        for (int64_t j = 0; j < K; ++j) hinv[i * K + j] = L[j * K + i];
    rc = ORC_OK;
out:
    free(L);
    free(X);
    free(Ai);
    return rc;
}

/*
 * The damped Hessian of gptq_int8: dead = (H[d][d] == 0) gets H[d][d] = 1 and
 * its weight column zeroed (done by the caller), then damp * mean(diag H) is
 * added to the diagonal, the mean an ascending sum divided by K.
 */
int orc_gptq_damp(const double *H, int64_t K, double damp, double *Hd, uint8_t *dead)
{
    if (K <= 0) return ORC_BAD;
    for (int64_t i = 0; i < K * K; ++i) Hd[i] = H[i];
    for (int64_t k = 0; k < K; ++k) {
        dead[k] = Hd[k * K + k] == 0.0;
        if (dead[k]) Hd[k * K + k] = 1.0;
    }
    double sum = 0.0;
    for (int64_t k = 0; k < K; ++k) sum = sum + Hd[k * K + k];
    const double c = damp * (sum / (double)K);
    for (int64_t k = 0; k < K; ++k) Hd[k * K + k] = Hd[k * K + k] + c;
    return ORC_OK;
}

/*
 * gptq_int8 proper, given hinv and the per-channel scales (the SYM127_5 weight
 * quantizer's, amax / 127.5 in binary32, used as doubles). Columns in blocks of
 * `block`; inside a block column i of row n: qc = clamp(round(w/s), -128, 127)
 * (round half to even), e = (w - qc s) / hinv[i][i], then w[j] -= e hinv[i][j]
 * for the block's columns j >= i; after the block, w[j] -= sum_t e_t hinv[t][j]
 * for every later column j (the ascending dot product over the block's t,
 * subtracted once). Rows are independent. wsum (may be NULL) = sum of codes.
 * rows: a list of the rows to compute (NULL: all N, written at their index);
 * with a list, row r of the output is row rows[r] of w.
 */
int orc_gptq_quantize(const float *w, int64_t N, int64_t K, const uint8_t *dead,
                      const double *hinv, const float *scale, int64_t block,
                      const int64_t *rows, int64_t nrows, int8_t *q, int32_t *wsum)
{
    if (N < 0 || K <= 0 || block <= 0) return ORC_BAD;
    const int64_t R = rows ? nrows : N;
    int bad = 0;
#pragma omp parallel for schedule(dynamic)
    for (int64_t r = 0; r < R; ++r) {
        const int64_t n = rows ? rows[r] : r;
        double *wr = malloc(sizeof(double) * K);
        double *err = malloc(sizeof(double) * block);
        if (!wr || !err) {
            bad = 1;
            free(wr);
            free(err);
            continue;
        }
        const double s = (double)scale[n];
        for (int64_t k = 0; k < K; ++k) wr[k] = dead[k] ? 0.0 : (double)w[n * K + k];
        int64_t total = 0;
        for (int64_t i1 = 0; i1 < K; i1 += block) {
            const int64_t i2 = i1 + block < K ? i1 + block : K;
            for (int64_t i = i1; i < i2; ++i) {
                const double col = wr[i];
                double qc = nearbyint(col / s);
                if (qc < -128.0) qc = -128.0;
                if (qc > 127.0) qc = 127.0;
                q[r * K + i] = (int8_t)(int)qc;
                total += (int)qc;
                const double e = (col - qc * s) / hinv[i * K + i];
                for (int64_t j = i; j < i2; ++j) wr[j] = wr[j] - e * hinv[i * K + j];
                err[i - i1] = e;
            }
            for (int64_t j = i2; j < K; ++j) {
                double a = 0.0;
                for (int64_t t = i1; t < i2; ++t) a = a + err[t - i1] * hinv[t * K + j];
                wr[j] = wr[j] - a;
            }
        }
        if (wsum) wsum[r] = (int32_t)total;
        free(wr);
        free(err);
    }
    return bad ? ORC_BAD : ORC_OK;
}

/* Threads of the OpenMP loops above (n >= 1); the results do not depend on it. */
int orc_set_threads(int n)
{
    if (n < 1) return ORC_BAD;
    omp_set_num_threads(n);
    return ORC_OK;
}
