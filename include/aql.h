/*
 * aql.h — C ABI of the MI355X (gfx950) per-output-channel INT8 quantized
 * linear library (libaql.so).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers named "device" are HIP device pointers owned by the caller. The
 *   library never allocates, frees or synchronizes; every launch is ordered on
 *   `stream` (a hipStream_t passed as void*, NULL = the legacy default stream)
 *   and returns as soon as it is queued.
 * - Matrices are row-major and contiguous. Weights are stored [N, K] =
 *   [out_features, in_features], as the pages store a linear's weight.
 * - Device base pointers must be 16-byte aligned (AQL_ERR_ALIGN otherwise).
 * - An empty problem (M == 0 or N == 0 where the function has them) is valid:
 *   it returns AQL_OK without any HIP call, and pointers to its zero-element
 *   buffers may be NULL. K must always be at least its stated minimum.
 * - bf16 values travel as their 16-bit patterns (uint16_t).
 * - Every argument is validated before anything is launched; a rejected call
 *   launches nothing and returns a negative status. aql_last_error() then
 *   describes the first problem found (thread-local text). There is no silent
 *   fallback to another algorithm or to the host.
 * - Inputs must be finite; results for NaN/Inf inputs are unspecified.
 * - Rounding: round-half-to-even everywhere a float becomes an integer code,
 *   IEEE binary32 division where the definition divides, no flush of
 *   subnormals. Integer results (codes, zero points, weight sums, int32
 *   accumulators) are exact; float outputs carry fp32 rounding of the sums.
 *
 * Citations name the page and the section that defines the operation:
 *   [SmolVLM q8 recipe]   SmolVLM-500M-Instruct ExecuTorch WebGPU 8-bit recipe
 *                         building blocks (module docstring, weight_int8,
 *                         fake_quant, Q8Linear, fix_q8ta_fake, act_observer,
 *                         Recorder, calibrate, gptq_int8)
 *   [Ming INT8 linear]    Ming-Image-0.1-Design-ROCm-INT8 int8_linear
 *                         (QUANT_RULE, quantize_weight, Int8Linear)
 *   [tiny-llm quant]      tiny-llm quant module (Step 4.6 docstring,
 *                         quantize_per_channel, Int8Linear.forward)
 *   [ExecuTorch PR 8da4w] ExecuTorch WebGPU PR "Add linear_dq8ca_q4gsw +
 *                         choose_qparams_affine (8da4w)", Impl paragraph
 *   [flashrt schemes]     flashrt-structures schemes, W8A16Decode
 */
#ifndef AQL_H_
#define AQL_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------------ status */
#define AQL_OK 0
#define AQL_ERR_NULL (-1)      /* a required pointer is NULL */
#define AQL_ERR_SHAPE (-2)     /* a size is out of range or not a required multiple */
#define AQL_ERR_ALIGN (-3)     /* a device base pointer is not 16-byte aligned */
#define AQL_ERR_PARAM (-4)     /* a scale, zero point, mode, format or flag is invalid */
#define AQL_ERR_WORKSPACE (-5) /* workspace missing or smaller than aql_workspace_bytes() */
#define AQL_ERR_DEVICE (-6)    /* the current HIP device is not a gfx950 */
#define AQL_ERR_HIP (-7)       /* a HIP call or launch failed (message kept) */

/* ------------------------------------------------------------- enumerations */
#define AQL_F32 0  /* float32 input */
#define AQL_BF16 1 /* bfloat16 input (16-bit patterns) */

#define AQL_WQ_SYM127 0   /* scale = absmax/127,   codes in [-127, 127] */
#define AQL_WQ_SYM127_5 1 /* scale = absmax/127.5, codes in [-128, 127] */

#define AQL_W_Q8CSW 0 /* int8 weights [N, K], one fp32 scale per output channel */
#define AQL_W_Q4GSW 1 /* 4-bit group-symmetric weights, packed [N, K/2], fp32 scales [N, K/group] */

#define AQL_OP_Q8TA_Q8CSW 1 /* workspace of aql_linear_q8ta_q8csw */
#define AQL_OP_DQ8CA 2      /* workspace of aql_linear_dq8ca */
#define AQL_OP_GPTQ_INT8 3  /* workspace of aql_gptq_int8 (M = the column block) */
#define AQL_OP_W8A16 4      /* optional workspace of aql_linear_w8a16 (0: none used) */

/* Largest K accepted by the int8 paths: keeps |sum_k (xq - z) q| below 2^31. */
#define AQL_MAX_K_INT8 65536

/* Bytes of the fixed device scratch of aql_linear_q8ta_q8csw_noalloc (8 MiB:
 * M * K up to 4 Mi elements). */
#define AQL_NOALLOC_SCRATCH_BYTES (8 << 20)

/* ------------------------------------------------------------------ helpers */

/* Library version, major*10000 + minor*100 + patch. Never fails. */
int aql_version(void);

/* Text describing the last failure on the calling thread ("" if none). The
 * pointer stays valid until the next aql_* call on this thread. */
const char *aql_last_error(void);

/* Bytes of device workspace an operation needs for the given sizes (op is
 * AQL_OP_*); 0 for an unknown op or negative sizes. Workspace contents need
 * no initialization and are scratch after the call. */
size_t aql_workspace_bytes(int op, int64_t M, int64_t N, int64_t K);

/* ----------------------------------------------------------- quantizers */

/*
 * Per-output-channel symmetric int8 weight quantization.
 * [Ming INT8 linear] QUANT_RULE / quantize_weight and [tiny-llm quant]
 * quantize_per_channel (mode AQL_WQ_SYM127): scale[n] = max_k |w[n,k]| / 127,
 * q = clamp(round(w / scale), -127, 127). [SmolVLM q8 recipe] weight_int8
 * (mode AQL_WQ_SYM127_5): scale = absmax / 127.5, q = clamp(round(w /
 * scale), -128, 127). An all-zero row gets scale 1.0 and q 0 in both modes.
 *
 *   w       device, [N, K] float32 (w_dtype AQL_F32) or bf16 (AQL_BF16)
 *   q       device, [N, K] int8 codes (output)
 *   scale   device, [N] float32 (output)
 *   wsum    device, [N] int32 sum_k q[n,k] (output; may be NULL). This is the
 *           weight_sums operand of the q8ta_q8csw op ([SmolVLM q8 recipe]
 *           fix_q8ta_fake) and of aql_linear_dq8ca.
 * Errors: NULL w/q/scale (N > 0); N < 0, K < 1 or K % 4 != 0; unknown w_dtype or
 * mode; misaligned pointers.
 */
int aql_quantize_weight_int8(const void *w, int w_dtype, int64_t N, int64_t K, int mode,
                             int8_t *q, float *scale, int32_t *wsum, void *stream);

/*
 * 4-bit group-symmetric weights for aql_linear_dq8ca (AQL_W_Q4GSW).
 * [ExecuTorch PR 8da4w] consumes "4-bit group weights" with group scales but
 * prints no producer or layout; the rule here is the symmetric observer rule
 * of [SmolVLM q8 recipe] weight_int8 on the int4 range: per (n, group g)
 * gs = amax_g / 7.5, q4 = clamp(round(w / gs), -8, 7), an all-zero group gets
 * gs = 1 and q4 = 0.
 *
 *   w      device, [N, K] float32
 *   q4     device, [N, K/2] bytes: byte n*K/2 + k/2 holds k even in the low
 *          nibble and k odd in the high nibble, two's complement (output)
 *   gscale device, [N, K/group] float32 (output)
 *   gsum   device, [N, K/group] int32 sum of each group's codes (output; may be NULL)
 * Errors: group must be 32; K < 32 or K % 32 != 0; N < 0; NULL (N > 0) or
 * misaligned pointers.
 */
int aql_quantize_weight_q4gsw(const float *w, int64_t N, int64_t K, int group, uint8_t *q4,
                              float *gscale, int32_t *gsum, void *stream);

/*
 * Per-row asymmetric int8 activation qparams, optionally fused with the
 * quantization ([ExecuTorch PR 8da4w] choose_qparams_affine: per-row min/max,
 * then scale and zero point; the rule is the affine min/max one of
 * [SmolVLM q8 recipe] act_observer): mn = min(min_k x, 0),
 * mx = max(max_k x, 0), scale = max((mx - mn) / 255, FLT_EPSILON),
 * zp = clamp(-128 - round(mn / scale), -128, 127), and if xq is not NULL
 * xq = clamp(round(x * (1/scale)) + zp, -128, 127).
 *
 *   x      device, [M, K] float32
 *   scale  device, [M] float32 (output)
 *   zp     device, [M] int32 holding values in [-128, 127] (output). The page
 *          packs four int8 zero points per word to dodge a WebGPU write race;
 *          here each row owns its own int32.
 *   xq     device, [M, K] int8 (output; may be NULL)
 * Errors: NULL x/scale/zp (M > 0); M < 0, K < 1, K % 4 != 0; misaligned pointers.
 */
int aql_choose_qparams_rows(const float *x, int64_t M, int64_t K, float *scale, int32_t *zp,
                            int8_t *xq, void *stream);

/*
 * Static per-tensor affine activation quantization, one or two passes: the
 * prologue of aql_linear_q8ta_q8csw exposed as a stage.
 * [SmolVLM q8 recipe] fake_quant / Q8Linear.forward:
 * xq1 = clamp(round(x * (1/s1)) + z1, -128, 127); with two_pass,
 * r = x - (xq1 - z1) * s1 (a rounded multiply, then a rounded subtract) and
 * xq2 = clamp(round(r * (1/s2)) + z2, -128, 127).
 *
 *   x         device, [M, K] float32
 *   xq1, xq2  device, [M, K] int8 (outputs; xq2 unused and may be NULL when
 *             two_pass == 0)
 * Errors: s1 (and s2 with two_pass) not finite and > 0; z outside [-128, 127];
 * M < 0, K < 1, K % 4 != 0; NULL (M > 0) or misaligned pointers.
 */
int aql_quantize_act_per_tensor(const float *x, int64_t M, int64_t K, float s1, int32_t z1,
                                int two_pass, float s2, int32_t z2, int8_t *xq1, int8_t *xq2,
                                void *stream);

/* --------------------------------------------------------------- linears */

/*
 * Weight-only W8A16 linear. [tiny-llm quant] Step 4.6 docstring and
 * Int8Linear.forward: the per-channel scale factors out of the matmul,
 * y[m, n] = scale[n] * sum_k x[m, k] * q[n, k] (+ bias[n]), int8 -> bf16 is
 * exact (|q| <= 128 < 256). [Ming INT8 linear] Int8Linear keeps an optional
 * bias. Decode-sized M runs a streaming kernel that reads the int8 rows
 * once; larger M runs a tiled kernel ([flashrt schemes] W8A16Decode's
 * M-dispatch; both branches are HIP).
 *
 *   x      device, [M, K] bf16
 *   q      device, [N, K] int8 (from aql_quantize_weight_int8)
 *   scale  device, [N] float32
 *   bias   device, [N] bf16 (may be NULL)
 *   y      device, [M, N] bf16, fp32 accumulate, round-to-nearest-even (output)
 *   ws     device workspace (may be NULL). With at least
 *          aql_workspace_bytes(AQL_OP_W8A16, M, N, K) bytes (nonzero only for
 *          shapes of few output tiles and long rows: prefill, and 12 <= M < 64
 *          with fewer than 8192 channels and K >= 8192), the kernel splits K
 *          over more workgroups and adds their fp32 partial sums in a second
 *          launch; otherwise, or with a smaller workspace, it does not. The
 *          result is the same up to the order of the fp32 additions.
 * Errors: NULL x/q/scale/y (M, N > 0); M, N < 0; K < 16 or K % 16 != 0;
 * misaligned pointers (ws included).
 */
int aql_linear_w8a16(const uint16_t *x, int64_t M, int64_t K, const int8_t *q,
                     const float *scale, const uint16_t *bias, int64_t N, uint16_t *y,
                     void *ws, size_t ws_bytes, void *stream);

/*
 * W8A8 linear with a static per-tensor affine activation scale and an
 * optional second pass on the rounding residual (et_vk.linear_q8ta_q8csw of
 * [SmolVLM q8 recipe], module docstring and Q8Linear.forward):
 *   xq1 = q(x; s1, z1), r = x - dq(xq1), xq2 = q(r; s2, z2)
 *   y[m, n] = wscale[n] * ( s1 * sum_k (xq1 - z1) q  +  s2 * sum_k (xq2 - z2) q ) + bias[n]
 * with sum_k (xq - z) q = sum_k xq q - z * wsum[n] in exact int32, the same
 * int8 weight for both passes, the bias added once.
 *
 *   x       device, [M, K] float32
 *   q       device, [N, K] int8; wsum device [N] int32 = sum_k q[n, k];
 *           wscale device [N] float32
 *   bias    device, [N] float32 (may be NULL)
 *   y       device, [M, N] float32 (output)
 *   ws      device workspace of at least aql_workspace_bytes(AQL_OP_Q8TA_Q8CSW, M, N, K)
 *           bytes; it receives the int8 codes xq1 [M, K] then xq2 [M, K].
 * Errors: as aql_quantize_act_per_tensor, plus K < 16, K % 16 != 0 or K > AQL_MAX_K_INT8,
 * NULL q/wsum/wscale/y, workspace too small.
 */
int aql_linear_q8ta_q8csw(const float *x, int64_t M, int64_t K, float s1, int32_t z1,
                          int two_pass, float s2, int32_t z2, const int8_t *q,
                          const int32_t *wsum, const float *wscale, const float *bias, int64_t N,
                          float *y, void *ws, size_t ws_bytes, void *stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * operation, arguments and results as aql_linear_q8ta_q8csw, without the
 * workspace argument. The activation codes go to a fixed scratch array of
 * AQL_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on
 * until the process ends; nothing is allocated or freed. The caller still
 * provides x, the weights and y.
 *   Every call on one GPU shares that GPU's scratch and leaves its codes
 *   there: calls that overlap on one GPU (on different streams, or from
 *   different threads) race and give undefined results; calls ordered on one
 *   stream do not. Results are bit-identical to aql_linear_q8ta_q8csw.
 * Errors: as aql_linear_q8ta_q8csw; AQL_ERR_WORKSPACE when the call needs
 * more scratch than AQL_NOALLOC_SCRATCH_BYTES (the workspace size of
 * aql_linear_q8ta_q8csw: twice M * K rounded up to 256), checked before any
 * HIP call;
 * AQL_ERR_HIP if the scratch address cannot be obtained on the device.
 */
int aql_linear_q8ta_q8csw_noalloc(const float *x, int64_t M, int64_t K, float s1, int32_t z1,
                                  int two_pass, float s2, int32_t z2, const int8_t *q,
                                  const int32_t *wsum, const float *wscale, const float *bias,
                                  int64_t N, float *y, void *stream);

/*
 * W8A8 linear with dynamic per-row asymmetric int8 activations
 * ([ExecuTorch PR 8da4w]: choose_qparams_affine, then linear_dq8ca with
 * out[m, n] = s[m] * sum_k (xq[m, k] - z[m]) * dequant(w)[n, k]).
 *   wfmt AQL_W_Q8CSW, group 0:  dequant(w) = q[n, k] * wscale[n];
 *       y = s[m] * wscale[n] * (sum_k xq q - z[m] * wsum[n]) + bias[n]
 *   wfmt AQL_W_Q4GSW, group 32: dequant(w) = q4[n, k] * wscale[n, k/32];
 *       y = s[m] * sum_g wscale[n, g] * (sum_{k in g} xq q4 - z[m] * wsum[n, g]) + bias[n]
 * Integer parts exact, group and output scaling in fp32. Any M >= 1 (the
 * page's rows-multiple-of-4 limit does not apply).
 *
 *   x            device, [M, K] float32
 *   wq           device, int8 [N, K] (Q8CSW) or packed q4 [N, K/2] (Q4GSW)
 *   wscale       device, float32 [N] (Q8CSW) or [N, K/32] (Q4GSW)
 *   wsum         device, int32 [N] or [N, K/32]: sums of the codes (as written by
 *                the weight quantizer). The Q4GSW kernels do not read them: they
 *                form the group sums from the codes (M <= 16) or fold the zero
 *                point on the activation side (M > 16)
 *   bias         device, [N] float32 (may be NULL)
 *   y            device, [M, N] float32 (output)
 *   x_scale_out  device, [M] float32 (optional output: the row scales)
 *   x_zp_out     device, [M] int32 (optional output: the row zero points)
 *   ws           workspace of aql_workspace_bytes(AQL_OP_DQ8CA, M, N, K) bytes
 * Errors: unknown wfmt or a group other than 0 (Q8CSW) / 32 (Q4GSW); K not a
 * positive multiple of 16 (Q8CSW) / 32 (Q4GSW)
 * or K > AQL_MAX_K_INT8; NULL or misaligned pointers; workspace too small.
 */
int aql_linear_dq8ca(const float *x, int64_t M, int64_t K, int wfmt, const void *wq,
                     const float *wscale, const int32_t *wsum, int group, const float *bias,
                     int64_t N, float *y, float *x_scale_out, int32_t *x_zp_out, void *ws,
                     size_t ws_bytes, void *stream);

/* ----------------------------------------------------------- grouped W8A16 */

/*
 * Several independent W8A16 linears in one launch: the same operation as
 * aql_linear_w8a16 on each problem, with all problems' tiles in one grid, so
 * that a decode step's linears that do not feed one another (a sweep over the
 * layers' MLP weights, or up and gate sharing x) stream their weights back to
 * back instead of paying a launch and a pipeline fill per linear ([flashrt
 * schemes] W8A16Decode: the decode band is bound by reading the weights).
 *
 * Plan / execute. aql_w8a16_group_plan validates the problems on the host and
 * writes a table (aql_w8a16_group_table_bytes(count) bytes of host memory);
 * the caller copies that table unchanged into device memory (any host-to-device
 * copy) and launches with aql_linear_w8a16_grouped, passing the host table
 * (read for the grid size) and its device copy (read by the kernel). The
 * launch allocates and copies nothing, so it can be captured in a HIP graph.
 * The table holds the problems' device pointers: it stays valid while they do.
 */
typedef struct aql_w8a16_problem {
  const uint16_t *x;     /* device, [M, K] bf16 */
  const int8_t *q;       /* device, [N, K] int8 */
  const float *scale;    /* device, [N] float32 */
  const uint16_t *bias;  /* device, [N] bf16, may be NULL */
  uint16_t *y;           /* device, [M, N] bf16 (output) */
  int64_t M, N, K;       /* as in aql_linear_w8a16; M or N == 0 skips the problem */
} aql_w8a16_problem;

/* Bytes of the table for `count` problems (0 if count < 1). */
size_t aql_w8a16_group_table_bytes(int count);

/* Validate `count` problems (each as aql_linear_w8a16 would) and write the
 * table. Errors: count < 1, table NULL or smaller than
 * aql_w8a16_group_table_bytes(count) (AQL_ERR_WORKSPACE), any problem invalid
 * (its index is in aql_last_error()), more than 2^31 - 1 tiles in total. */
int aql_w8a16_group_plan(const aql_w8a16_problem *problems, int count, void *table,
                         size_t table_bytes);

/* Run a planned group. table: the host table written by aql_w8a16_group_plan;
 * dev_table: its device copy (16-byte aligned). Errors: table not written by
 * the plan function (AQL_ERR_PARAM), dev_table NULL or misaligned. A group
 * whose problems are all empty returns AQL_OK without launching. A
 * single-row group of at most 4 problems whose K all lie in the range of the
 * contiguous-pieces kernel takes its entries from the host table at launch
 * (they travel in the kernel arguments); larger groups read dev_table when
 * the kernel runs. Both tables must describe the same plan. */
int aql_linear_w8a16_grouped(const void *table, const void *dev_table, void *stream);

/* ------------------------------------------------------------ stage entry */

/*
 * The int8 x int8 -> int32 contraction core of the W8A8 linears, exposed so
 * that its accumulators can be checked bit for bit: c[m, n] = sum_k a[m, k] *
 * b[n, k] (the integer sum inside [SmolVLM q8 recipe] Q8Linear's linear of
 * dequantized operands, before any scale).
 *
 *   a  device, [M, K] int8;  b  device, [N, K] int8;  c  device, [M, N] int32 (output)
 * Errors: M, N < 0; K < 16, K % 16 != 0 or K > AQL_MAX_K_INT8; NULL (M, N > 0) or
 * misaligned pointers.
 */
int aql_gemm_i8_i32(const int8_t *a, const int8_t *b, int32_t *c, int64_t M, int64_t N,
                    int64_t K, void *stream);

/* ------------------------------------------------------ static calibration */

/*
 * Static per-tensor activation qparams, calibrated on the device
 * ([SmolVLM q8 recipe] act_observer, Recorder, calibrate, qparams): one
 * running (min, max) per observed activation, folded over any number of
 * calibration batches, then turned into the per-tensor affine int8 (s, z)
 * that aql_linear_q8ta_q8csw takes. A two-pass linear's second pair
 * (s2, z2) comes from a second observer fed with each input's first-pass
 * rounding error.
 *
 * state: device float32[2] = {min, max}; (+inf, -inf) is the empty observer.
 * All calls are ordered on `stream` and allocate nothing.
 *
 * aql_minmax_reset: state = (+inf, -inf).
 *
 * aql_minmax_observe: state = (min(state.min, min x), max(state.max, max x))
 * over x [rows, cols] float32, row-major. With seq > 0, row r is at position
 * r % seq of its sequence and the rows at position 0 are not observed (the
 * recipe's Recorder drops the attention-sink position). With residual != 0
 * each element is replaced by x - (clamp(round(x * (1/s1)) + z1, -128, 127)
 * - z1) * s1, the rounding error of the first pass formed exactly as
 * aql_quantize_act_per_tensor forms it. NaN elements are ignored.
 * Errors: rows < 0, seq < 0, cols < 0 or cols % 4 != 0; residual with s1 not
 * finite and positive or z1 outside [-128, 127]; NULL or misaligned x
 * (rows, cols > 0) / state.
 *
 * aql_minmax_qparams: scale[0], zp[0] from state by MinMaxObserver's
 * per-tensor affine rule: mn = min(min, 0), mx = max(max, 0),
 * s = max((mx - mn) / 255, FLT_EPSILON), z = clamp(-128 - round(mn / s),
 * -128, 127); an observer that saw nothing gives (1, 0). Device outputs.
 * Errors: NULL or misaligned pointers.
 *
 * aql_keep_outliers (host, no GPU): the keep-at-host-precision decision of
 * [flashrt schemes] Fp8Static.keep_outliers. amax[p] is the statistic of
 * point p (NaN: the point has none), seam[p] in [0, nseams) the seam that owns
 * it. With m the median of all positive statistics (the mean of the two
 * middle ones for an even count), keep[s] = 1 when the largest statistic of
 * seam s exceeds factor * m; factor 0, or no positive statistic, keeps
 * nothing. Arithmetic in double, as the page's Python floats.
 * Errors: npoints or nseams < 0; NULL arrays for non-zero counts; a seam
 * index out of range.
 */
int aql_minmax_reset(float *state, void *stream);
int aql_minmax_observe(const float *x, int64_t rows, int64_t cols, int64_t seq, int residual,
                       float s1, int32_t z1, float *state, void *stream);
int aql_minmax_qparams(const float *state, float *scale, int32_t *zp, void *stream);
int aql_keep_outliers(const float *amax, const int32_t *seam, int64_t npoints, int32_t nseams,
                      double factor, int32_t *keep);

/* ------------------------------------------------------------- GPTQ int8 */

/*
 * GPTQ codes for the int8 weight grid ([SmolVLM q8 recipe] gptq_int8, after
 * Frantar et al.), in binary64, on the device. The scales are the weight
 * quantizer's (AQL_WQ_SYM127_5 of the original w: amax / 127.5, fp32); the
 * codes replace its rounding to nearest:
 *   dead = (H[k][k] == 0): H[k][k] = 1 and weight column k zeroed;
 *   Hd = H + damp * mean(diag H) * I;  hinv = chol(Hd^-1)^T (upper);
 *   for each block of `block` columns, for each column i in order:
 *     q[:, i] = clamp(round(w[:, i] / s), -128, 127),
 *     e = (w[:, i] - q[:, i] s) / hinv[i][i],
 *     w[:, j] -= e hinv[i][j] for the block's later columns j;
 *   after the block, w[:, j] -= sum_t e_t hinv[t][j] for every later column j.
 * The page leaves the order of its library reductions to LAPACK/BLAS. Here
 * every sum (an element of a Cholesky factor, of the triangular inverse, of
 * the product forming Hd^-1, of a block's trailing update, the diagonal's
 * mean) is an ascending sum from 0, each product and addition rounded on its
 * own, used once complete; fp64 division and square root correctly rounded,
 * round half to even. Results are therefore reproducible bit for bit.
 *
 *   w         device, [N, K] float32
 *   H         device, [K, K] float64, symmetric; only the lower triangle and
 *             the diagonal are read
 *   damp      relative damping (the page's default 0.01), finite and >= 0
 *   block     columns per block, 1..256 (the page's default 128)
 *   q         device, [N, K] int8 codes (output)
 *   scale     device, [N] float32 (output)
 *   wsum      device, [N] int32 sums of the codes (output; may be NULL)
 *   hinv_out  device, [K, K] float64 (output; may be NULL): the upper factor,
 *             zero below the diagonal
 *   info      device, int32 (output): 0 on success; c (1-based) if pivot c of
 *             the factor of Hd was not positive; K + c if pivot c of the factor
 *             of Hd^-1 was not. Outputs are meaningless when info != 0.
 *   ws        device workspace of aql_workspace_bytes(AQL_OP_GPTQ_INT8, block, N, K)
 *             bytes (about 32 K^2 + 8 N K + 8 N block)
 * Errors: N < 0; K < 4, K % 4 != 0 or K > AQL_MAX_K_INT8; block outside
 * 1..256; damp not finite or negative; NULL or misaligned pointers; workspace
 * too small. N == 0 launches nothing.
 */
int aql_gptq_int8(const float *w, int64_t N, int64_t K, const double *H, double damp,
                  int64_t block, int8_t *q, float *scale, int32_t *wsum, double *hinv_out,
                  int32_t *info, void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------- measurement helpers */

/*
 * Not part of the method: the attainable ceilings the linears are measured
 * against on this GPU (published peaks are HBM 8 TB/s and dense int8 MFMA
 * 5.0 POP/s).
 *
 * aql_measure_read: one launch that reads `bytes` of device memory once
 * (a read-only HBM stream in the fastest shape measured here: 1 KB per wave
 * instruction, 8 in flight, nontemporal, 4 waves per CU). Time it with events
 * to get the read ceiling; rotate buffers larger than the 256 MB Infinity
 * Cache. sink: device, 4 bytes, written only in a case that does not arise for
 * ordinary data (it keeps the loads from being optimized away).
 * Errors: buf or sink NULL / misaligned; bytes < 1024, not a multiple of 1024,
 * or above 2^31 - 1024.
 *
 * aql_measure_mfma_i8: one launch of 2 waves per SIMD on every CU (256 x 8
 * waves), each issuing 16 * iters back-to-back v_mfma_i32_16x16x64_i8 (32768
 * integer ops each) on register operands: 2048 * 32768 * 16 * iters ops in total.
 * Errors: iters < 1 or > 2^30; sink NULL / misaligned.
 */
int aql_measure_read(const void *buf, int64_t bytes, uint32_t *sink, void *stream);
int aql_measure_mfma_i8(int64_t iters, int32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* AQL_H_ */
