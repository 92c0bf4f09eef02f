// Quantizer launchers (internal to libaql.so): weights, per-tensor and
// per-row activations. Each returns hipSuccess or the launch error; arguments
// are validated by the C ABI layer.
#pragma once

#include "common.h"

namespace aql {

hipError_t launch_quantize_weight_int8(const void *w, bool bf16, int64_t N, int64_t K, int mode,
                                       int8_t *q, float *scale, int32_t *wsum,
                                       hipStream_t st);
hipError_t launch_quantize_weight_q4gsw(const float *w, int64_t N, int64_t K, uint8_t *q4,
                                        float *gs, int32_t *gsum, hipStream_t st);
hipError_t launch_quantize_act_per_tensor(const float *x, int64_t count, float s1, int32_t z1,
                                          bool two_pass, float s2, int32_t z2, int8_t *xq1,
                                          int8_t *xq2, hipStream_t st);
// Per-row qparams; the activation output (may be null) is, by mode: int8 codes
// xq in natural k order; int8 codes with every 8-k block stored as
// k = 0,2,4,6,1,3,5,7 (the order the streaming 4-bit kernel unpacks its weights
// in); or bf16 differences xq - zp (integers in [-255, 255], exact in bf16) in
// natural k order, the operand of the tiled 4-bit kernel.
enum QpOut { QP_CODES = 0, QP_CODES_PERM8 = 1, QP_DIFF_BF16 = 2 };
hipError_t launch_choose_qparams_rows(const float *x, int64_t M, int64_t K, float *scale,
                                      int32_t *zp, void *out, QpOut mode, hipStream_t st);

}  // namespace aql
