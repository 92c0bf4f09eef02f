// Static activation calibration (internal to libaql.so): a running per-tensor
// (min, max) on the device and its affine qparams. Each returns hipSuccess or
// the launch error; arguments are validated by the C ABI layer.
#pragma once

#include "common.h"

namespace aql {

hipError_t launch_minmax_reset(float *state, hipStream_t st);
// Fold x [rows, cols] (cols % 4 == 0) into state {min, max}; seq > 0 skips
// rows r with r % seq == 0; residual observes x - fake_quant(x, s1, z1).
hipError_t launch_minmax_observe(const float *x, int64_t rows, int64_t cols, int64_t seq,
                                 bool residual, float s1, int32_t z1, float *state,
                                 hipStream_t st);
hipError_t launch_minmax_qparams(const float *state, float *scale, int32_t *zp, hipStream_t st);

}  // namespace aql
