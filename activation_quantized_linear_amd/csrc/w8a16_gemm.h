// W8A16 tiled GEMM for prefill-sized M (internal to libaql.so). Declared apart
// from common.h so the decode kernels' shared header does not change with it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace aql {

// y[M, N] bf16 = scale[n] * x[M, K] bf16 . q[N, K]^T int8 (+ bias[n] bf16);
// K <= 2^22 (32-bit buffer offsets of a 128-row tile of x).
hipError_t launch_w8a16_gemm(const uint16_t *x, int64_t M, int64_t K, const int8_t *q,
                             const float *scale, const uint16_t *bias, int64_t N, uint16_t *y,
                             hipStream_t st);

}  // namespace aql
