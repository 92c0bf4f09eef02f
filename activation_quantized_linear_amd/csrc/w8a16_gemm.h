// W8A16 tiled GEMM for prefill-sized M (internal to libaql.so). Declared apart
// from common.h so the decode kernels' shared header does not change with it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace aql {

// K splits of the wide tile this shape takes when a workspace is given (1:
// none): grids of fewer than 160 wide tiles with K >= 8192, split until there
// are 256 units of at least 16 stages of 64 k. The partial sums then need
// w8a16_gemm_part_bytes(M, N, K) bytes (0 when the shape is not split).
int w8a16_gemm_splits(int64_t M, int64_t N, int64_t K);
size_t w8a16_gemm_part_bytes(int64_t M, int64_t N, int64_t K);

// y[m, n] = bf16(scale[n] (part[0][m][n] + ... + part[S-1][m][n]) + bias[n]),
// the partial sums (fp32, S x M x N) added in split order.
hipError_t launch_w8a16_splitk_reduce(const float *part, int S, int64_t M, int64_t N,
                                      const float *scale, const uint16_t *bias, uint16_t *y,
                                      hipStream_t st);

// y[M, N] bf16 = scale[n] * x[M, K] bf16 . q[N, K]^T int8 (+ bias[n] bf16);
// K <= 2^22 (32-bit buffer offsets of a 128-row tile of x). part (may be
// null): device memory for the split-K partial sums; with at least
// w8a16_gemm_part_bytes bytes the shapes that split do so.
hipError_t launch_w8a16_gemm(const uint16_t *x, int64_t M, int64_t K, const int8_t *q,
                             const float *scale, const uint16_t *bias, int64_t N, uint16_t *y,
                             float *part, size_t part_bytes, hipStream_t st);

}  // namespace aql
