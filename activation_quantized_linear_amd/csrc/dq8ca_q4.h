// 8da4w linear: 4-bit group weights, dynamic per-row int8 activations
// (internal to libaql.so). Returns hipSuccess or the launch error; arguments
// are validated by the C ABI layer.
#pragma once

#include "common.h"

namespace aql {

// 4-bit group-32 weights, dynamic per-row activations. M <= kQ4StreamMaxM reads
// xq in the permute8 order, larger M the bf16 differences xd (see
// launch_choose_qparams_rows).
constexpr int64_t kQ4StreamMaxM = 16;
// M <= kQ4FewMaxM and K <= kQ4FewMaxK: the few-rows kernel (group sums on the
// matrix cores, all of a wave's K in flight); the codes are in the permute8
// order as well
constexpr int64_t kQ4FewMaxM = 4;
constexpr int64_t kQ4FewMaxK = 8192;
struct Q4Args {
  const int8_t *xq;     // [M, K] int8, permute8 order (M <= 16)
  const uint16_t *xd;   // [M, K] bf16 xq - zp, natural order (M > 16)
  const float *xs;      // [M]
  const int32_t *xz;    // [M]
  const uint8_t *q4;    // [N, K/2] packed nibbles
  const float *gs;      // [N, K/32]
  const int32_t *gsum;  // [N, K/32]
  const float *bias;    // [N] or null
  float *y;             // [M, N]
  int64_t M, N, K;
};
hipError_t launch_dq8ca_q4(const Q4Args &a, hipStream_t st);

}  // namespace aql
