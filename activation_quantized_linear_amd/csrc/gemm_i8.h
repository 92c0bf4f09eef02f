// int8 x int8 GEMM with the W8A8 epilogues (internal to libaql.so). Returns
// hipSuccess or the launch error; arguments are validated by the C ABI layer.
#pragma once

#include "common.h"

namespace aql {

// int8 GEMM epilogues
enum GemmEpi { EPI_RAW = 0, EPI_Q8TA = 1, EPI_DQ8 = 2 };

struct GemmArgs {
  const int8_t *a1;     // [M, K] int8 (pass 1 codes, or the only A)
  const int8_t *a2;     // [M, K] int8 (pass 2 codes, two-pass only)
  const int8_t *b;      // [N, K] int8 weights
  int64_t M, N, K;
  // EPI_RAW
  int32_t *c;           // [M, N]
  // EPI_Q8TA / EPI_DQ8
  float *y;             // [M, N]
  const int32_t *wsum;  // [N]
  const float *wscale;  // [N]
  const float *bias;    // [N] or null
  float s1, s2;         // EPI_Q8TA: per-tensor act scales
  int32_t z1, z2;       // EPI_Q8TA: zero points
  const float *xs;      // EPI_DQ8: [M] per-row act scales
  const int32_t *xz;    // EPI_DQ8: [M] per-row act zero points
};
hipError_t launch_gemm_i8(const GemmArgs &a, GemmEpi epi, bool two_pass, hipStream_t st);

}  // namespace aql
