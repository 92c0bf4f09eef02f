// GPTQ for the int8 weight grid (internal to libaql.so), in binary64 with every
// sum taken in one fixed order, so that codes and the inverse-Hessian factor are
// reproducible bit for bit. Arguments are validated by the C ABI layer.
#pragma once

#include "common.h"

namespace aql {

// Largest GPTQ column block (one wave holds a block row, four columns a lane).
constexpr int kGptqMaxBlock = 256;

// Device workspace of launch_gptq_int8 for N rows, K columns and column block `block`.
size_t gptq_workspace_bytes(int64_t N, int64_t K, int64_t block);

// w [N, K] f32, H [K, K] f64 (lower triangle and diagonal read) -> q [N, K] int8,
// scale [N] f32, wsum [N] int32 (may be NULL), hinv_out [K, K] f64 (may be NULL),
// info (device int32: 0, or the 1-based column of the first non-positive pivot,
// plus K when it was in the factor of the inverse).
hipError_t launch_gptq_int8(const float *w, int64_t N, int64_t K, const double *H, double damp,
                            int block, int8_t *q, float *scale, int32_t *wsum, double *hinv_out,
                            int32_t *info, void *ws, hipStream_t st);

}  // namespace aql
