// Internal declarations shared by the HIP sources of libaql.so (not installed).
//
// Numerics used by every kernel:
//  * float -> integer code: rintf (v_rndne_f32, round half to even) of an IEEE
//    binary32 quotient or product, clamped in float, then converted;
//  * divisions are IEEE-correct (the library is built with
//    -fhip-fp32-correctly-rounded-divide-sqrt, no fast-math) and subnormals
//    are kept (-fno-gpu-flush-denormals-to-zero);
//  * products and sums that feed a rounding decision are never contracted
//    into fused multiply-adds (#pragma clang fp contract(off) in those kernels).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace aql {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------- launchers
// Each returns hipSuccess or the launch error. Arguments are validated by the
// C ABI layer before these are called.

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

hipError_t launch_w8a16(const uint16_t *x, int64_t M, int64_t K, const int8_t *q,
                        const float *scale, const uint16_t *bias, int64_t N, uint16_t *y,
                        hipStream_t st);

// Launch shape of the W8A16 kernel: waves per channel group (they split K),
// groups of 4 output channels per wave tile (1, 2 or 4) and blocks of 4 rows of
// x per tile (1, 2 or 4; 0 selects the single-row tile, M = 1). The single-row
// tile also takes cgroups, wave tiles along N per workgroup (1, 2 or 4), and
// xlds, the LDS bytes the workgroup copies x into (0: each wave loads its x
// from memory; else 2 K rounded up to 1 KiB for the largest K it serves).
struct W8A16Shape {
  int waves, tgroups, mblocks;
  int cgroups = 1;
  int xlds = 0;
};
W8A16Shape w8a16_shape(int64_t M, int64_t N, int64_t K);
// LDS budget for x in the single-row tile (K <= 16384), and the xlds value for
// a given K (0 past the budget).
constexpr int kW8A16MaxXlds = 32768;
int w8a16_xlds_bytes(int64_t K);
hipError_t launch_w8a16_shape(const W8A16Shape &sh, const uint16_t *x, int64_t M, int64_t K,
                              const int8_t *q, const float *scale, const uint16_t *bias,
                              int64_t N, uint16_t *y, hipStream_t st);

// One problem of a grouped W8A16 launch, as stored in the device table.
struct W8A16GroupEntry {
  const uint16_t *x;
  const int8_t *q;
  const float *scale;
  const uint16_t *bias;
  uint16_t *y;
  int64_t M, N, K;
  int32_t blk_begin;  // first grid block of this problem
  int32_t nblk;       // tiles along N
  int32_t pad[2];
};
static_assert(sizeof(W8A16GroupEntry) == 80, "table layout");

hipError_t launch_w8a16_grouped(const W8A16GroupEntry *dev_tab, int count, int total_blocks,
                                const W8A16Shape &sh, hipStream_t st);

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

// 4-bit group-32 weights, dynamic per-row activations. M <= kQ4StreamMaxM reads
// xq in the permute8 order, larger M the bf16 differences xd (see
// launch_choose_qparams_rows).
constexpr int64_t kQ4StreamMaxM = 16;
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

// ------------------------------------------------------------ device helpers

__device__ __forceinline__ float clamp_code(float v, float lo, float hi) {
  return fminf(fmaxf(v, lo), hi);
}

// float -> bf16 bit pattern, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float((uint32_t)h << 16);
}

template <int TPR>
__device__ __forceinline__ float group_reduce_max(float v, float *lds) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  if constexpr (TPR > 64) {
    const int w = (threadIdx.x % TPR) >> 6, base = (threadIdx.x / TPR) * (TPR / 64);
    if ((threadIdx.x & 63) == 0) lds[base + w] = v;
    __syncthreads();
    v = lds[base];
#pragma unroll
    for (int i = 1; i < TPR / 64; ++i) v = fmaxf(v, lds[base + i]);
    __syncthreads();
  }
  return v;
}

template <int TPR>
__device__ __forceinline__ float group_reduce_min(float v, float *lds) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fminf(v, __shfl_xor(v, o));
  if constexpr (TPR > 64) {
    const int w = (threadIdx.x % TPR) >> 6, base = (threadIdx.x / TPR) * (TPR / 64);
    if ((threadIdx.x & 63) == 0) lds[base + w] = v;
    __syncthreads();
    v = lds[base];
#pragma unroll
    for (int i = 1; i < TPR / 64; ++i) v = fminf(v, lds[base + i]);
    __syncthreads();
  }
  return v;
}

template <int TPR>
__device__ __forceinline__ int group_reduce_sum(int v, int *lds) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  if constexpr (TPR > 64) {
    const int w = (threadIdx.x % TPR) >> 6, base = (threadIdx.x / TPR) * (TPR / 64);
    if ((threadIdx.x & 63) == 0) lds[base + w] = v;
    __syncthreads();
    int s = 0;
#pragma unroll
    for (int i = 0; i < TPR / 64; ++i) s += lds[base + i];
    __syncthreads();
    v = s;
  }
  return v;
}

}  // namespace aql
