// Types and device helpers shared by the HIP sources of libaql.so (not
// installed); each kernel family declares its launchers in its own header.
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
