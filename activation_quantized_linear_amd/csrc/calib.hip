// Static per-tensor activation calibration on the device.
//
// SmolVLM q8 recipe, act_observer / Recorder / calibrate: every linear has one
// min/max observer that folds in everything it is fed over the calibration
// batches (the row at position 0 of a sequence, the attention sink, may be
// left out), and a two-pass linear has a second observer fed with each
// input's first-pass rounding error x - fake_quant(x, s1, z1). qparams turns
// an observer into the per-tensor affine (scale, zero point).
//
// The running (min, max) lives in two device floats, so a calibration loop
// never leaves the stream. A workgroup reduces its rows with the same wave and
// workgroup min/max reductions as the per-row qparams kernel and folds its
// result into the state with one compare-and-swap loop per bound: min and max
// are exact, so the order in which workgroups land does not matter.
#include "calib.h"

#include <float.h>
#include <math.h>

namespace aql {
namespace {

__device__ __forceinline__ void atomic_min_f32(float *addr, float v) {
  unsigned int *a = reinterpret_cast<unsigned int *>(addr);
  unsigned int old = __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  while (v < __uint_as_float(old)) {
    const unsigned int prev = atomicCAS(a, old, __float_as_uint(v));
    if (prev == old) break;
    old = prev;
  }
}

__device__ __forceinline__ void atomic_max_f32(float *addr, float v) {
  unsigned int *a = reinterpret_cast<unsigned int *>(addr);
  unsigned int old = __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  while (v > __uint_as_float(old)) {
    const unsigned int prev = atomicCAS(a, old, __float_as_uint(v));
    if (prev == old) break;
    old = prev;
  }
}

__global__ void k_minmax_reset(float *state) {
  state[0] = INFINITY;
  state[1] = -INFINITY;
}

// The residual is the per-tensor activation quantizer's: a rounded multiply
// by the reciprocal scale, round half to even, clamp, then (q - z1) * s1 and
// x - t as separately rounded operations.
#pragma clang fp contract(off)
__device__ __forceinline__ float residual_of(float v, float s1, float inv1, float fz1) {
  const float q = clamp_code(rintf(v * inv1) + fz1, -128.0f, 127.0f);
  return v - (q - fz1) * s1;
}

// One workgroup folds whole rows, rows b, b + G, ...; its 256 threads stride
// over a row's float4s.
template <bool RESID>
__global__ __launch_bounds__(256) void k_minmax_observe(const float4 *__restrict__ x, int64_t rows,
                                                        int64_t vpr, int64_t seq, float s1,
                                                        float inv1, float fz1,
                                                        float *__restrict__ state) {
  __shared__ float red[4];
  float mn = INFINITY, mx = -INFINITY;
  for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
    if (seq > 0 && r % seq == 0) continue;  // uniform
    const float4 *row = x + r * vpr;
    for (int64_t j = threadIdx.x; j < vpr; j += 256) {
      f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(row + j));
      if constexpr (RESID) {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = residual_of(v[e], s1, inv1, fz1);
      }
      mn = fminf(mn, fminf(fminf(v[0], v[1]), fminf(v[2], v[3])));
      mx = fmaxf(mx, fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])));
    }
  }
  mn = group_reduce_min<256>(mn, red);
  mx = group_reduce_max<256>(mx, red);
  if (threadIdx.x == 0) {
    atomic_min_f32(state, mn);
    atomic_max_f32(state + 1, mx);
  }
}

// MinMaxObserver.calculate_qparams for per-tensor affine int8, in binary32;
// an observer that saw nothing keeps its defaults (1, 0).
__global__ void k_minmax_qparams(const float *__restrict__ state, float *__restrict__ scale,
                                 int32_t *__restrict__ zp) {
  const float lo = state[0], hi = state[1];
  if (!(lo <= hi)) {
    scale[0] = 1.0f;
    zp[0] = 0;
    return;
  }
  const float mn = fminf(lo, 0.0f), mx = fmaxf(hi, 0.0f);
  const float s = fmaxf((mx - mn) / 255.0f, FLT_EPSILON);
  scale[0] = s;
  zp[0] = (int32_t)clamp_code(-128.0f - rintf(mn / s), -128.0f, 127.0f);
}

}  // namespace

hipError_t launch_minmax_reset(float *state, hipStream_t st) {
  hipLaunchKernelGGL(k_minmax_reset, dim3(1), dim3(1), 0, st, state);
  return hipGetLastError();
}

hipError_t launch_minmax_observe(const float *x, int64_t rows, int64_t cols, int64_t seq,
                                 bool residual, float s1, int32_t z1, float *state,
                                 hipStream_t st) {
  const int64_t vpr = cols / 4;
  const dim3 grid((unsigned)(rows < 2048 ? rows : 2048));
  const float inv1 = residual ? 1.0f / s1 : 0.0f;
  if (residual)
    hipLaunchKernelGGL(k_minmax_observe<true>, grid, dim3(256), 0, st,
                       reinterpret_cast<const float4 *>(x), rows, vpr, seq, s1, inv1, (float)z1,
                       state);
  else
    hipLaunchKernelGGL(k_minmax_observe<false>, grid, dim3(256), 0, st,
                       reinterpret_cast<const float4 *>(x), rows, vpr, seq, s1, inv1, (float)z1,
                       state);
  return hipGetLastError();
}

hipError_t launch_minmax_qparams(const float *state, float *scale, int32_t *zp, hipStream_t st) {
  hipLaunchKernelGGL(k_minmax_qparams, dim3(1), dim3(1), 0, st, state, scale, zp);
  return hipGetLastError();
}

}  // namespace aql
