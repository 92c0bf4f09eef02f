// Quantizers: per-output-channel int8 weights, 4-bit group weights, static
// per-tensor activations (one or two passes) and per-row asymmetric
// activation qparams. All are HBM-bound streaming kernels: one read of the
// float input, one write of the codes; a row that has to be reduced first
// (absmax, min/max) is held in registers between the reduction and the
// quantization so it is read from HBM once.
#include "quant.h"

#include <float.h>

namespace aql {
namespace {

template <bool BF16>
__device__ __forceinline__ float4 load4(const void *p, int64_t idx) {
  if constexpr (BF16) {
    const uint2 u = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(p) + idx);
    return make_float4(bf16_to_f32((uint16_t)(u.x & 0xffffu)), bf16_to_f32((uint16_t)(u.x >> 16)),
                       bf16_to_f32((uint16_t)(u.y & 0xffffu)), bf16_to_f32((uint16_t)(u.y >> 16)));
  } else {
    return *reinterpret_cast<const float4 *>(static_cast<const float *>(p) + idx);
  }
}

__device__ __forceinline__ float absmax4(float4 v) {
  return fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
}

__device__ __forceinline__ uint32_t pack4(int a, int b, int c, int d) {
  return (uint32_t)(a & 0xff) | ((uint32_t)(b & 0xff) << 8) | ((uint32_t)(c & 0xff) << 16) |
         ((uint32_t)(d & 0xff) << 24);
}

// ---------------------------------------------------------------- int8 weights
// Ming INT8 linear quantize_weight / tiny-llm quantize_per_channel (den 127,
// lo -127) and SmolVLM q8 recipe weight_int8 (den 127.5, lo -128):
// q = clamp(rint(w / s), lo, 127) with s = absmax / den (1.0 for a zero row).

__device__ __forceinline__ int wcode(float w, float s, float lo) {
  return (int)clamp_code(rintf(w / s), lo, 127.0f);
}

// The same code from r = 1 / s (IEEE, s normal): |w / s| <= 128 here, so
// t = w r is within 2^-16 of w / s (r's relative error and t's rounding, 2^-17
// each at most) and the IEEE quotient within 2^-18 of it. Unless t lies within
// 2^-10 of a half-integer, both fall strictly inside the same rounding interval
// and rint(t) is rint(w / s); those few take the division itself.
__device__ __forceinline__ int wcode_r(float w, float s, float r, float lo) {
  const float t = w * r;
  float c = rintf(t);
  if (fabsf(t - c) > 0.5f - 0x1p-10f) c = rintf(w / s);
  return (int)clamp_code(c, lo, 127.0f);
}

// TPR threads own one row (TPR = 64: a wave per row, 4 rows per workgroup;
// TPR = 256: the workgroup per row). VPT float4 vectors per thread stay in
// registers between the absmax and the quantization; VPT = 0 re-reads the
// row instead (rows longer than 16384).
template <bool BF16, int TPR, int VPT>
__global__ __launch_bounds__(256) void k_quantize_weight_int8(
    const void *__restrict__ w, int64_t N, int64_t K, float den, float lo,
    int8_t *__restrict__ q, float *__restrict__ scale, int32_t *__restrict__ wsum) {
  __shared__ float red_f[4];
  __shared__ int red_i[4];
  constexpr int RPW = 256 / TPR;
  const int t = threadIdx.x % TPR;
  const int64_t n = (int64_t)blockIdx.x * RPW + threadIdx.x / TPR;
  const bool active = n < N;
  const int64_t nvec = K >> 2;
  const int64_t base = (active ? n : 0) * K;
  uint32_t *qrow = reinterpret_cast<uint32_t *>(q + base);

  float amax = 0.0f;
  int sum = 0;
  if constexpr (VPT > 0) {
    float4 v[VPT];
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int64_t j = t + (int64_t)i * TPR;
      v[i] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (active && j < nvec) v[i] = load4<BF16>(w, base + 4 * j);
      amax = fmaxf(amax, absmax4(v[i]));
    }
    amax = group_reduce_max<TPR>(amax, red_f);
    const float s = (amax == 0.0f) ? 1.0f : amax / den;
    const float r = 1.0f / s;
    if (s >= 0x1p-126f) {  // uniform: the reciprocal path needs a normal s
#pragma unroll
      for (int i = 0; i < VPT; ++i) {
        const int64_t j = t + (int64_t)i * TPR;
        if (active && j < nvec) {
          const int a = wcode_r(v[i].x, s, r, lo), b = wcode_r(v[i].y, s, r, lo);
          const int c = wcode_r(v[i].z, s, r, lo), d = wcode_r(v[i].w, s, r, lo);
          qrow[j] = pack4(a, b, c, d);
          sum += a + b + c + d;
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < VPT; ++i) {
        const int64_t j = t + (int64_t)i * TPR;
        if (active && j < nvec) {
          const int a = wcode(v[i].x, s, lo), b = wcode(v[i].y, s, lo);
          const int c = wcode(v[i].z, s, lo), d = wcode(v[i].w, s, lo);
          qrow[j] = pack4(a, b, c, d);
          sum += a + b + c + d;
        }
      }
    }
    sum = group_reduce_sum<TPR>(sum, red_i);
    if (active && t == 0) {
      scale[n] = s;
      if (wsum) wsum[n] = sum;
    }
  } else {
    for (int64_t j = t; j < nvec; j += TPR)
      if (active) amax = fmaxf(amax, absmax4(load4<BF16>(w, base + 4 * j)));
    amax = group_reduce_max<TPR>(amax, red_f);
    const float s = (amax == 0.0f) ? 1.0f : amax / den;
    for (int64_t j = t; j < nvec; j += TPR) {
      if (!active) break;
      const float4 v = load4<BF16>(w, base + 4 * j);
      const int a = wcode(v.x, s, lo), b = wcode(v.y, s, lo);
      const int c = wcode(v.z, s, lo), d = wcode(v.w, s, lo);
      qrow[j] = pack4(a, b, c, d);
      sum += a + b + c + d;
    }
    sum = group_reduce_sum<TPR>(sum, red_i);
    if (active && t == 0) {
      scale[n] = s;
      if (wsum) wsum[n] = sum;
    }
  }
}

template <bool BF16>
hipError_t quant_w8_dispatch(const void *w, int64_t N, int64_t K, float den, float lo, int8_t *q,
                             float *scale, int32_t *wsum, hipStream_t st) {
  const int64_t nvec = K / 4;
  if (nvec <= 64 * 4) {
    const dim3 grid((unsigned)((N + 3) / 4));
    if (nvec <= 64)
      hipLaunchKernelGGL((k_quantize_weight_int8<BF16, 64, 1>), grid, dim3(256), 0, st, w, N, K,
                         den, lo, q, scale, wsum);
    else if (nvec <= 128)
      hipLaunchKernelGGL((k_quantize_weight_int8<BF16, 64, 2>), grid, dim3(256), 0, st, w, N, K,
                         den, lo, q, scale, wsum);
    else
      hipLaunchKernelGGL((k_quantize_weight_int8<BF16, 64, 4>), grid, dim3(256), 0, st, w, N, K,
                         den, lo, q, scale, wsum);
  } else {
    const dim3 grid((unsigned)N);
    if (nvec <= 256 * 2)
      hipLaunchKernelGGL((k_quantize_weight_int8<BF16, 256, 2>), grid, dim3(256), 0, st, w, N, K,
                         den, lo, q, scale, wsum);
    else if (nvec <= 256 * 4)
      hipLaunchKernelGGL((k_quantize_weight_int8<BF16, 256, 4>), grid, dim3(256), 0, st, w, N, K,
                         den, lo, q, scale, wsum);
    else if (nvec <= 256 * 8)
      hipLaunchKernelGGL((k_quantize_weight_int8<BF16, 256, 8>), grid, dim3(256), 0, st, w, N, K,
                         den, lo, q, scale, wsum);
    else if (nvec <= 256 * 16)
      hipLaunchKernelGGL((k_quantize_weight_int8<BF16, 256, 16>), grid, dim3(256), 0, st, w, N,
                         K, den, lo, q, scale, wsum);
    else
      hipLaunchKernelGGL((k_quantize_weight_int8<BF16, 256, 0>), grid, dim3(256), 0, st, w, N, K,
                         den, lo, q, scale, wsum);
  }
  return hipGetLastError();
}

// ------------------------------------------------------------ q4gsw weights
// One thread per (row, group of 32): gs = amax / 7.5 (1.0 for a zero group),
// q4 = clamp(rint(w / gs), -8, 7), packed two per byte (k even low nibble).
__global__ __launch_bounds__(256) void k_quantize_weight_q4gsw(
    const float *__restrict__ w, int64_t N, int64_t K, uint8_t *__restrict__ q4,
    float *__restrict__ gs, int32_t *__restrict__ gsum) {
  const int64_t G = K / 32;
  const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= N * G) return;
  const int64_t n = id / G, g = id % G;
  const float4 *src = reinterpret_cast<const float4 *>(w + n * K + g * 32);
  float4 v[8];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[i] = src[i];
    amax = fmaxf(amax, absmax4(v[i]));
  }
  const float s = (amax == 0.0f) ? 1.0f : amax / 7.5f;
  uint32_t words[4];
  int sum = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float e[8] = {v[2 * i].x, v[2 * i].y, v[2 * i].z, v[2 * i].w,
                        v[2 * i + 1].x, v[2 * i + 1].y, v[2 * i + 1].z, v[2 * i + 1].w};
    uint32_t word = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int c = (int)clamp_code(rintf(e[j] / s), -8.0f, 7.0f);
      sum += c;
      word |= (uint32_t)(c & 0xf) << (4 * j);
    }
    words[i] = word;
  }
  *reinterpret_cast<uint4 *>(q4 + n * (K / 2) + g * 16) =
      make_uint4(words[0], words[1], words[2], words[3]);
  gs[id] = s;
  if (gsum) gsum[id] = sum;
}

// ------------------------------------------------------ per-tensor activations
// SmolVLM q8 recipe fake_quant / Q8Linear.forward: xq = clamp(rint(x * inv) + z),
// inv = 1/s; the two-pass residual r = x - (xq1 - z1) * s1 is a rounded
// multiply followed by a rounded subtract (no FMA contraction).
#pragma clang fp contract(off)
__device__ __forceinline__ float act_code(float v, float inv, float z) {
  return clamp_code(rintf(v * inv) + z, -128.0f, 127.0f);
}

// A wave handles 64 U float4 (U KB) per round: U loads of 64 lanes x 16 B, each
// a contiguous 1 KB, all in flight before any code is formed; each load's 64
// codes go out as one contiguous 256-byte store per pass.
template <int U, bool TWO>
__global__ __launch_bounds__(256) void k_quantize_act_per_tensor(
    const float4 *__restrict__ x, int64_t nvec, float s1, float inv1, float z1, float inv2,
    float z2, uint32_t *__restrict__ xq1, uint32_t *__restrict__ xq2) {
  const int lane = threadIdx.x & 63;
  const int64_t nw = (int64_t)gridDim.x * (blockDim.x >> 6);
  for (int64_t base = ((int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6)) * (64 * U);
       base < nvec; base += nw * (64 * U)) {
    float4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = base + 64 * u + lane;
      const f32x4 t = i < nvec ? __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(x + i))
                               : f32x4{0.f, 0.f, 0.f, 0.f};
      v[u] = make_float4(t[0], t[1], t[2], t[3]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = base + 64 * u + lane;
      if (i >= nvec) continue;
      const float a = act_code(v[u].x, inv1, z1), b = act_code(v[u].y, inv1, z1);
      const float c = act_code(v[u].z, inv1, z1), d = act_code(v[u].w, inv1, z1);
      xq1[i] = pack4((int)a, (int)b, (int)c, (int)d);
      if constexpr (TWO) {
        const float ra = v[u].x - (a - z1) * s1, rb = v[u].y - (b - z1) * s1;
        const float rc = v[u].z - (c - z1) * s1, rd = v[u].w - (d - z1) * s1;
        xq2[i] = pack4((int)act_code(ra, inv2, z2), (int)act_code(rb, inv2, z2),
                       (int)act_code(rc, inv2, z2), (int)act_code(rd, inv2, z2));
      }
    }
  }
}

// ------------------------------------------------------------ per-row qparams
// The min and the max over the TPR threads that own a row, both at once (both
// are exact in any order): within a wave by DPP moves over lane bits 0-3 and
// lane-half swaps over bits 4 and 5, across the row's waves through LDS with a
// single barrier.
template <int CTRL>
__device__ __forceinline__ float qp_dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
template <int TPR>
__device__ __forceinline__ void row_minmax(float &mn, float &mx, float2 *lds) {
  mn = fminf(mn, qp_dpp<0xB1>(mn));  // quad_perm 1,0,3,2
  mx = fmaxf(mx, qp_dpp<0xB1>(mx));
  mn = fminf(mn, qp_dpp<0x4E>(mn));  // quad_perm 2,3,0,1
  mx = fmaxf(mx, qp_dpp<0x4E>(mx));
  mn = fminf(mn, qp_dpp<0x124>(mn));  // row_ror:4
  mx = fmaxf(mx, qp_dpp<0x124>(mx));
  mn = fminf(mn, qp_dpp<0x128>(mn));  // row_ror:8
  mx = fmaxf(mx, qp_dpp<0x128>(mx));
  // each lane gets its own value and its partner's (lane ^ 16, then ^ 32)
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(mn), __float_as_uint(mn), false, false);
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
  mn = fminf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  mx = fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
  a = __builtin_amdgcn_permlane32_swap(__float_as_uint(mn), __float_as_uint(mn), false, false);
  b = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
  mn = fminf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  mx = fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
  if constexpr (TPR > 64) {
    const int w = (threadIdx.x % TPR) >> 6, base = (threadIdx.x / TPR) * (TPR / 64);
    if ((threadIdx.x & 63) == 0) lds[base + w] = make_float2(mn, mx);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < TPR / 64; ++i) {
      const float2 p = lds[base + i];
      mn = fminf(mn, p.x);
      mx = fmaxf(mx, p.y);
    }
  }
}

// ExecuTorch 8da4w choose_qparams_affine, read as the affine min/max rule:
// mn = min(min x, 0), mx = max(max x, 0), s = max((mx - mn) / 255, eps),
// zp = clamp(-128 - rint(mn / s)), then xq = clamp(rint(x * (1/s)) + zp).
template <int TPR, int VPT, int MODE>
__global__ __launch_bounds__(256) void k_choose_qparams_rows(
    const float *__restrict__ x, int64_t M, int64_t K, float *__restrict__ scale,
    int32_t *__restrict__ zp, void *__restrict__ xq) {
  __shared__ float2 red_mm[4];
  constexpr int RPW = 256 / TPR;
  const int t = threadIdx.x % TPR;
  const int64_t m = (int64_t)blockIdx.x * RPW + threadIdx.x / TPR;
  const bool active = m < M;
  const int64_t nvec = K >> 2;
  const int64_t base = (active ? m : 0) * K;
  const float4 *row = reinterpret_cast<const float4 *>(x + base);

  float mn = 0.0f, mx = 0.0f;
  float4 v[VPT > 0 ? VPT : 1];
  if constexpr (VPT > 0) {
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int64_t j = t + (int64_t)i * TPR;
      v[i] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (active && j < nvec) v[i] = row[j];
      mn = fminf(mn, fminf(fminf(v[i].x, v[i].y), fminf(v[i].z, v[i].w)));
      mx = fmaxf(mx, fmaxf(fmaxf(v[i].x, v[i].y), fmaxf(v[i].z, v[i].w)));
    }
  } else {
    for (int64_t j = t; j < nvec; j += TPR) {
      if (!active) break;
      const float4 u = row[j];
      mn = fminf(mn, fminf(fminf(u.x, u.y), fminf(u.z, u.w)));
      mx = fmaxf(mx, fmaxf(fmaxf(u.x, u.y), fmaxf(u.z, u.w)));
    }
  }
  row_minmax<TPR>(mn, mx, red_mm);
  const float s = fmaxf((mx - mn) / 255.0f, FLT_EPSILON);
  const float zf = clamp_code(-128.0f - rintf(mn / s), -128.0f, 127.0f);
  if (active && t == 0) {
    scale[m] = s;
    zp[m] = (int32_t)zf;
  }
  if (xq == nullptr || !active) return;
  const float inv = 1.0f / s;
  int8_t *out = static_cast<int8_t *>(xq) + base;
  auto emit = [&](int64_t j, float4 u) {
    const int a = (int)act_code(u.x, inv, zf), b = (int)act_code(u.y, inv, zf);
    const int c = (int)act_code(u.z, inv, zf), d = (int)act_code(u.w, inv, zf);
    if constexpr (MODE == QP_CODES) {
      reinterpret_cast<uint32_t *>(out)[j] = pack4(a, b, c, d);
    } else if constexpr (MODE == QP_DIFF_BF16) {
      // xq - zp is an integer of at most 9 bits: its float's top half is the
      // exact bf16. Each 8-k block is stored as k = 0,4,1,5,2,6,3,7 (the order
      // the tiled 4-bit kernel unpacks nibbles in): the lanes holding k0..k3
      // (even j) and k4..k7 (odd j, the next lane) swap two values each, then
      // the even lane writes k0,k4,k1,k5 and the odd lane k2,k6,k3,k7. Both
      // lanes of a pair are always active: rows hold a multiple of 8 codes.
      const int z = (int)zf;
      const uint32_t ba = __float_as_uint((float)(a - z)) >> 16, bb = __float_as_uint((float)(b - z)) >> 16;
      const uint32_t bc = __float_as_uint((float)(c - z)) >> 16, bd = __float_as_uint((float)(d - z)) >> 16;
      const bool odd = (j & 1) != 0;
      const uint32_t got = (uint32_t)__shfl_xor((int)(odd ? (ba | (bb << 16)) : (bc | (bd << 16))), 1);
      const uint32_t w0 = odd ? ((got & 0xffffu) | (bc << 16)) : (ba | (got << 16));
      const uint32_t w1 = odd ? ((got >> 16) | (bd << 16)) : (bb | (got & 0xffff0000u));
      reinterpret_cast<uint2 *>(static_cast<uint16_t *>(xq) + base)[j] = make_uint2(w0, w1);
    } else {
      // 8-k block stored as k = 0,2,4,6,1,3,5,7: the even half of the vector
      // (k0..k3) fills bytes (0,1) and (4,5); the odd half (k4..k7) bytes (2,3), (6,7).
      const int64_t blk = (j >> 1) * 8;
      const int off = (j & 1) ? 2 : 0;
      uint16_t *o16 = reinterpret_cast<uint16_t *>(out + blk + off);
      o16[0] = (uint16_t)((a & 0xff) | ((c & 0xff) << 8));
      o16[2] = (uint16_t)((b & 0xff) | ((d & 0xff) << 8));
    }
  };
  if constexpr (VPT > 0) {
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int64_t j = t + (int64_t)i * TPR;
      if (j < nvec) emit(j, v[i]);
    }
  } else {
    for (int64_t j = t; j < nvec; j += TPR) emit(j, row[j]);
  }
}

template <int PERM>
hipError_t cq_dispatch(const float *x, int64_t M, int64_t K, float *scale, int32_t *zp,
                       void *xq, hipStream_t st) {
  const int64_t nvec = K / 4;
  if (nvec <= 64 * 4) {
    const dim3 grid((unsigned)((M + 3) / 4));
    if (nvec <= 64)
      hipLaunchKernelGGL((k_choose_qparams_rows<64, 1, PERM>), grid, dim3(256), 0, st, x, M, K,
                         scale, zp, xq);
    else if (nvec <= 128)
      hipLaunchKernelGGL((k_choose_qparams_rows<64, 2, PERM>), grid, dim3(256), 0, st, x, M, K,
                         scale, zp, xq);
    else
      hipLaunchKernelGGL((k_choose_qparams_rows<64, 4, PERM>), grid, dim3(256), 0, st, x, M, K,
                         scale, zp, xq);
  } else {
    const dim3 grid((unsigned)M);
    if (nvec <= 256 * 2)
      hipLaunchKernelGGL((k_choose_qparams_rows<256, 2, PERM>), grid, dim3(256), 0, st, x, M, K,
                         scale, zp, xq);
    else if (nvec <= 256 * 4)
      hipLaunchKernelGGL((k_choose_qparams_rows<256, 4, PERM>), grid, dim3(256), 0, st, x, M, K,
                         scale, zp, xq);
    else if (nvec <= 256 * 8)
      hipLaunchKernelGGL((k_choose_qparams_rows<256, 8, PERM>), grid, dim3(256), 0, st, x, M, K,
                         scale, zp, xq);
    else if (nvec <= 256 * 16)
      hipLaunchKernelGGL((k_choose_qparams_rows<256, 16, PERM>), grid, dim3(256), 0, st, x, M,
                         K, scale, zp, xq);
    else
      hipLaunchKernelGGL((k_choose_qparams_rows<256, 0, PERM>), grid, dim3(256), 0, st, x, M, K,
                         scale, zp, xq);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_weight_int8(const void *w, bool bf16, int64_t N, int64_t K, int mode,
                                       int8_t *q, float *scale, int32_t *wsum, hipStream_t st) {
  const float den = mode == 0 ? 127.0f : 127.5f;
  const float lo = mode == 0 ? -127.0f : -128.0f;
  return bf16 ? quant_w8_dispatch<true>(w, N, K, den, lo, q, scale, wsum, st)
              : quant_w8_dispatch<false>(w, N, K, den, lo, q, scale, wsum, st);
}

hipError_t launch_quantize_weight_q4gsw(const float *w, int64_t N, int64_t K, uint8_t *q4,
                                        float *gs, int32_t *gsum, hipStream_t st) {
  const int64_t items = N * (K / 32);
  hipLaunchKernelGGL(k_quantize_weight_q4gsw, dim3((unsigned)((items + 255) / 256)), dim3(256), 0,
                     st, w, N, K, q4, gs, gsum);
  return hipGetLastError();
}

hipError_t launch_quantize_act_per_tensor(const float *x, int64_t count, float s1, int32_t z1,
                                          bool two_pass, float s2, int32_t z2, int8_t *xq1,
                                          int8_t *xq2, hipStream_t st) {
  const int64_t nvec = count / 4;
  const float inv1 = 1.0f / s1;
  const float inv2 = two_pass ? 1.0f / s2 : 0.0f;
  // one wave per 64 float4 (one 1 KB load a round), at most 64 waves per CU
  // (the rest grid-strides): at 512 x 4096 from HBM 3.9 us, against 4.5 us
  // with four loads a wave and a quarter of the waves
  int64_t blocks = (nvec + 255) / 256;
  if (blocks > 256 * 16) blocks = 256 * 16;
  if (blocks < 1) blocks = 1;
  if (two_pass)
    hipLaunchKernelGGL((k_quantize_act_per_tensor<1, true>), dim3((unsigned)blocks), dim3(256), 0,
                       st, reinterpret_cast<const float4 *>(x), nvec, s1, inv1, (float)z1, inv2,
                       (float)z2, reinterpret_cast<uint32_t *>(xq1),
                       reinterpret_cast<uint32_t *>(xq2));
  else
    hipLaunchKernelGGL((k_quantize_act_per_tensor<1, false>), dim3((unsigned)blocks), dim3(256),
                       0, st, reinterpret_cast<const float4 *>(x), nvec, s1, inv1, (float)z1,
                       inv2, (float)z2, reinterpret_cast<uint32_t *>(xq1), nullptr);
  return hipGetLastError();
}

hipError_t launch_choose_qparams_rows(const float *x, int64_t M, int64_t K, float *scale,
                                      int32_t *zp, void *out, QpOut mode, hipStream_t st) {
  switch (mode) {
    case QP_CODES: return cq_dispatch<QP_CODES>(x, M, K, scale, zp, out, st);
    case QP_CODES_PERM8: return cq_dispatch<QP_CODES_PERM8>(x, M, K, scale, zp, out, st);
    case QP_DIFF_BF16: return cq_dispatch<QP_DIFF_BF16>(x, M, K, scale, zp, out, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace aql
