// Weight-only W8A16 linear: y[m, n] = scale[n] * sum_k x[m, k] * q[n, k] (+ bias[n]).
//
// tiny-llm quant, Step 4.6: the per-channel scale factors out of the sum, and
// int8 -> bf16 is exact, so the sum can run on the bf16 matrix cores with the
// int8 codes widened in registers and the scale applied once per output.
//
// Kernel shape (decode and skinny M): one workgroup owns 16 output channels
// and 16 rows of x; its W waves split K into 64-wide chunks. Per chunk a lane
// reads 16 int8 weights of one channel (16 B; a wave covers 16 channels x 64 B),
// the matching 16 bf16 of x, and issues two v_mfma_f32_16x16x32_bf16. The MFMA
// performs the K reduction across the wave's lanes, so no shuffles are needed;
// the waves' partial 16x16 tiles meet once in LDS at the end. Weights are
// read exactly once per 16 rows of x; larger M re-runs the weight stream per
// 16-row slice (grid.y).
#include "common.h"

namespace aql {
namespace {

// Two sign-extended int8 -> one dword of two bf16. The integer converts to
// float exactly and its low 16 mantissa bits are zero, so the top half of the
// float is the exact bf16.
__device__ __forceinline__ uint32_t bf16x2_from_i8(int lo, int hi) {
  return __builtin_amdgcn_perm(__float_as_uint((float)hi), __float_as_uint((float)lo),
                               0x07060302u);
}

// 8 int8 codes (two dwords, little-endian) -> 8 bf16 in order.
__device__ __forceinline__ bf16x8 widen8(int w0, int w1) {
  i32x4 r;
  r.x = (int)bf16x2_from_i8((int)(int8_t)(w0), (int)(int8_t)(w0 >> 8));
  r.y = (int)bf16x2_from_i8((int)(int8_t)(w0 >> 16), (w0 >> 24));
  r.z = (int)bf16x2_from_i8((int)(int8_t)(w1), (int)(int8_t)(w1 >> 8));
  r.w = (int)bf16x2_from_i8((int)(int8_t)(w1 >> 16), (w1 >> 24));
  return __builtin_bit_cast(bf16x8, r);
}

template <int W, int U>
__global__ __launch_bounds__(64 * W) void k_w8a16_skinny(
    const uint16_t *__restrict__ x, int64_t M, int64_t K, const int8_t *__restrict__ q,
    const float *__restrict__ scale, const uint16_t *__restrict__ bias, int64_t N,
    uint16_t *__restrict__ y) {
  __shared__ f32x4 red[W > 1 ? W - 1 : 1][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * 16, m0 = (int64_t)blockIdx.y * 16;
  const int64_t n = n0 + r, m = m0 + r;
  const bool nv = n < N, mv = m < M;
  const int8_t *qp = q + (nv ? n : 0) * K + g * 16;
  const uint16_t *xp = x + (mv ? m : 0) * K + g * 16;
  const int64_t nch = (K + 63) >> 6;

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int64_t c = wave; c < nch; c += (int64_t)U * W) {
    i32x4 wv[U], xa[U], xb[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t k = (c + (int64_t)u * W) * 64;
      const bool ok = (c + (int64_t)u * W) < nch && (k + g * 16) < K;
      const i32x4 z = {0, 0, 0, 0};
      wv[u] = (ok && nv) ? __builtin_nontemporal_load(reinterpret_cast<const i32x4 *>(qp + k)) : z;
      xa[u] = (ok && mv) ? *reinterpret_cast<const i32x4 *>(xp + k) : z;
      xb[u] = (ok && mv) ? *reinterpret_cast<const i32x4 *>(xp + k + 8) : z;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xa[u]),
                                                    widen8(wv[u].x, wv[u].y), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xb[u]),
                                                    widen8(wv[u].z, wv[u].w), acc, 0, 0, 0);
    }
  }

  if constexpr (W > 1) {
    if (wave > 0) red[wave - 1][lane] = acc;
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int i = 0; i < W - 1; ++i) acc += red[i][lane];
  }
  // lane holds D[4g + v][r]: row m0 + 4g + v of x, output channel n0 + r.
  if (!nv) return;
  const float s = scale[n];
  const float b = bias ? bf16_to_f32(bias[n]) : 0.0f;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int64_t mm = m0 + 4 * g + v;
    if (mm < M) y[mm * N + n] = f32_to_bf16_rne(s * acc[v] + b);
  }
}

template <int W>
void launch_w(dim3 grid, hipStream_t st, const uint16_t *x, int64_t M, int64_t K, const int8_t *q,
              const float *scale, const uint16_t *bias, int64_t N, uint16_t *y) {
  hipLaunchKernelGGL((k_w8a16_skinny<W, 4>), grid, dim3(64 * W), 0, st, x, M, K, q, scale, bias,
                     N, y);
}

}  // namespace

hipError_t launch_w8a16(const uint16_t *x, int64_t M, int64_t K, const int8_t *q,
                        const float *scale, const uint16_t *bias, int64_t N, uint16_t *y,
                        hipStream_t st) {
  const int64_t nblk = (N + 15) / 16, mblk = (M + 15) / 16;
  const int64_t nch = (K + 63) / 64;
  // Enough waves to keep ~2048 16-byte loads per XCD in flight, but never more
  // waves than 64-wide K chunks.
  const int64_t blocks = nblk * mblk;
  int W = 4;
  if (blocks < 256) W = 16;
  else if (blocks < 512) W = 8;
  else if (blocks > 2048) W = 2;
  while (W > 1 && W * 2 > nch) W >>= 1;
  const dim3 grid((unsigned)nblk, (unsigned)mblk);
  switch (W) {
    case 16: launch_w<16>(grid, st, x, M, K, q, scale, bias, N, y); break;
    case 8: launch_w<8>(grid, st, x, M, K, q, scale, bias, N, y); break;
    case 4: launch_w<4>(grid, st, x, M, K, q, scale, bias, N, y); break;
    case 2: launch_w<2>(grid, st, x, M, K, q, scale, bias, N, y); break;
    default: launch_w<1>(grid, st, x, M, K, q, scale, bias, N, y); break;
  }
  return hipGetLastError();
}

}  // namespace aql
