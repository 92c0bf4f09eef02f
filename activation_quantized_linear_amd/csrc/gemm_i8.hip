// int8 x int8 -> int32 tiled GEMM on the gfx950 matrix cores
// (v_mfma_i32_16x16x64_i8) with the W8A8 epilogues fused:
//
//   EPI_RAW   c[m, n] = sum_k a[m, k] b[n, k]                      (stage entry)
//   EPI_Q8TA  y = ws[n] (s1 (acc1 - z1 wsum[n]) + s2 (acc2 - z2 wsum[n])) + bias[n]
//             SmolVLM q8 recipe, Q8Linear / et_vk.linear_q8ta_q8csw; the two
//             passes share every weight tile: a workgroup's A tile holds 64 rows
//             of the first-pass codes and the same 64 rows of the residual codes.
//   EPI_DQ8   y = xs[m] ws[n] (acc - xz[m] wsum[n]) + bias[n]
//             ExecuTorch 8da4w linear_dq8ca with int8 per-channel weights.
// The zero points fold through the weight sums in exact int32 before any float
// op, so the integer part is bit-exact whatever the tiling.
//
// Tiling: 128 (A rows) x 128 (N) per 256-thread workgroup, K step 64 bytes, 4
// waves in a 2x2 arrangement each owning 64x64 = 4x4 MFMA tiles. A and B tiles
// are staged through registers into double-buffered LDS (row stride 80 B:
// the 16-byte fragment reads of 16 consecutive rows hit distinct banks).
// Workgroups are mapped to tiles so that each XCD (blocks are dealt to the 8
// XCDs round-robin) works on a contiguous band of N tiles, sharing them in its L2.
#include "common.h"

namespace aql {
namespace {

constexpr int BM = 128, BN = 128, BK = 64, LDSW = 80;

template <int EPI, bool TWO>
__global__ __launch_bounds__(256) void k_gemm_i8(GemmArgs p, int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(16))) int8_t sa[2][BM * LDSW];
  __shared__ __attribute__((aligned(16))) int8_t sb[2][BN * LDSW];

  const int nt = tiles_m * tiles_n;
  const int lin = blockIdx.x;
  int tile = lin;
  if ((nt & 7) == 0) tile = (lin & 7) * (nt >> 3) + (lin >> 3);
  const int tn = tile / tiles_m, tm = tile % tiles_m;
  const int64_t n0 = (int64_t)tn * BN;
  const int64_t m0 = (int64_t)tm * (TWO ? BM / 2 : BM);
  const int64_t M = p.M, N = p.N, K = p.K;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int r = lane & 15, g = lane >> 4;

  // Global -> LDS assignment: 512 16-byte chunks per operand tile, 2 per thread.
  const int kc = tid & 3;
  const int8_t *ga[2], *gb[2];
  bool va[2], vb[2];
  int lofs[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int rho = (tid + 256 * j) >> 2;
    lofs[j] = rho * LDSW + kc * 16;
    int64_t m;
    const int8_t *src = p.a1;
    if constexpr (TWO) {
      const int h = rho >> 6, pr = rho & 63;
      if (pr >= 32) src = p.a2;
      m = m0 + 32 * h + (pr & 31);
    } else {
      m = m0 + rho;
    }
    va[j] = m < M;
    ga[j] = src + (va[j] ? m : 0) * K + kc * 16;
    const int64_t nr = n0 + rho;
    vb[j] = nr < N;
    gb[j] = p.b + (vb[j] ? nr : 0) * K + kc * 16;
  }

  i32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = i32x4{0, 0, 0, 0};

  const int nk = (int)((K + BK - 1) / BK);
  i32x4 ra[2], rb[2];
  auto gload = [&](int kt) {
    const int64_t k = (int64_t)kt * BK;
    const bool kok = k + kc * 16 < K;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const i32x4 z = {0, 0, 0, 0};
      ra[j] = (kok && va[j]) ? *reinterpret_cast<const i32x4 *>(ga[j] + k) : z;
      rb[j] = (kok && vb[j]) ? *reinterpret_cast<const i32x4 *>(gb[j] + k) : z;
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      *reinterpret_cast<i32x4 *>(&sa[buf][lofs[j]]) = ra[j];
      *reinterpret_cast<i32x4 *>(&sb[buf][lofs[j]]) = rb[j];
    }
  };

  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    i32x4 fa[4], fb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      fa[i] = *reinterpret_cast<const i32x4 *>(&sa[cur][(wm * 64 + i * 16 + r) * LDSW + g * 16]);
      fb[i] = *reinterpret_cast<const i32x4 *>(&sb[cur][(wn * 64 + i * 16 + r) * LDSW + g * 16]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa[i], fb[j], acc[i][j], 0, 0, 0);
    if (kt + 1 < nk) sstore(cur ^ 1);
    __syncthreads();
  }

  // Epilogue. acc[i][j] lane holds D[4g + v][r] of MFMA tile (i, j).
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t n = n0 + wn * 64 + j * 16 + r;
    if (n >= N) continue;
    if constexpr (EPI == EPI_RAW) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int64_t m = m0 + wm * 64 + i * 16 + 4 * g + v;
          if (m < M) p.c[m * N + n] = acc[i][j][v];
        }
    } else if constexpr (EPI == EPI_Q8TA) {
      const int ws = p.wsum[n];
      const float wsc = p.wscale[n];
      const float b = p.bias ? p.bias[n] : 0.0f;
      // sum_k (xq - z) q = acc - z * wsum fits int32 (|.| <= K * 255 * 128); the
      // intermediate terms are formed in wrapping unsigned arithmetic.
      const uint32_t zw1 = (uint32_t)p.z1 * (uint32_t)ws, zw2 = (uint32_t)p.z2 * (uint32_t)ws;
      if constexpr (TWO) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int64_t m = m0 + wm * 32 + i * 16 + 4 * g + v;
            if (m >= M) continue;
            const float f = p.s1 * (float)(int)((uint32_t)acc[i][j][v] - zw1) +
                            p.s2 * (float)(int)((uint32_t)acc[i + 2][j][v] - zw2);
            p.y[m * N + n] = wsc * f + b;
          }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int64_t m = m0 + wm * 64 + i * 16 + 4 * g + v;
            if (m >= M) continue;
            p.y[m * N + n] = wsc * (p.s1 * (float)(int)((uint32_t)acc[i][j][v] - zw1)) + b;
          }
      }
    } else {  // EPI_DQ8
      const int ws = p.wsum[n];
      const float wsc = p.wscale[n];
      const float b = p.bias ? p.bias[n] : 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int64_t m = m0 + wm * 64 + i * 16 + 4 * g + v;
          if (m >= M) continue;
          const int A = (int)((uint32_t)acc[i][j][v] - (uint32_t)p.xz[m] * (uint32_t)ws);
          p.y[m * N + n] = p.xs[m] * (wsc * (float)A) + b;
        }
    }
  }
}

}  // namespace

hipError_t launch_gemm_i8(const GemmArgs &a, GemmEpi epi, bool two_pass, hipStream_t st) {
  const int rows = two_pass ? BM / 2 : BM;
  const int tiles_m = (int)((a.M + rows - 1) / rows);
  const int tiles_n = (int)((a.N + BN - 1) / BN);
  const dim3 grid((unsigned)(tiles_m * tiles_n));
  switch (epi) {
    case EPI_RAW:
      hipLaunchKernelGGL((k_gemm_i8<EPI_RAW, false>), grid, dim3(256), 0, st, a, tiles_m, tiles_n);
      break;
    case EPI_Q8TA:
      if (two_pass)
        hipLaunchKernelGGL((k_gemm_i8<EPI_Q8TA, true>), grid, dim3(256), 0, st, a, tiles_m,
                           tiles_n);
      else
        hipLaunchKernelGGL((k_gemm_i8<EPI_Q8TA, false>), grid, dim3(256), 0, st, a, tiles_m,
                           tiles_n);
      break;
    case EPI_DQ8:
      hipLaunchKernelGGL((k_gemm_i8<EPI_DQ8, false>), grid, dim3(256), 0, st, a, tiles_m, tiles_n);
      break;
  }
  return hipGetLastError();
}

}  // namespace aql
