// Weight-only W8A16 linear: y[m, n] = scale[n] * sum_k x[m, k] * q[n, k] (+ bias[n]).
//
// tiny-llm quant, Step 4.6: the per-channel scale factors out of the sum, and
// int8 -> bf16 is exact, so the sum can run on the bf16 matrix cores with the
// int8 codes widened in registers and the scale applied once per output.
//
// Tile: one workgroup owns 16 output channels and 16 rows of x; its W waves
// split K into 64-wide chunks (wave w takes chunks w, w + W, ...). Per chunk a
// lane reads 16 int8 weights of one channel (a wave covers 16 channels x 64
// contiguous bytes) and the matching 16 bf16 of x, widens the weights and
// issues two v_mfma_f32_16x16x32_bf16; the MFMA does the K reduction across
// the lanes. Loads are buffer loads: the hardware range check returns zero
// past the end of the tile's rows (no branches, 32-bit offsets), and chunks
// are fetched in batches of U with the next batch in flight while the current
// one is multiplied. The waves' partial 16x16 tiles meet once in LDS.
//
// Launches: a single problem (grid = N/16 x M/16 tiles), or a group of
// independent problems in one launch (a decode sweep's linears), whose tiles
// are laid end to end in one grid and found through a device table.
#include "common.h"

namespace aql {
namespace {

constexpr int OOB = 0x40000000;  // an offset past any tile's range: loads return 0

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                           0x00020000);
}

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

struct Tile {
  const uint16_t *x;
  const int8_t *q;
  const float *scale;
  const uint16_t *bias;
  uint16_t *y;
  int64_t M, N, K;
  int64_t n0, m0;
};

template <int W, int U>
__device__ __forceinline__ void w8a16_tile(const Tile &t, f32x4 (*red)[64]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int64_t K = t.K;
  const int64_t nrows = t.N - t.n0 < 16 ? t.N - t.n0 : 16;
  const int64_t mrows = t.M - t.m0 < 16 ? t.M - t.m0 : 16;
  const __amdgpu_buffer_rsrc_t rq = rsrc(t.q + t.n0 * K, (uint32_t)(nrows * K));
  const __amdgpu_buffer_rsrc_t rx = rsrc(t.x + t.m0 * K, (uint32_t)(mrows * K * 2));
  const uint32_t qlane = (uint32_t)(r * K + g * 16);
  const uint32_t xlane = 2u * qlane;
  const int nch = (int)((K + 63) >> 6);
  const int cnt = wave < nch ? (nch - wave + W - 1) / W : 0;

  i32x4 wv[U], xa[U], xb[U];
  auto fetch = [&](int i0, i32x4 *w_, i32x4 *a_, i32x4 *b_) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u;
      const int c = wave + W * i;
      const bool valid = i < cnt;
      const bool kin = valid && (64 * c + 16 * g) < K;
      const int qo = valid ? (int)(qlane + 64u * c) : OOB;
      const int xo = kin ? (int)(xlane + 128u * c) : OOB;
      w_[u] = __builtin_amdgcn_raw_buffer_load_b128(rq, qo, 0, 2);
      a_[u] = __builtin_amdgcn_raw_buffer_load_b128(rx, xo, 0, 0);
      b_[u] = __builtin_amdgcn_raw_buffer_load_b128(rx, xo + 16, 0, 0);
    }
  };

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  fetch(0, wv, xa, xb);
  for (int b = 0; b < cnt; b += U) {
    i32x4 wn[U], xan[U], xbn[U];
    fetch(b + U, wn, xan, xbn);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xa[u]),
                                                    widen8(wv[u].x, wv[u].y), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xb[u]),
                                                    widen8(wv[u].z, wv[u].w), acc, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      wv[u] = wn[u];
      xa[u] = xan[u];
      xb[u] = xbn[u];
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
  const int64_t n = t.n0 + r;
  if (n >= t.N) return;
  const float s = t.scale[n];
  const float bv = t.bias ? bf16_to_f32(t.bias[n]) : 0.0f;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int64_t mm = t.m0 + 4 * g + v;
    if (mm < t.M) t.y[mm * t.N + n] = f32_to_bf16_rne(s * acc[v] + bv);
  }
}

template <int W, int U>
__global__ __launch_bounds__(64 * W) void k_w8a16(const uint16_t *__restrict__ x, int64_t M,
                                                  int64_t K, const int8_t *__restrict__ q,
                                                  const float *__restrict__ scale,
                                                  const uint16_t *__restrict__ bias, int64_t N,
                                                  uint16_t *__restrict__ y) {
  __shared__ f32x4 red[W > 1 ? W - 1 : 1][64];
  const Tile t{x, q, scale, bias, y, M, N, K, (int64_t)blockIdx.x * 16, (int64_t)blockIdx.y * 16};
  w8a16_tile<W, U>(t, red);
}

// Grouped launch: blocks [begin, begin + nblk * mblk) of the grid belong to
// problem p, n-block fastest. The table is read through the scalar cache.
template <int W, int U>
__global__ __launch_bounds__(64 * W) void k_w8a16_grouped(const W8A16GroupEntry *__restrict__ tab,
                                                          int count) {
  __shared__ f32x4 red[W > 1 ? W - 1 : 1][64];
  const int blk = blockIdx.x;
  int lo = 0, hi = count - 1;
  while (lo < hi) {  // last entry with begin <= blk
    const int mid = (lo + hi + 1) >> 1;
    if (tab[mid].blk_begin <= blk) lo = mid;
    else hi = mid - 1;
  }
  const W8A16GroupEntry &e = tab[lo];
  const int local = blk - e.blk_begin;
  const int nb = local % e.nblk, mb = local / e.nblk;
  const Tile t{e.x, e.q, e.scale, e.bias, e.y, e.M, e.N, e.K, (int64_t)nb * 16, (int64_t)mb * 16};
  w8a16_tile<W, U>(t, red);
}

template <int W>
void launch_w(dim3 grid, hipStream_t st, const uint16_t *x, int64_t M, int64_t K, const int8_t *q,
              const float *scale, const uint16_t *bias, int64_t N, uint16_t *y) {
  hipLaunchKernelGGL((k_w8a16<W, 4>), grid, dim3(64 * W), 0, st, x, M, K, q, scale, bias, N, y);
}

template <int W>
void launch_g(int blocks, hipStream_t st, const W8A16GroupEntry *tab, int count) {
  hipLaunchKernelGGL((k_w8a16_grouped<W, 4>), dim3((unsigned)blocks), dim3(64 * W), 0, st, tab,
                     count);
}

}  // namespace

int w8a16_waves(int64_t K, int64_t blocks) {
  const int64_t nch = (K + 63) / 64;
  int W = 4;
  if (blocks < 256) W = 16;
  else if (blocks < 512) W = 8;
  while (W > 1 && W * 2 > nch) W >>= 1;
  return W;
}

hipError_t launch_w8a16(const uint16_t *x, int64_t M, int64_t K, const int8_t *q,
                        const float *scale, const uint16_t *bias, int64_t N, uint16_t *y,
                        hipStream_t st) {
  const int64_t nblk = (N + 15) / 16, mblk = (M + 15) / 16;
  const int W = w8a16_waves(K, nblk * mblk);
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

hipError_t launch_w8a16_grouped(const W8A16GroupEntry *dev_tab, int count, int total_blocks,
                                int waves, hipStream_t st) {
  switch (waves) {
    case 8: launch_g<8>(total_blocks, st, dev_tab, count); break;
    case 4: launch_g<4>(total_blocks, st, dev_tab, count); break;
    case 2: launch_g<2>(total_blocks, st, dev_tab, count); break;
    default: launch_g<1>(total_blocks, st, dev_tab, count); break;
  }
  return hipGetLastError();
}

}  // namespace aql
