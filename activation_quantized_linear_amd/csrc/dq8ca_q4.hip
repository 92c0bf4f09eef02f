// 8da4w linear: dynamic per-row int8 activations x 4-bit group-32 weights.
//
// ExecuTorch 8da4w PR: out[m, n] = s[m] * sum_k (xq[m, k] - z[m]) * dequant(w)[n, k]
// with dequant(w) = q4[n, k] * gs[n, k / 32]. Per group g the integer part
//     A_g[m, n] = sum_{k in g} xq q4 - z[m] gsum[n, g]
// is exact; y = s[m] * sum_g gs[n, g] * A_g + bias[n] in fp32.
//
// Unpacking: a packed word holds 8 nibbles (k = 0..7, k even in the low
// nibble of each byte). (word << 4) & 0xF0F0F0F0 puts the even-k nibbles in the
// high half of each byte and word & 0xF0F0F0F0 the odd-k ones: each byte is
// then the int8 value 16 * c, exact for c in [-8, 7]. Two masks make eight
// MFMA operands, and the int8 MFMA accumulates 16 * sum xq c exactly (a
// power-of-two factor removed once at the end). The operand order is
// k = 0,2,4,6,1,3,5,7 in every 8-k block, so the activation codes are written
// in that order by the qparams kernel (they are internal to this op).
//
// One v_mfma_i32_16x16x32_i8 covers exactly one 32-k group, and its int32
// result is folded into the fp32 accumulator with the group scale right away.
#include "common.h"

namespace aql {
namespace {

__device__ __forceinline__ long unpack_q4x8(uint32_t w) {
  const uint32_t even = (w << 4) & 0xF0F0F0F0u;
  const uint32_t odd = w & 0xF0F0F0F0u;
  return (long)((uint64_t)even | ((uint64_t)odd << 32));
}

// --------------------------------------------------------- skinny (M <= 16)
// A workgroup owns 16 output channels; its W waves split K into 128-k chunks
// (4 groups). A lane loads the 16 packed bytes of one group of one channel
// (a wave reads 16 channels x 64 contiguous bytes); a wave-private LDS
// transpose hands each lane the 8-k slice of each of the 4 groups that the
// MFMA layout asks for.
template <int W>
__global__ __launch_bounds__(64 * W) void k_dq8ca_q4_skinny(Q4Args p) {
  __shared__ __attribute__((aligned(16))) uint32_t xt[W][16 * 20];
  __shared__ f32x4 red[W > 1 ? W - 1 : 1][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int64_t M = p.M, N = p.N, K = p.K, G = K / 32;
  const int64_t n0 = (int64_t)blockIdx.x * 16, m0 = (int64_t)blockIdx.y * 16;
  const int64_t n = n0 + r, m = m0 + r;
  const bool nv = n < N, mv = m < M;
  const uint8_t *qp = p.q4 + (nv ? n : 0) * (K / 2) + g * 16;
  const int8_t *xp = p.xq + (mv ? m : 0) * K + g * 8;
  const float *gsp = p.gs + (nv ? n : 0) * G;
  const int32_t *gmp = p.gsum + (nv ? n : 0) * G;
  int zp16[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int64_t mm = m0 + 4 * g + v;
    zp16[v] = mm < M ? -16 * p.xz[mm] : 0;
  }
  uint32_t *tp = xt[wave];

  f32x4 f = {0.f, 0.f, 0.f, 0.f};
  const int64_t nch = (G + 3) / 4;
  for (int64_t c = wave; c < nch; c += W) {
    const int64_t gb = 4 * c;
    const bool ok = nv && (gb + g) < G;
    i32x4 wq = {0, 0, 0, 0};
    if (ok) wq = __builtin_nontemporal_load(reinterpret_cast<const i32x4 *>(qp + 64 * c));
    tp[r * 20 + 0 * 4 + g] = (uint32_t)wq.x;
    tp[r * 20 + 1 * 4 + g] = (uint32_t)wq.y;
    tp[r * 20 + 2 * 4 + g] = (uint32_t)wq.z;
    tp[r * 20 + 3 * 4 + g] = (uint32_t)wq.w;
    __builtin_amdgcn_wave_barrier();
    const i32x4 mine = *reinterpret_cast<const i32x4 *>(&tp[r * 20 + g * 4]);
    __builtin_amdgcn_wave_barrier();
    const uint32_t words[4] = {(uint32_t)mine.x, (uint32_t)mine.y, (uint32_t)mine.z,
                               (uint32_t)mine.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t grp = gb + j;
      if (grp >= G) break;
      const long b = unpack_q4x8(words[j]);
      const long a = mv ? *reinterpret_cast<const long *>(xp + 32 * grp) : 0L;
      const i32x4 t = __builtin_amdgcn_mfma_i32_16x16x32_i8(a, b, i32x4{0, 0, 0, 0}, 0, 0, 0);
      const float gsv = nv ? gsp[grp] : 0.0f;
      const int gmv = nv ? gmp[grp] : 0;
#pragma unroll
      for (int v = 0; v < 4; ++v) f[v] += gsv * (float)(t[v] + zp16[v] * gmv);
    }
  }

  if constexpr (W > 1) {
    if (wave > 0) red[wave - 1][lane] = f;
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int i = 0; i < W - 1; ++i) f += red[i][lane];
  }
  if (!nv) return;
  const float b = p.bias ? p.bias[n] : 0.0f;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int64_t mm = m0 + 4 * g + v;
    if (mm < M) p.y[mm * N + n] = p.xs[mm] * (f[v] * 0.0625f) + b;
  }
}

// ----------------------------------------------------------------- tiled
// 128 x 128 output tile per 256-thread workgroup, K step 64 (two groups),
// 2x2 waves of 64x64, operands staged through double-buffered LDS; the B tile
// is unpacked from nibbles to 16 * c bytes on its way into LDS, and the two
// groups' scales and sums ride along.
constexpr int BM = 128, BN = 128, LDSW = 80;

__global__ __launch_bounds__(256) void k_dq8ca_q4_tiled(Q4Args p, int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(16))) int8_t sa[2][BM * LDSW];
  __shared__ __attribute__((aligned(16))) int8_t sb[2][BN * LDSW];
  __shared__ float sgs[2][BN][2];
  __shared__ int sgm[2][BN][2];

  const int nt = tiles_m * tiles_n;
  const int lin = blockIdx.x;
  int tile = lin;
  if ((nt & 7) == 0) tile = (lin & 7) * (nt >> 3) + (lin >> 3);
  const int tn = tile / tiles_m, tm = tile % tiles_m;
  const int64_t n0 = (int64_t)tn * BN, m0 = (int64_t)tm * BM;
  const int64_t M = p.M, N = p.N, K = p.K, G = K / 32;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int r = lane & 15, g = lane >> 4;

  const int kc = tid & 3;
  const int8_t *ga[2];
  bool va[2];
  int lofs[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int rho = (tid + 256 * j) >> 2;
    lofs[j] = rho * LDSW + kc * 16;
    const int64_t m = m0 + rho;
    va[j] = m < M;
    ga[j] = p.xq + (va[j] ? m : 0) * K + kc * 16;
  }
  const int brow = tid >> 1, half = tid & 1;
  const int64_t bn = n0 + brow;
  const bool vbn = bn < N;
  const uint8_t *gq = p.q4 + (vbn ? bn : 0) * (K / 2) + half * 16;
  const float *ggs = p.gs + (vbn ? bn : 0) * G + half;
  const int32_t *ggm = p.gsum + (vbn ? bn : 0) * G + half;

  int zp16[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t mm = m0 + wm * 64 + i * 16 + 4 * g + v;
      zp16[i][v] = mm < M ? -16 * p.xz[mm] : 0;
    }

  f32x4 f[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) f[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = (int)((K + 63) / 64);
  i32x4 ra[2];
  i32x4 rq;
  float rgs;
  int rgm;
  auto gload = [&](int kt) {
    const int64_t k = (int64_t)kt * 64;
    const bool kok = k + kc * 16 < K;
#pragma unroll
    for (int j = 0; j < 2; ++j)
      ra[j] = (kok && va[j]) ? *reinterpret_cast<const i32x4 *>(ga[j] + k) : i32x4{0, 0, 0, 0};
    const bool gok = vbn && (2 * (int64_t)kt + half) < G;
    rq = gok ? __builtin_nontemporal_load(reinterpret_cast<const i32x4 *>(gq + k / 2))
             : i32x4{0, 0, 0, 0};
    rgs = gok ? ggs[2 * kt] : 0.0f;
    rgm = gok ? ggm[2 * kt] : 0;
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int j = 0; j < 2; ++j) *reinterpret_cast<i32x4 *>(&sa[buf][lofs[j]]) = ra[j];
    const long u0 = unpack_q4x8((uint32_t)rq.x), u1 = unpack_q4x8((uint32_t)rq.y);
    const long u2 = unpack_q4x8((uint32_t)rq.z), u3 = unpack_q4x8((uint32_t)rq.w);
    int8_t *dst = &sb[buf][brow * LDSW + half * 32];
    *reinterpret_cast<i32x4 *>(dst) =
        i32x4{(int)u0, (int)((uint64_t)u0 >> 32), (int)u1, (int)((uint64_t)u1 >> 32)};
    *reinterpret_cast<i32x4 *>(dst + 16) =
        i32x4{(int)u2, (int)((uint64_t)u2 >> 32), (int)u3, (int)((uint64_t)u3 >> 32)};
    sgs[buf][brow][half] = rgs;
    sgm[buf][brow][half] = rgm;
  };

  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
#pragma unroll
    for (int gg = 0; gg < 2; ++gg) {
      long fa[4], fb[4];
      float gsv[4];
      int gmv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        fa[i] = *reinterpret_cast<const long *>(&sa[cur][(wm * 64 + i * 16 + r) * LDSW + gg * 32 + g * 8]);
        const int nb = wn * 64 + i * 16 + r;
        fb[i] = *reinterpret_cast<const long *>(&sb[cur][nb * LDSW + gg * 32 + g * 8]);
        gsv[i] = sgs[cur][nb][gg];
        gmv[i] = sgm[cur][nb][gg];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const i32x4 t = __builtin_amdgcn_mfma_i32_16x16x32_i8(fa[i], fb[j], i32x4{0, 0, 0, 0}, 0, 0, 0);
#pragma unroll
          for (int v = 0; v < 4; ++v) f[i][j][v] += gsv[j] * (float)(t[v] + zp16[i][v] * gmv[j]);
        }
    }
    if (kt + 1 < nk) sstore(cur ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t n = n0 + wn * 64 + j * 16 + r;
    if (n >= N) continue;
    const float b = p.bias ? p.bias[n] : 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t m = m0 + wm * 64 + i * 16 + 4 * g + v;
        if (m < M) p.y[m * N + n] = p.xs[m] * (f[i][j][v] * 0.0625f) + b;
      }
  }
}

template <int W>
void launch_skinny(dim3 grid, const Q4Args &a, hipStream_t st) {
  hipLaunchKernelGGL((k_dq8ca_q4_skinny<W>), grid, dim3(64 * W), 0, st, a);
}

}  // namespace

hipError_t launch_dq8ca_q4(const Q4Args &a, hipStream_t st) {
  if (a.M <= 16) {
    const int64_t nblk = (a.N + 15) / 16;
    const int64_t nch = (a.K / 32 + 3) / 4;
    int W = nblk < 512 ? 8 : 4;
    while (W > 1 && W * 2 > nch) W >>= 1;
    const dim3 grid((unsigned)nblk, 1);
    switch (W) {
      case 8: launch_skinny<8>(grid, a, st); break;
      case 4: launch_skinny<4>(grid, a, st); break;
      case 2: launch_skinny<2>(grid, a, st); break;
      default: launch_skinny<1>(grid, a, st); break;
    }
  } else {
    const int tiles_m = (int)((a.M + BM - 1) / BM);
    const int tiles_n = (int)((a.N + BN - 1) / BN);
    hipLaunchKernelGGL(k_dq8ca_q4_tiled, dim3((unsigned)(tiles_m * tiles_n)), dim3(256), 0, st, a,
                       tiles_m, tiles_n);
  }
  return hipGetLastError();
}

}  // namespace aql
