// Weight-only W8A16 linear for prefill-sized M (tiny-llm quant, Step 4.6):
// y[m, n] = scale[n] * sum_k x[m, k] * q[n, k] (+ bias[n]), bf16 in and out.
//
// The scale factors out of the sum and int8 -> bf16 is exact, so the sum runs
// on the bf16 matrix cores (v_mfma_f32_16x16x32_bf16, fp32 accumulation) with
// the weights widened in registers, and the scale is applied once per output.
//
// Tiles: on large grids 128 rows of x x 256 output channels per workgroup of 8
// waves side by side along N (k_w8a16_gemm_wide, below); otherwise BM (64 or
// 128) rows x 128 channels, waves (BM / 64) x 2 quadrants of 64 x 64 (4 x 4
// MFMA tiles each) times 2 halves of every 64-k stage, the halves' fp32
// accumulators added once at the end.
// Operands go global -> LDS by buffer loads that write LDS directly (hardware
// zero-fill past M, N and K): x as bf16 rows of 128 B, the weights as int8 rows
// of 64 B (half the bytes of bf16; they are widened after the fragment read).
// A 4-stage ring (2 stages for the wide tile on the largest grids) keeps the
// next stages in flight behind exact vmcnt waits and a fence-free barrier (a
// straight-line loop, so the compiler's wait counts stay exact). x rows store their 16-byte chunks XOR-swizzled by (row / 2) mod 8 and
// weight rows by (row / 4) mod 4, which makes every fragment read conflict-free.
// The output tile is staged in LDS as bf16 and written as whole rows.
#include "common.h"
#include "w8a16_gemm.h"

namespace aql {
namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int BN = 128, BK = 64, STAGES = 4;
constexpr int OOB = 0x40000000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// Two sign-extended int8 -> one dword of two bf16 (exact; see w8a16.hip).
__device__ __forceinline__ uint32_t bf16x2_from_i8(int lo, int hi) {
  return __builtin_amdgcn_perm(__float_as_uint((float)hi), __float_as_uint((float)lo),
                               0x07060302u);
}

// Eight int8 codes (two dwords) -> eight bf16 in order.
__device__ __forceinline__ bf16x8 widen8(uint32_t w0, uint32_t w1) {
  const uint32_t a = bf16x2_from_i8((int)(int8_t)(w0), (int)(int8_t)(w0 >> 8));
  const uint32_t b = bf16x2_from_i8((int)(int8_t)(w0 >> 16), (int)w0 >> 24);
  const uint32_t c = bf16x2_from_i8((int)(int8_t)(w1), (int)(int8_t)(w1 >> 8));
  const uint32_t d = bf16x2_from_i8((int)(int8_t)(w1 >> 16), (int)w1 >> 24);
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  return __builtin_bit_cast(bf16x8, u32x4{a, b, c, d});
}

__device__ __forceinline__ int swz_x(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ int swz_w(int row) { return (row >> 2) & 3; }

template <int WM>
struct GemmLds {
  static constexpr int BM = 64 * WM;
  static constexpr int XS = BM * 128;           // x stage: BM rows x 64 bf16
  static constexpr int WS = BN * 64;            // weight stage: 128 rows x 64 int8
  static constexpr int STAGE = XS + WS;
  static constexpr int RING = STAGES * STAGE;
  static constexpr int XCH = 2 * WM * 16 * 64 * 16;  // fp32 half-sums of the kh = 1 waves
  static constexpr int TLD = BN + 8;            // bf16 per staged output row
  static constexpr int TILE = BM * TLD * 2;
  static constexpr int BYTES = RING > XCH + TILE ? RING : XCH + TILE;
};

template <int WM>
__global__ __launch_bounds__(256 * WM) void k_w8a16_gemm(const uint16_t *__restrict__ x,
                                                          const int8_t *__restrict__ q,
                                                          const float *__restrict__ scale,
                                                          const uint16_t *__restrict__ bias,
                                                          uint16_t *__restrict__ y, int64_t M,
                                                          int64_t N, int64_t K, int tiles_m,
                                                          int tiles_n) {
  using L = GemmLds<WM>;
  constexpr int BM = L::BM, NW = 4 * WM, NL = WM == 1 ? 4 : 3;  // loads per wave per stage
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int nt = tiles_m * tiles_n;
  const int lin = blockIdx.x;
  int tile = lin;
  if ((nt & 7) == 0) tile = (lin & 7) * (nt >> 3) + (lin >> 3);
  const int tn = tile / tiles_m, tm = tile % tiles_m;
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kh = wave / (2 * WM), wm = (wave >> 1) % WM, wn = wave & 1;
  const int r = lane & 15, g = lane >> 4;
  const int64_t mval = M - m0 < BM ? M - m0 : BM;
  const int64_t nval = N - n0 < BN ? N - n0 : BN;
  const __amdgpu_buffer_rsrc_t rx = rsrc(x + m0 * K, (uint32_t)(mval * K * 2));
  const __amdgpu_buffer_rsrc_t rq = rsrc(q + n0 * K, (uint32_t)(nval * K));

  // Loads per stage: BM/8 x-slots (8 rows x 128 B) and 8 weight slots (16 rows
  // x 64 B), NL per wave; load q of every wave is of one kind: q < 2 x-slot
  // q * NW + wave, else weight slot (q - 2) * NW + wave.
  uint32_t off[NL], ldso[NL], kstep[NL];
  int kin_lim[NL];
#pragma unroll
  for (int qq = 0; qq < NL; ++qq) {
    if (qq < 2) {
      const int slot = qq * NW + wave;
      const int row = 8 * slot + (lane >> 3), c = (lane & 7) ^ swz_x(row);
      off[qq] = (uint32_t)row * (uint32_t)(2 * K) + 16u * c;
      ldso[qq] = (uint32_t)(slot * 1024);
      kstep[qq] = 128;
      kin_lim[qq] = (int)((2 * K - 16 * c + 127) / 128);
    } else {
      const int slot = (qq - 2) * NW + wave;
      const int row = 16 * slot + (lane >> 2), c = (lane & 3) ^ swz_w(row);
      off[qq] = (uint32_t)row * (uint32_t)K + 16u * c;
      ldso[qq] = (uint32_t)(L::XS + slot * 1024);
      kstep[qq] = 64;
      kin_lim[qq] = (int)((K - 16 * c + 63) / 64);
    }
  }
  const uint32_t lds_base = (uint32_t)(uintptr_t)smem;
  auto issue = [&](int kt) {
#pragma unroll
    for (int qq = 0; qq < NL; ++qq) {
      const uint32_t dst = lds_base + (uint32_t)((kt % STAGES) * L::STAGE) + ldso[qq];
      const int o = kt < kin_lim[qq] ? (int)(off[qq] + kstep[qq] * (uint32_t)kt) : OOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          qq < 2 ? rx : rq, (lds_void *)(uintptr_t)__builtin_amdgcn_readfirstlane(dst), 16, o, 0,
          0, 0);
    }
  };

  // fragment offsets within a stage
  int fxo[4], fwo[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int R = wm * 64 + i * 16 + r;
    fxo[i] = R * 128 + 16 * ((4 * kh + g) ^ swz_x(R));
    const int S = wn * 64 + i * 16 + r;
    fwo[i] = L::XS + S * 64 + 16 * ((2 * kh + (g >> 1)) ^ swz_w(S)) + 8 * (g & 1);
  }

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int kt) {
    const char *st = smem + (kt % STAGES) * L::STAGE;
    bf16x8 fa[4], fb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      fa[i] = *reinterpret_cast<const bf16x8 *>(st + fxo[i]);
      const i32x2 w = *reinterpret_cast<const i32x2 *>(st + fwo[i]);
      fb[i] = widen8((uint32_t)w[0], (uint32_t)w[1]);
    }
    __builtin_amdgcn_s_setprio(1);  // as in the wide tile below
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    __builtin_amdgcn_s_setprio(0);
  };

  const int nk = (int)((K + BK - 1) / BK);
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s) issue(s);
  int kt = 0;
  auto step = [&](int k) {
    __builtin_amdgcn_s_waitcnt(0x0F70 | (NL * (STAGES - 2)));
    __builtin_amdgcn_s_barrier();  // stage k complete everywhere; slot of k-1 free
    issue(k + STAGES - 1);
    compute(k);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // this stage's fragment reads done
  };
  // whole turns of the ring first: each stage's LDS offsets become constants
  const int nmain = nk - (STAGES - 1);
  for (; kt + STAGES - 1 < nmain; kt += STAGES) {
#pragma unroll
    for (int u = 0; u < STAGES; ++u) step(kt + u);
  }
  for (; kt < nmain; ++kt) step(kt);
#pragma unroll
  for (int t = 0; t < STAGES - 1; ++t) {
    if (kt < nk) {
      if (t == 0) __builtin_amdgcn_s_waitcnt(0x0F70 | (NL * (STAGES - 2)));
      else if (t == 1) __builtin_amdgcn_s_waitcnt(0x0F70 | (NL * (STAGES - 3)));
      else __builtin_amdgcn_s_waitcnt(0x0F70);
      __builtin_amdgcn_s_barrier();
      compute(kt);
      __builtin_amdgcn_s_waitcnt(0xC07F);
    }
    ++kt;
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();

  // ---- add the K halves, then scale + bias + bf16 into the LDS output tile.
  // acc[i][j] lane holds D[4g + v][r] of MFMA tile (i, j): row m, column n.
  f32x4 *xch = reinterpret_cast<f32x4 *>(smem);
  if (kh == 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) xch[((wave - 2 * WM) * 16 + i * 4 + j) * 64 + lane] = acc[i][j];
  }
  __syncthreads();
  uint16_t *tl = reinterpret_cast<uint16_t *>(smem + L::XCH);
  if (kh == 0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = wn * 64 + j * 16 + r;
      const int64_t n = n0 + col;
      const float s = n < N ? scale[n] : 0.0f;
      const float b = (n < N && bias) ? bf16_to_f32(bias[n]) : 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x4 v4 = acc[i][j] + xch[(wave * 16 + i * 4 + j) * 64 + lane];
#pragma unroll
        for (int v = 0; v < 4; ++v)
          tl[(wm * 64 + i * 16 + 4 * g + v) * L::TLD + col] = f32_to_bf16_rne(s * v4[v] + b);
      }
    }
  }
  __syncthreads();
  // 16 lanes x 16 B per 256-byte row
  const bool vec = (N & 7) == 0;
  for (int u = tid; u < BM * 16; u += 256 * WM) {
    const int row = u >> 4, c = u & 15;
    const int64_t m = m0 + row, n = n0 + 8 * c;
    if (m >= M || n >= N) continue;
    const i32x4 val = *reinterpret_cast<const i32x4 *>(tl + row * L::TLD + 8 * c);
    uint16_t *dst = y + m * N + n;
    if (vec) {
      *reinterpret_cast<i32x4 *>(dst) = val;
    } else {
      const uint16_t *h = reinterpret_cast<const uint16_t *>(&val);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (n + e < N) dst[e] = h[e];
    }
  }
}

// Wide tile: 128 rows of x x 256 output channels, 8 waves side by side along
// N, each 128 x 32 (8 x 2 MFMA tiles) over the whole 64-k stage (32 MFMAs a
// stage, no K halves to add). The weights are the cheap operand (1 byte an
// element against x's 2), so doubling the channels per tile cuts the operand
// bytes per MFMA by a third: 32 KB a stage for 2 x 128 x 256 x 64 flops
// instead of 24 KB for half that. Each wave widens only its own 32 channels
// and uses every widened fragment for 8 MFMAs; with 2 x 4 waves of 64 x 64 the
// widening was done twice and took ~20% longer.
template <int SG>
struct WideLds {
  static constexpr int BM = 128, BNW = 256;
  static constexpr int XS = BM * 128;           // x stage: 128 rows x 64 bf16
  static constexpr int WS = BNW * 64;           // weight stage: 256 rows x 64 int8
  static constexpr int STAGE = XS + WS;         // 32 KB
  static constexpr int RING = SG * STAGE;       // SG stages of 32 KB
  static constexpr int TLD = BNW + 8;           // bf16 per staged output row
  static constexpr int TILE = BM * TLD * 2;
  static constexpr int BYTES = RING > TILE ? RING : TILE;
};

// SG = 4: a 4-stage ring, one workgroup a CU. SG = 2: a 2-stage ring in
// 64 KB, so two workgroups share a CU and each covers the other's waits at
// the stage barrier (from 512 tiles on, where every CU gets two).
template <int SG>
__global__ __launch_bounds__(512, SG == 2 ? 4 : 2) void k_w8a16_gemm_wide(const uint16_t *__restrict__ x,
                                                         const int8_t *__restrict__ q,
                                                         const float *__restrict__ scale,
                                                         const uint16_t *__restrict__ bias,
                                                         uint16_t *__restrict__ y, int64_t M,
                                                         int64_t N, int64_t K, int tiles_m,
                                                         int tiles_n) {
  using L = WideLds<SG>;
  constexpr int BM = L::BM, BNW = L::BNW, NL = 4;  // loads per wave per stage
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int nt = tiles_m * tiles_n;
  const int lin = blockIdx.x;
  int tile = lin;
  if ((nt & 7) == 0) tile = (lin & 7) * (nt >> 3) + (lin >> 3);
  const int tn = tile / tiles_m, tm = tile % tiles_m;
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BNW;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave;  // 32 channels a wave
  const int r = lane & 15, g = lane >> 4;
  const int64_t mval = M - m0 < BM ? M - m0 : BM;
  const int64_t nval = N - n0 < BNW ? N - n0 : BNW;
  const __amdgpu_buffer_rsrc_t rx = rsrc(x + m0 * K, (uint32_t)(mval * K * 2));
  const __amdgpu_buffer_rsrc_t rq = rsrc(q + n0 * K, (uint32_t)(nval * K));

  // Loads per stage: 16 x-slots (8 rows x 128 B) and 16 weight slots (16 rows
  // x 64 B); load qq of wave w is x-slot 8 qq + w (qq < 2), else weight slot
  // 8 (qq - 2) + w.
  uint32_t off[NL], ldso[NL], kstep[NL];
  int kin_lim[NL];
#pragma unroll
  for (int qq = 0; qq < NL; ++qq) {
    if (qq < 2) {
      const int slot = qq * 8 + wave;
      const int row = 8 * slot + (lane >> 3), c = (lane & 7) ^ swz_x(row);
      off[qq] = (uint32_t)row * (uint32_t)(2 * K) + 16u * c;
      ldso[qq] = (uint32_t)(slot * 1024);
      kstep[qq] = 128;
      kin_lim[qq] = (int)((2 * K - 16 * c + 127) / 128);
    } else {
      const int slot = (qq - 2) * 8 + wave;
      const int row = 16 * slot + (lane >> 2), c = (lane & 3) ^ swz_w(row);
      off[qq] = (uint32_t)row * (uint32_t)K + 16u * c;
      ldso[qq] = (uint32_t)(L::XS + slot * 1024);
      kstep[qq] = 64;
      kin_lim[qq] = (int)((K - 16 * c + 63) / 64);
    }
  }
  const uint32_t lds_base = (uint32_t)(uintptr_t)smem;
  auto issue = [&](int kt) {
#pragma unroll
    for (int qq = 0; qq < NL; ++qq) {
      const uint32_t dst = lds_base + (uint32_t)((kt % SG) * L::STAGE) + ldso[qq];
      const int o = kt < kin_lim[qq] ? (int)(off[qq] + kstep[qq] * (uint32_t)kt) : OOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          qq < 2 ? rx : rq, (lds_void *)(uintptr_t)__builtin_amdgcn_readfirstlane(dst), 16, o, 0,
          0, 0);
    }
  };

  // fragment offsets within a stage, per 32-k half kk of the stage
  int fxo[2][8], fwo[2][2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int R = i * 16 + r;
      fxo[kk][i] = R * 128 + 16 * ((4 * kk + g) ^ swz_x(R));
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int S = wn * 32 + j * 16 + r;
      fwo[kk][j] = L::XS + S * 64 + 16 * ((2 * kk + (g >> 1)) ^ swz_w(S)) + 8 * (g & 1);
    }
  }

  f32x4 acc[8][2];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int kt) {
    const char *st = smem + (kt % SG) * L::STAGE;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      bf16x8 fa[8], fb[2];
#pragma unroll
      for (int i = 0; i < 8; ++i) fa[i] = *reinterpret_cast<const bf16x8 *>(st + fxo[kk][i]);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const i32x2 w = *reinterpret_cast<const i32x2 *>(st + fwo[kk][j]);
        fb[j] = widen8((uint32_t)w[0], (uint32_t)w[1]);
      }
      // the MFMA run issues at raised wave priority, so the other wave of the
      // SIMD fills the gaps with its loads and widening instead of competing
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
      __builtin_amdgcn_s_setprio(0);
    }
  };

  const int nk = (int)((K + BK - 1) / BK);
#pragma unroll
  for (int s = 0; s < SG - 1; ++s) issue(s);
  int kt = 0;
  auto step = [&](int k) {
    __builtin_amdgcn_s_waitcnt(0x0F70 | (NL * (SG - 2)));
    __builtin_amdgcn_s_barrier();  // stage k complete everywhere; slot of k-1 free
    issue(k + SG - 1);
    compute(k);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // this stage's fragment reads done
  };
  const int nmain = nk - (SG - 1);
  if constexpr (SG == 4) {
    // whole turns of the ring first: each stage's LDS offsets become
    // constants (the 2-stage ring keeps its loop rolled: within the register
    // budget of two workgroups a CU the unrolled loop spills)
    for (; kt + SG - 1 < nmain; kt += SG) {
#pragma unroll
      for (int u = 0; u < SG; ++u) step(kt + u);
    }
  }
  for (; kt < nmain; ++kt) step(kt);
#pragma unroll
  for (int t = 0; t < SG - 1; ++t) {
    if (kt < nk) {
      if (t == 0) __builtin_amdgcn_s_waitcnt(0x0F70 | (NL * (SG - 2)));
      else if (t == 1) __builtin_amdgcn_s_waitcnt(0x0F70 | (SG > 3 ? NL * (SG - 3) : 0));
      else __builtin_amdgcn_s_waitcnt(0x0F70);
      __builtin_amdgcn_s_barrier();
      compute(kt);
      __builtin_amdgcn_s_waitcnt(0xC07F);
    }
    ++kt;
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();

  // scale + bias + bf16 into the LDS output tile; acc[i][j] lane holds
  // D[4g + v][r] of MFMA tile (i, j): row m, column n.
  uint16_t *tl = reinterpret_cast<uint16_t *>(smem);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int col = wn * 32 + j * 16 + r;
    const int64_t n = n0 + col;
    const float s = n < N ? scale[n] : 0.0f;
    const float b = (n < N && bias) ? bf16_to_f32(bias[n]) : 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        tl[(i * 16 + 4 * g + v) * L::TLD + col] = f32_to_bf16_rne(s * acc[i][j][v] + b);
  }
  __syncthreads();
  // 32 lanes x 16 B per 512-byte row
  const bool vec = (N & 7) == 0;
  for (int u = tid; u < BM * 32; u += 512) {
    const int row = u >> 5, c = u & 31;
    const int64_t m = m0 + row, n = n0 + 8 * c;
    if (m >= M || n >= N) continue;
    const i32x4 val = *reinterpret_cast<const i32x4 *>(tl + row * L::TLD + 8 * c);
    uint16_t *dst = y + m * N + n;
    if (vec) {
      *reinterpret_cast<i32x4 *>(dst) = val;
    } else {
      const uint16_t *h = reinterpret_cast<const uint16_t *>(&val);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (n + e < N) dst[e] = h[e];
    }
  }
}

template <int SG>
hipError_t launch_wide(const uint16_t *x, int64_t M, int64_t K, const int8_t *q, const float *scale,
                       const uint16_t *bias, int64_t N, uint16_t *y, hipStream_t st) {
  using L = WideLds<SG>;
  static bool attr_set = false;
  if (!attr_set) {  // more than 64 KB of dynamic LDS; a launch the limit refuses reports itself
    (void)hipFuncSetAttribute((const void *)k_w8a16_gemm_wide<SG>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, L::BYTES);
    (void)hipGetLastError();
    attr_set = true;
  }
  const int tiles_m = (int)((M + L::BM - 1) / L::BM), tiles_n = (int)((N + L::BNW - 1) / L::BNW);
  hipLaunchKernelGGL(k_w8a16_gemm_wide<SG>, dim3((unsigned)(tiles_m * tiles_n)), dim3(512),
                     L::BYTES, st, x, q, scale, bias, y, M, N, K, tiles_m, tiles_n);
  return hipGetLastError();
}

template <int WM>
hipError_t launch_wm(const uint16_t *x, int64_t M, int64_t K, const int8_t *q, const float *scale,
                     const uint16_t *bias, int64_t N, uint16_t *y, hipStream_t st) {
  using L = GemmLds<WM>;
  static bool attr_set = false;
  if (!attr_set) {  // more than 64 KB of dynamic LDS; a launch the limit refuses reports itself
    (void)hipFuncSetAttribute((const void *)k_w8a16_gemm<WM>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, L::BYTES);
    (void)hipGetLastError();
    attr_set = true;
  }
  const int tiles_m = (int)((M + L::BM - 1) / L::BM), tiles_n = (int)((N + BN - 1) / BN);
  hipLaunchKernelGGL(k_w8a16_gemm<WM>, dim3((unsigned)(tiles_m * tiles_n)), dim3(256 * WM),
                     L::BYTES, st, x, q, scale, bias, y, M, N, K, tiles_m, tiles_n);
  return hipGetLastError();
}

}  // namespace

// 128 x 256 tiles from 160 of them on (fewer than one per CU still beats the
// smaller tiles' extra round), two workgroups a CU from 512 on; else 128 x 128
// tiles when those fill the CUs, else 64 x 128 tiles.
hipError_t launch_w8a16_gemm(const uint16_t *x, int64_t M, int64_t K, const int8_t *q,
                             const float *scale, const uint16_t *bias, int64_t N, uint16_t *y,
                             hipStream_t st) {
  const int64_t twide = ((M + 127) / 128) * ((N + 255) / 256);
  if (twide >= 512) return launch_wide<2>(x, M, K, q, scale, bias, N, y, st);
  if (twide >= 160) return launch_wide<4>(x, M, K, q, scale, bias, N, y, st);
  const int64_t t128 = ((M + 127) / 128) * ((N + BN - 1) / BN);
  if (t128 >= 256) return launch_wm<2>(x, M, K, q, scale, bias, N, y, st);
  return launch_wm<1>(x, M, K, q, scale, bias, N, y, st);
}

}  // namespace aql
