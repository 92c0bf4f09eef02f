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
// Tiling: a 512-thread workgroup computes a 128 (A rows) x 128 (N) tile. Its
// 8 waves are 2 x 2 output quadrants of 64 x 64 (4 x 4 MFMA tiles each) times
// 2 halves of every 128-byte K stage, so two waves share each SIMD; the halves'
// int32 accumulators are added once at the end.
//
// Operand path: global memory -> LDS by buffer loads that write LDS directly
// (no registers on the way; the hardware range check zero-fills rows past M or
// N and bytes past K) into a 4-stage ring, three stages in flight. Every wave
// waits for its own loads of the stage it is about to read (an explicit vmcnt
// whose count the straight-line loop makes exact) and then meets the others at
// a bare s_barrier: no memory fence, so loads of later stages stay in flight
// across it. In LDS each 128-byte row stores its 16-byte chunks XOR-swizzled by
// (row / 2) mod 8, so the 16 rows x 16 bytes a fragment read touches hit
// distinct banks. Workgroups are mapped to tiles so that each XCD (blocks are
// dealt to the 8 XCDs round-robin) works on a contiguous band of N tiles.
//
// Epilogue: the output tile is assembled in LDS (row stride 132 words, bank-
// conflict free for the MFMA output layout) and written with 16-byte stores of
// whole rows.
#include "gemm_i8.h"

namespace aql {
namespace {

constexpr int BM = 128, BN = 128, BK = 128, STAGES = 4;
constexpr int ROWB = BK;                       // bytes per LDS ring row
constexpr int STAGE_BYTES = (BM + BN) * ROWB;  // 32 KB
constexpr int RING_BYTES = STAGES * STAGE_BYTES;
constexpr int XCH_BYTES = 4 * 16 * 64 * 16;    // 4 waves x 16 MFMA tiles x 64 lanes x 16 B
constexpr int TILE_LD = BN + 4;                // words per staged output row
constexpr int TILE_BYTES = BM * TILE_LD * 4;
constexpr int LDS_BYTES = RING_BYTES > XCH_BYTES + TILE_BYTES ? RING_BYTES : XCH_BYTES + TILE_BYTES;
constexpr int OOB = 0x40000000;

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                           0x00020000);
}

__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

// s_waitcnt vmcnt(N) with expcnt / lgkmcnt left at their maxima (N < 16).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}
// s_waitcnt lgkmcnt(0) (vmcnt / expcnt at their maxima).
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// MODE: 0 one pass, 128 rows a tile; 1 two passes stacked, 64 rows a tile;
// 2 one pass, 64 rows a tile, in the two-pass layout with the pass-2 half of
// the A tile zero-filled (for grids that would otherwise leave CUs idle).
template <int EPI, int MODE>
__global__ __launch_bounds__(512) void k_gemm_i8(GemmArgs p, int tiles_m, int tiles_n) {
  constexpr bool TWO = MODE != 0;  // the two-pass A-tile layout
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int nt = tiles_m * tiles_n;
  const int lin = blockIdx.x;
  int tile = lin;
  if ((nt & 7) == 0) tile = (lin & 7) * (nt >> 3) + (lin >> 3);
  const int tn = tile / tiles_m, tm = tile % tiles_m;
  constexpr int MROWS = TWO ? BM / 2 : BM;  // output rows per tile
  const int64_t n0 = (int64_t)tn * BN;
  const int64_t m0 = (int64_t)tm * MROWS;
  const int64_t M = p.M, N = p.N, K = p.K;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kh = wave >> 2, wm = (wave >> 1) & 1, wn = wave & 1;
  const int r = lane & 15, g = lane >> 4;

  // ---- loads: per stage 32 instructions of 8 rows x 128 B. Wave w fills tile
  // rows 16w .. 16w+15 of A and of B (2 instructions each). Lane i of an
  // instruction writes LDS row 8q + i/8, slot i % 8, i.e. global chunk
  // (i % 8) ^ swz(row). For the two-pass tile, rows [64h, 64h+32) hold pass-1
  // rows 32h .. 32h+31 and rows [64h+32, 64h+64) the same rows of pass 2; a
  // wave's 16 rows never straddle the halves, so its source is uniform.
  const int64_t mval = M - m0 < MROWS ? M - m0 : MROWS;
  const int64_t nval = N - n0 < BN ? N - n0 : BN;
  const bool apass2 = TWO && ((16 * wave) & 63) >= 32;
  const int8_t *abase = apass2 && MODE == 1 ? p.a2 : p.a1;
  // MODE 2: the pass-2 half of the tile reads nothing (an empty range loads zeros)
  const __amdgpu_buffer_rsrc_t ra =
      rsrc(abase + m0 * K, MODE == 2 && apass2 ? 0u : (uint32_t)(mval * K));
  const __amdgpu_buffer_rsrc_t rb = rsrc(p.b + n0 * K, (uint32_t)(nval * K));
  uint32_t aoff[2], boff[2];
  int chunk[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int row = 16 * wave + 8 * q + (lane >> 3);  // tile row 0..127
    const int c = (lane & 7) ^ swz(row);
    const int arow = TWO ? 32 * (row >> 6) + (row & 31) : row;
    aoff[q] = (uint32_t)arow * (uint32_t)K + 16u * c;
    boff[q] = (uint32_t)row * (uint32_t)K + 16u * c;
    chunk[q] = 16 * c;
  }
  const uint32_t lds_base = (uint32_t)(uintptr_t)smem;
  auto issue = [&](int kt) {
    const uint32_t k0 = (uint32_t)kt * BK;
    const uint32_t sa = lds_base + (uint32_t)((kt % STAGES) * STAGE_BYTES) + (uint32_t)(wave * 16 * ROWB);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const bool kin = (int64_t)k0 + chunk[q] < K;
      const int ao = kin ? (int)(aoff[q] + k0) : OOB;
      const int bo = kin ? (int)(boff[q] + k0) : OOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          ra, (lds_void *)(uintptr_t)__builtin_amdgcn_readfirstlane(sa + q * 8 * ROWB), 16, ao, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rb, (lds_void *)(uintptr_t)__builtin_amdgcn_readfirstlane(sa + BM * ROWB + q * 8 * ROWB), 16,
          bo, 0, 0, 0);
    }
  };

  // fragment offsets within a stage: 16 rows x this lane's 16-byte chunk
  int fao[4], fbo[4];
  {
    const int c = 4 * kh + g;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ra_ = wm * 64 + i * 16 + r, rb_ = wn * 64 + i * 16 + r;
      fao[i] = ra_ * ROWB + 16 * (c ^ swz(ra_));
      fbo[i] = BM * ROWB + rb_ * ROWB + 16 * (c ^ swz(rb_));
    }
  }

  i32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = i32x4{0, 0, 0, 0};

  auto compute = [&](int kt) {
    const char *st = smem + (kt % STAGES) * STAGE_BYTES;
    i32x4 fa[4], fb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      fa[i] = *reinterpret_cast<const i32x4 *>(st + fao[i]);
      fb[i] = *reinterpret_cast<const i32x4 *>(st + fbo[i]);
    }
    // the MFMA run issues at raised wave priority, so the other wave of the
    // SIMD fills the gaps with its loads instead of competing
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa[i], fb[j], acc[i][j], 0, 0, 0);
    __builtin_amdgcn_s_setprio(0);
  };

  // Prologue issues stages 0 .. STAGES-2 (ranges past K load zeros). The main
  // loop keeps STAGES-1 stages in flight; the tail drains them. Every wave
  // issues 4 loads per stage, so "stage kt landed" is vmcnt <= 4 x (stages
  // issued after it).
  const int nk = (int)((K + BK - 1) / BK);
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s) issue(s);
  int kt = 0;
  auto step = [&](int k) {
    wait_vm<4 * (STAGES - 2)>();
    __builtin_amdgcn_s_barrier();  // stage k complete everywhere; slot of k-1 free
    issue(k + STAGES - 1);
    compute(k);
    wait_lgkm0();  // this stage's fragment reads done before its slot is refilled
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
      if (t == 0) wait_vm<4 * (STAGES - 2)>();
      else if (t == 1) wait_vm<4 * (STAGES - 3)>();
      else wait_vm<0>();
      __builtin_amdgcn_s_barrier();
      compute(kt);
      wait_lgkm0();
    }
    ++kt;
  }
  wait_vm<0>();

  // ---- add the two K halves: waves 4..7 hand their tiles to waves 0..3
  __syncthreads();  // ring no longer read or written
  i32x4 *xch = reinterpret_cast<i32x4 *>(smem);
  if (kh == 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) xch[((wave - 4) * 16 + i * 4 + j) * 64 + lane] = acc[i][j];
  }
  __syncthreads();

  // ---- epilogue into the LDS output tile (after the exchange area).
  // acc[i][j] lane holds D[4g + v][r] of MFMA tile (i, j).
  char *tl = smem + XCH_BYTES;
  if (kh == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] += xch[(wave * 16 + i * 4 + j) * 64 + lane];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = wn * 64 + j * 16 + r;
      const int64_t n = n0 + col;
      const bool nin = n < N;
      // output rows of this wave: MROWS / 2 from row wm MROWS / 2 (MODE 2: only
      // the first two MFMA rows of each wave hold pass-1 rows)
      constexpr int RI = MODE == 2 ? 2 : 4;
      if constexpr (EPI == EPI_RAW) {
        int *t = reinterpret_cast<int *>(tl);
#pragma unroll
        for (int i = 0; i < RI; ++i)
#pragma unroll
          for (int v = 0; v < 4; ++v) t[(wm * (MROWS / 2) + i * 16 + 4 * g + v) * TILE_LD + col] = acc[i][j][v];
      } else if constexpr (EPI == EPI_Q8TA) {
        float *t = reinterpret_cast<float *>(tl);
        const int ws = nin ? p.wsum[n] : 0;
        const float wsc = nin ? p.wscale[n] : 0.0f;
        const float b = (nin && p.bias) ? p.bias[n] : 0.0f;
        // sum_k (xq - z) q = acc - z * wsum fits int32 (|.| <= K * 255 * 128); the
        // intermediate terms are formed in wrapping unsigned arithmetic.
        const uint32_t zw1 = (uint32_t)p.z1 * (uint32_t)ws, zw2 = (uint32_t)p.z2 * (uint32_t)ws;
        if constexpr (MODE == 2) {
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int v = 0; v < 4; ++v)
              t[(wm * 32 + i * 16 + 4 * g + v) * TILE_LD + col] =
                  wsc * (p.s1 * (float)(int)((uint32_t)acc[i][j][v] - zw1)) + b;
        } else if constexpr (TWO) {
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const float f = p.s1 * (float)(int)((uint32_t)acc[i][j][v] - zw1) +
                              p.s2 * (float)(int)((uint32_t)acc[i + 2][j][v] - zw2);
              t[(wm * 32 + i * 16 + 4 * g + v) * TILE_LD + col] = wsc * f + b;
            }
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int v = 0; v < 4; ++v)
              t[(wm * 64 + i * 16 + 4 * g + v) * TILE_LD + col] =
                  wsc * (p.s1 * (float)(int)((uint32_t)acc[i][j][v] - zw1)) + b;
        }
      } else {  // EPI_DQ8
        float *t = reinterpret_cast<float *>(tl);
        const int ws = nin ? p.wsum[n] : 0;
        const float wsc = nin ? p.wscale[n] : 0.0f;
        const float b = (nin && p.bias) ? p.bias[n] : 0.0f;
#pragma unroll
        for (int i = 0; i < RI; ++i)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int row = wm * (MROWS / 2) + i * 16 + 4 * g + v;
            const int64_t m = m0 + row;
            const bool min_ = m < M;
            const int xz = min_ ? p.xz[m] : 0;
            const float xs = min_ ? p.xs[m] : 0.0f;
            const int A = (int)((uint32_t)acc[i][j][v] - (uint32_t)xz * (uint32_t)ws);
            t[row * TILE_LD + col] = xs * (wsc * (float)A) + b;
          }
      }
    }
  }
  __syncthreads();

  // ---- write the tile: 32 lanes x 16 B per row
  const bool vec = (N & 3) == 0;
#pragma unroll
  for (int s = 0; s < MROWS / 16; ++s) {
    const int u = tid + 512 * s, row = u >> 5, c = u & 31;
    const int64_t m = m0 + row, n = n0 + 4 * c;
    if (m >= M || n >= N) continue;
    const i32x4 val = *reinterpret_cast<const i32x4 *>(tl + (row * TILE_LD + 4 * c) * 4);
    int *dst = EPI == EPI_RAW ? p.c + m * N + n : reinterpret_cast<int *>(p.y + m * N + n);
    if (vec) {
      *reinterpret_cast<i32x4 *>(dst) = val;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (n + e < N) dst[e] = val[e];
    }
  }
}

template <int EPI, int MODE>
hipError_t launch_one(const GemmArgs &a, int tiles_m, int tiles_n, hipStream_t st) {
  // More than 64 KB of dynamic LDS: raise the function's limit once. Its status
  // is not needed: a launch the limit does not allow reports its own error.
  static bool attr_set = false;
  if (!attr_set) {
    (void)hipFuncSetAttribute((const void *)k_gemm_i8<EPI, MODE>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
    (void)hipGetLastError();
    attr_set = true;
  }
  hipLaunchKernelGGL((k_gemm_i8<EPI, MODE>), dim3((unsigned)(tiles_m * tiles_n)), dim3(512),
                     LDS_BYTES, st, a, tiles_m, tiles_n);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_i8(const GemmArgs &a, GemmEpi epi, bool two_pass, hipStream_t st) {
  const int tiles_n = (int)((a.N + BN - 1) / BN);
  const int tiles_m128 = (int)((a.M + BM - 1) / BM), tiles_m64 = (int)((a.M + BM / 2 - 1) / (BM / 2));
  // one pass: 64-row tiles while 128-row tiles would leave CUs idle (M = 512,
  // N = K = 4096: 128 tiles of 128 rows; 27.3 -> 24.9 us for the static op)
  const bool half = tiles_m128 * tiles_n < 256;
  switch (epi) {
    case EPI_RAW:
      return half ? launch_one<EPI_RAW, 2>(a, tiles_m64, tiles_n, st)
                  : launch_one<EPI_RAW, 0>(a, tiles_m128, tiles_n, st);
    case EPI_Q8TA:
      if (two_pass) return launch_one<EPI_Q8TA, 1>(a, tiles_m64, tiles_n, st);
      return half ? launch_one<EPI_Q8TA, 2>(a, tiles_m64, tiles_n, st)
                  : launch_one<EPI_Q8TA, 0>(a, tiles_m128, tiles_n, st);
    case EPI_DQ8:
      return half ? launch_one<EPI_DQ8, 2>(a, tiles_m64, tiles_n, st)
                  : launch_one<EPI_DQ8, 0>(a, tiles_m128, tiles_n, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace aql
