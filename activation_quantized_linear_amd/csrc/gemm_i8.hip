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
// Tiling: a 512-thread workgroup computes a 128 (A rows) x 128
// (N) tile. Its 8 waves are 2 x 2 output quadrants of 64 x 64 (4 x 4 MFMA
// tiles each) times 2 halves of every 128-byte K stage, so two waves share
// each SIMD and one multiplies while the other waits on LDS; the halves' int32
// accumulators are added once at the end. Operand tiles go from global memory
// straight into a 4-stage LDS ring with buffer loads that write LDS (no
// registers on the way, and the hardware range check zero-fills rows past M
// or N and bytes past K). In LDS every 128-byte row stores its 16-byte chunks
// XOR-swizzled by (row / 2) mod 8, so the 16 rows x 16 bytes an MFMA fragment
// read touches hit distinct banks. Workgroups are mapped to tiles so that each
// XCD (blocks are dealt to the 8 XCDs round-robin) works on a contiguous band
// of N tiles, sharing them in its L2.
#include "common.h"

namespace aql {
namespace {

constexpr int BM = 128, BN = 128, BK = 128, STAGES = 4;
constexpr int ROWB = BK;                       // bytes per LDS row
constexpr int STAGE_BYTES = (BM + BN) * ROWB;  // 32 KB
constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
constexpr int OOB = 0x40000000;

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                           0x00020000);
}

__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

// s_waitcnt with vmcnt = n (expcnt / lgkmcnt left at their maxima).
__device__ __forceinline__ void wait_vm(int n) {
  switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt(0xF70); break;
    case 4: __builtin_amdgcn_s_waitcnt(0xF74); break;
    case 8: __builtin_amdgcn_s_waitcnt(0xF78); break;
    default: __builtin_amdgcn_s_waitcnt(0xF70); break;
  }
}

template <int EPI, bool TWO>
__global__ __launch_bounds__(512) void k_gemm_i8(GemmArgs p, int tiles_m, int tiles_n) {
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int nt = tiles_m * tiles_n;
  const int lin = blockIdx.x;
  int tile = lin;
  if ((nt & 7) == 0) tile = (lin & 7) * (nt >> 3) + (lin >> 3);
  const int tn = tile / tiles_m, tm = tile % tiles_m;
  const int64_t n0 = (int64_t)tn * BN;
  const int64_t m0 = (int64_t)tm * (TWO ? BM / 2 : BM);
  const int64_t M = p.M, N = p.N, K = p.K;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kh = wave >> 2, wm = (wave >> 1) & 1, wn = wave & 1;
  const int r = lane & 15, g = lane >> 4;

  // ---- loads: per stage 32 instructions of 8 rows x 128 B (16 A, 16 B); wave
  // w issues A groups 2w, 2w+1 and B groups 2w, 2w+1. Lane i of a group loads
  // row 8 * grp + i / 8 into LDS slot i % 8, i.e. global chunk (i % 8) ^ swz(row).
  const int mrows = TWO ? BM / 2 : BM;
  const int64_t mval = M - m0 < mrows ? M - m0 : mrows;
  const int64_t nval = N - n0 < BN ? N - n0 : BN;
  const __amdgpu_buffer_rsrc_t ra1 = rsrc(p.a1 + m0 * K, (uint32_t)(mval * K));
  const __amdgpu_buffer_rsrc_t ra2 = rsrc(TWO ? p.a2 + m0 * K : p.a1, (uint32_t)(TWO ? mval * K : 0));
  const __amdgpu_buffer_rsrc_t rb = rsrc(p.b + n0 * K, (uint32_t)(nval * K));
  uint32_t aoff[2], boff[2];
  int achunk[2], bchunk[2];
  bool apass2[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int grp = 2 * wave + q;
    const int grow = 8 * grp;                 // first tile row of the group (uniform)
    const int row = grow + (lane >> 3);       // tile row 0..127
    const int c = (lane & 7) ^ swz(row);      // global chunk landing in slot lane % 8
    int arow;  // row within its source buffer's tile
    if constexpr (TWO) {
      apass2[q] = (grow & 63) >= 32;          // 8-row groups never straddle a 32-row half
      arow = 32 * (grow >> 6) + (row & 31);
    } else {
      apass2[q] = false;
      arow = row;
    }
    aoff[q] = (uint32_t)arow * (uint32_t)K + 16u * c;
    boff[q] = (uint32_t)row * (uint32_t)K + 16u * c;
    achunk[q] = 16 * c;
    bchunk[q] = 16 * c;
  }
  auto issue = [&](int kt) {
    const int64_t k0 = (int64_t)kt * BK;
    char *st = smem + (kt % STAGES) * STAGE_BYTES;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int grp = 2 * wave + q;
      const bool kin = k0 + achunk[q] < K;
      const int ao = kin ? (int)(aoff[q] + (uint32_t)k0) : OOB;
      const int bo = (k0 + bchunk[q] < K) ? (int)(boff[q] + (uint32_t)k0) : OOB;
      lds_void *da = (lds_void *)(st + grp * 8 * ROWB);
      lds_void *db = (lds_void *)(st + BM * ROWB + grp * 8 * ROWB);
      if (TWO && apass2[q])
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra2, da, 16, ao, 0, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra1, da, 16, ao, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, db, 16, bo, 0, 0, 0);
    }
  };

  i32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = i32x4{0, 0, 0, 0};

  const int nk = (int)((K + BK - 1) / BK);
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
    if (s < nk) issue(s);

  for (int kt = 0; kt < nk; ++kt) {
    // stage kt's loads are this wave's oldest; the ones issued after it may stay
    const int ahead = (nk - 1 - kt) < (STAGES - 2) ? (nk - 1 - kt) : (STAGES - 2);
    wait_vm(4 * ahead);
    __syncthreads();  // every wave's part of stage kt is in LDS; slot kt-1 is free
    if (kt + STAGES - 1 < nk) issue(kt + STAGES - 1);

    const char *st = smem + (kt % STAGES) * STAGE_BYTES;
    const int c = 4 * kh + g;  // this lane's 16-byte chunk in the stage
    i32x4 fa[4], fb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ra_ = wm * 64 + i * 16 + r;
      const int rb_ = wn * 64 + i * 16 + r;
      fa[i] = *reinterpret_cast<const i32x4 *>(st + ra_ * ROWB + 16 * (c ^ swz(ra_)));
      fb[i] = *reinterpret_cast<const i32x4 *>(st + BM * ROWB + rb_ * ROWB + 16 * (c ^ swz(rb_)));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa[i], fb[j], acc[i][j], 0, 0, 0);
  }

  // ---- add the two K halves: waves 4..7 hand their tiles to waves 0..3
  __syncthreads();  // ring no longer read
  i32x4 *xch = reinterpret_cast<i32x4 *>(smem);
  if (kh == 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) xch[((wave - 4) * 16 + i * 4 + j) * 64 + lane] = acc[i][j];
  }
  __syncthreads();
  if (kh == 1) return;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] += xch[(wave * 16 + i * 4 + j) * 64 + lane];

  // ---- epilogue. acc[i][j] lane holds D[4g + v][r] of MFMA tile (i, j).
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

template <int EPI, bool TWO>
hipError_t launch_one(const GemmArgs &a, int tiles_m, int tiles_n, hipStream_t st) {
  // 128 KB of dynamic LDS: raise the function's limit (idempotent; on a runtime
  // that does not need it the call's status is irrelevant, the launch reports).
  static bool attr_set = false;
  if (!attr_set) {
    (void)hipFuncSetAttribute((const void *)k_gemm_i8<EPI, TWO>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
    (void)hipGetLastError();
    attr_set = true;
  }
  hipLaunchKernelGGL((k_gemm_i8<EPI, TWO>), dim3((unsigned)(tiles_m * tiles_n)), dim3(512),
                     LDS_BYTES, st, a, tiles_m, tiles_n);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_i8(const GemmArgs &a, GemmEpi epi, bool two_pass, hipStream_t st) {
  const int rows = two_pass ? BM / 2 : BM;
  const int tiles_m = (int)((a.M + rows - 1) / rows);
  const int tiles_n = (int)((a.N + BN - 1) / BN);
  switch (epi) {
    case EPI_RAW: return launch_one<EPI_RAW, false>(a, tiles_m, tiles_n, st);
    case EPI_Q8TA:
      return two_pass ? launch_one<EPI_Q8TA, true>(a, tiles_m, tiles_n, st)
                      : launch_one<EPI_Q8TA, false>(a, tiles_m, tiles_n, st);
    case EPI_DQ8: return launch_one<EPI_DQ8, false>(a, tiles_m, tiles_n, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace aql
