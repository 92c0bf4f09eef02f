// Weight-only W8A16 linear: y[m, n] = scale[n] * sum_k x[m, k] * q[n, k] (+ bias[n]).
//
// tiny-llm quant, Step 4.6: the per-channel scale factors out of the sum, and
// int8 -> bf16 is exact, so the sum can run on the bf16 matrix cores with the
// int8 codes widened in registers and the scale applied once per output.
//
// Access shape. The kernel is bound by streaming the weights from HBM. On
// gfx950 a wave instruction that reads 4 rows x 256 contiguous bytes streams
// markedly faster than the 16 rows x 64 bytes a 16x16 MFMA fragment would ask
// for, so the weights are loaded in that 4-row shape and multiplied where they
// land with v_mfma_f32_4x4x4_16b_bf16: its 16 blocks of 4 lanes each take one
// 16-byte k-slice (block b = lane / 4) of 4 weight rows (column j = lane % 4),
// against the same k-slice of 4 rows of x (row i = lane % 4 of the A operand).
//
// Tile: one workgroup owns 16 output channels (4 row groups t of 4) and up to
// 16 rows of x (MB blocks of 4); its W waves split K into 256-byte steps (wave
// w takes steps w, w + W, ...). Per step a lane loads 16 weight bytes of each
// row group and the 16 matching bf16 of x per m block, and issues 4 MFMAs per
// (t, m block). Loads are buffer loads: the hardware range check returns zero
// past the tile's rows and past K (no branches), and steps are fetched in
// batches of U with the next batch in flight while the current one is
// multiplied. At the end the 16 k-slice partials are summed across lanes
// (shuffles over lane bits 2..5) and the waves' tiles meet once in LDS.
//
// Launches: a single problem (grid = N/16 x M/16 tiles), or a group of
// independent problems in one launch (a decode sweep's linears), whose tiles
// are laid end to end in one grid and found through a device table.
#include <type_traits>

#include "w8a16.h"
#include "w8a16_gemm.h"

namespace aql {
namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

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

// Four int8 codes (one dword, little-endian) -> four bf16 in order.
__device__ __forceinline__ s16x4 widen4(int w) {
  const uint32_t lo = bf16x2_from_i8((int)(int8_t)(w), (int)(int8_t)(w >> 8));
  const uint32_t hi = bf16x2_from_i8((int)(int8_t)(w >> 16), (w >> 24));
  return __builtin_bit_cast(s16x4, (uint64_t)lo | ((uint64_t)hi << 32));
}

// Cross-lane sums without LDS: DPP row rotations within a row of 16 lanes,
// and the gfx950 lane-half swaps across rows (v_permlane16_swap pairs rows
// 0-1 and 2-3, v_permlane32_swap the two halves of the wave).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
constexpr int kDppRowRor4 = 0x124, kDppRowRor8 = 0x128, kDppRowMirror = 0x140,
              kDppRowHalfMirror = 0x141, kDppQuadXor1 = 0xB1, kDppQuadXor2 = 0x4E;
// (a, b) -> a' + b' where lanes 0-31 get a[l] + a[l + 32] and lanes 32-63
// get b[l - 32] + b[l]: a's pair sum in the low half, b's in the high half.
__device__ __forceinline__ float swap32_sum(float a, float b) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}
// The same across rows of 16: rows 0 and 2 get a's sums with rows 1 and 3,
// rows 1 and 3 get b's.
__device__ __forceinline__ float swap16_sum(float a, float b) {
  const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
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

// LDS for the cross-wave reduction: per wave, per (row group, m block), per
// column j, four rows of x. MB = 0 is the single-row (M = 1) tile.
template <int W, int TG, int MB>
struct Red {
  f32x4 v[W][TG][MB > 0 ? MB : 1][4];
};

// M = 1: per step each lane takes 8 contiguous bytes of x (4 bf16; a wave's
// 64 lanes cover the step's 512 bytes), k-quarter i = lane % 4 of its block's
// 16-element slice, and uses it as the A operand row i for all four
// k-quarters e of the weights. Block b then computes D[i][j] = x_i . w_e(j),
// which is wanted only for i = e, so each e accumulates separately and the
// wanted value of accumulator e sits in its VGPR e.
//
// A workgroup holds CW wave tiles of 4 TG channels side by side along N, each
// with W waves splitting K. With XL the workgroup first copies x (2 K bytes)
// into LDS by direct buffer-to-LDS loads, so x is read from L2 once per
// workgroup instead of once per wave tile, and each step reads its 8 bytes per
// lane from LDS. The copy is issued before the first weight batch and waited
// for after it, so its latency hides behind the weights'.
template <int W, int CW, int TG, int U, bool XL>
__device__ __forceinline__ void w8a16_tile_m1(const Tile &t, Red<W * CW, TG, 0> &red,
                                              uint8_t *xs) {
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int cw = wid / W, wave = wid % W;
  const int j = lane & 3, blk = lane >> 2;
  const int64_t K = t.K;
  const int64_t n0 = t.n0 + 4 * TG * cw;
  // a wave tile wholly past N gets an empty range (all its weight loads read 0)
  const int64_t rem = t.N - n0;
  const int64_t nrows = rem <= 0 ? 0 : (rem < 4 * TG ? rem : 4 * TG);
  const __amdgpu_buffer_rsrc_t rq =
      rsrc(nrows > 0 ? t.q + n0 * K : t.q, (uint32_t)(nrows * K));
  const __amdgpu_buffer_rsrc_t rx = rsrc(t.x + t.m0 * K, (uint32_t)(K * 2));
  const uint32_t qlane = (uint32_t)(j * K + 16 * blk);
  const uint32_t xlane = 8u * (uint32_t)lane;
  const int nst = (int)((K + 255) >> 8);
  const int cnt = wave < nst ? (nst - wave + W - 1) / W : 0;

  if constexpr (XL) {
    // 1 KiB per wave instruction (16 bytes per lane); past 2 K the range check
    // writes zeros, which the last step's lanes past K then read
    const int nch = (int)((2 * K + 1023) >> 10);
    const uint32_t base = (uint32_t)(uintptr_t)xs;
    for (int c = wid; c < nch; c += W * CW)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rx, (lds_void *)(uintptr_t)__builtin_amdgcn_readfirstlane(base + 1024u * c), 16,
          (int)(16u * lane + 1024u * c), 0, 0, 0);
  }

  f32x4 acc[TG][4];
#pragma unroll
  for (int tg = 0; tg < TG; ++tg)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[tg][e] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto fetch_w = [&](int i0, i32x4 (*w_)[TG]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int st = wave + W * (i0 + u);
      const uint32_t qstep = i0 + u < cnt ? 256u * st : (uint32_t)OOB;  // uniform
#pragma unroll
      for (int tg = 0; tg < TG; ++tg) {
        const int qo = (int)(qlane + (uint32_t)(4 * tg) * (uint32_t)K + qstep);
        w_[u][tg] = __builtin_amdgcn_raw_buffer_load_b128(rq, qo, 0, 2);
      }
    }
  };
  auto fetch_x = [&](int i0, i32x2 *x_) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int st = wave + W * (i0 + u);
      const bool valid = i0 + u < cnt;  // uniform
      if constexpr (XL) {
        // steps past the wave's last read a valid address; mul zeroes them
        x_[u] = *reinterpret_cast<const i32x2 *>(xs + (valid ? 512u * st : 0u) + xlane);
      } else {
        const bool kin = (256 * st + 16 * blk) < K;
        const int xo = (valid && kin) ? (int)(xlane + 512u * st) : OOB;
        x_[u] = __builtin_bit_cast(i32x2, __builtin_amdgcn_raw_buffer_load_b64(rx, xo, 0, 0));
      }
    }
  };
  auto mul = [&](int i0, i32x4 (*w_)[TG], i32x2 *x_) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const i32x2 xv = (!XL || i0 + u < cnt) ? x_[u] : i32x2{0, 0};  // uniform
      const s16x4 a = __builtin_bit_cast(s16x4, xv);
#pragma unroll
      for (int tg = 0; tg < TG; ++tg)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          acc[tg][e] = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(a, widen4(w_[u][tg][e]), acc[tg][e], 0, 0, 0);
    }
  };

  // The loop body runs at least once (a wave without steps multiplies zeros):
  // the first batch is then used unconditionally and cannot be sunk past the
  // wait below, whose count assumes its U TG loads were issued after the copy.
  i32x4 w0[U][TG], w1[U][TG];
  i32x2 x0[U], x1[U];
  fetch_w(0, w0);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (XL) {
    static_assert(U * TG < 16, "vmcnt immediate");
    __builtin_amdgcn_s_waitcnt(0x0F70 | (U * TG));  // this wave's copies done
    __builtin_amdgcn_s_barrier();                   // every wave's copies done
  }
  fetch_x(0, x0);
  int b = 0;
  do {
    fetch_w(b + U, w1);
    fetch_x(b + U, x1);
    __builtin_amdgcn_sched_barrier(0);
    mul(b, w0, x0);
    __builtin_amdgcn_sched_barrier(0);
    fetch_w(b + 2 * U, w0);
    fetch_x(b + 2 * U, x0);
    __builtin_amdgcn_sched_barrier(0);
    mul(b + U, w1, x1);
    __builtin_amdgcn_sched_barrier(0);
    b += 2 * U;
  } while (b < cnt);

  // sum the 16 k-slice blocks of column j (lanes j, j + 4, ..., j + 60): two
  // row rotations, then the two lane-half swaps; every lane ends with its
  // column's total
  float v[TG];
#pragma unroll
  for (int tg = 0; tg < TG; ++tg) {
    v[tg] = (acc[tg][0][0] + acc[tg][1][1]) + (acc[tg][2][2] + acc[tg][3][3]);
    v[tg] += dpp_f32<kDppRowRor4>(v[tg]);
    v[tg] += dpp_f32<kDppRowRor8>(v[tg]);
    v[tg] = swap16_sum(v[tg], v[tg]);
    v[tg] = swap32_sum(v[tg], v[tg]);
  }
  if constexpr (W > 1) {
    if (lane < 4) {
#pragma unroll
      for (int tg = 0; tg < TG; ++tg) red.v[wid][tg][0][j] = f32x4{v[tg], 0.f, 0.f, 0.f};
    }
    __syncthreads();
  }
  if (wave != 0 || lane >= 4 * TG) return;
  const int64_t n = n0 + lane;
  if (n >= t.N) return;
  float sum;
  if constexpr (W > 1) {
    const int tg = lane >> 2, jj = lane & 3;
    sum = red.v[wid][tg][0][jj][0];
#pragma unroll
    for (int w = 1; w < W; ++w) sum += red.v[wid + w][tg][0][jj][0];
  } else {
    // lane 4 tg + jj holds v[tg] of column jj (every lane of a column agrees)
    sum = v[0];
#pragma unroll
    for (int tg = 1; tg < TG; ++tg) sum = (lane >> 2) == tg ? v[tg] : sum;
  }
  const float bv = t.bias ? bf16_to_f32(t.bias[n]) : 0.0f;
  t.y[t.m0 * t.N + n] = f32_to_bf16_rne(t.scale[n] * sum + bv);
}

// TG row groups of 4 output channels per tile (4 TG channels), MB blocks of 4
// rows of x, W waves, U steps per fetched batch.
template <int W, int TG, int MB, int U>
__device__ __forceinline__ void w8a16_tile(const Tile &t, Red<W, TG, MB> &red) {
  const int lane = threadIdx.x & 63;
  // wave-uniform (scalar) so that per-step offsets are scalar selects, not branches
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int j = lane & 3, blk = lane >> 2;  // column (weight row in group) / k-slice
  const int64_t K = t.K;
  const int64_t nrows = t.N - t.n0 < 4 * TG ? t.N - t.n0 : 4 * TG;
  const int64_t mrows = t.M - t.m0 < 16 ? t.M - t.m0 : 16;
  const __amdgpu_buffer_rsrc_t rq = rsrc(t.q + t.n0 * K, (uint32_t)(nrows * K));
  const __amdgpu_buffer_rsrc_t rx = rsrc(t.x + t.m0 * K, (uint32_t)(mrows * K * 2));
  // weights: row group tg, lane -> row 4 tg + j, bytes 16 blk of the step
  const uint32_t qlane = (uint32_t)(j * K + 16 * blk);
  // x: m block mb, lane -> row 4 mb + j of x (the A operand row is lane % 4)
  const uint32_t xlane = 2u * (uint32_t)(j * K + 16 * blk);
  const int nst = (int)((K + 255) >> 8);
  const int cnt = wave < nst ? (nst - wave + W - 1) / W : 0;

  f32x4 acc[TG][MB];
#pragma unroll
  for (int tg = 0; tg < TG; ++tg)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[tg][mb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // one step: 4 weight loads (row groups), 2 x loads per m block
  auto fetch = [&](int i0, i32x4 (*w_)[TG], i32x4 (*x_)[MB][2]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u;
      const int st = wave + W * i;
      const bool valid = i < cnt;  // uniform
      // per-lane: this lane's 16-byte k-slice lies before K (only the last step can end early)
      const bool kin = (256 * st + 16 * blk) < K;
      const uint32_t qstep = valid ? 256u * st : (uint32_t)OOB;
      const uint32_t xstep = valid ? 512u * st : (uint32_t)OOB;
#pragma unroll
      for (int tg = 0; tg < TG; ++tg) {
        const int qo = (int)(qlane + (uint32_t)(4 * tg) * (uint32_t)K + qstep);
        w_[u][tg] = __builtin_amdgcn_raw_buffer_load_b128(rq, qo, 0, 2);
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int xo = kin ? (int)(xlane + 2u * (uint32_t)(4 * mb) * (uint32_t)K + xstep) : OOB;
        x_[u][mb][0] = __builtin_amdgcn_raw_buffer_load_b128(rx, xo, 0, 0);
        x_[u][mb][1] = __builtin_amdgcn_raw_buffer_load_b128(rx, xo + 16, 0, 0);
      }
    }
  };
  auto mul = [&](i32x4 (*w_)[TG], i32x4 (*x_)[MB][2]) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int tg = 0; tg < TG; ++tg)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const s16x4 b = widen4(w_[u][tg][e]);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
            const i32x4 xv = x_[u][mb][e >> 1];
            const s16x4 a = __builtin_bit_cast(
                s16x4, (uint64_t)(uint32_t)xv[(e & 1) * 2] |
                           ((uint64_t)(uint32_t)xv[(e & 1) * 2 + 1] << 32));
            acc[tg][mb] = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(a, b, acc[tg][mb], 0, 0, 0);
          }
        }
  };

  // Ping-pong over two register batches; sched_barrier keeps the compiler from
  // regrouping the phases, and a batch past the wave's last step loads zeros
  // so the loop needs no early exit (one would let the loads sink).
  i32x4 w0[U][TG], w1[U][TG], x0[U][MB][2], x1[U][MB][2];
  fetch(0, w0, x0);
  for (int b = 0; b < cnt; b += 2 * U) {
    fetch(b + U, w1, x1);
    __builtin_amdgcn_sched_barrier(0);
    mul(w0, x0);
    __builtin_amdgcn_sched_barrier(0);
    fetch(b + 2 * U, w0, x0);
    __builtin_amdgcn_sched_barrier(0);
    mul(w1, x1);
    __builtin_amdgcn_sched_barrier(0);
  }

  // Sum the 16 k-slice blocks: lanes j, j + 4, ..., j + 60.
#pragma unroll
  for (int tg = 0; tg < TG; ++tg)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int o = 4; o < 64; o <<= 1)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[tg][mb][v] += __shfl_xor(acc[tg][mb][v], o);

  if (lane < 4) {
#pragma unroll
    for (int tg = 0; tg < TG; ++tg)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) red.v[wave][tg][mb][j] = acc[tg][mb];
  }
  if constexpr (W > 1) __syncthreads();
  // wave 0, lanes 0..4TG-1: output channel n0 + lane (row group lane / 4, column lane % 4)
  if (wave != 0 || lane >= 4 * TG) return;
  const int tg = lane >> 2, jj = lane & 3;
  const int64_t n = t.n0 + lane;
  if (n >= t.N) return;
  const float s = t.scale[n];
  const float bv = t.bias ? bf16_to_f32(t.bias[n]) : 0.0f;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    f32x4 sum = red.v[0][tg][mb][jj];
#pragma unroll
    for (int w = 1; w < W; ++w) sum += red.v[w][tg][mb][jj];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t mm = t.m0 + 4 * mb + v;
      if (mm < t.M) t.y[mm * t.N + n] = f32_to_bf16_rne(s * sum[v] + bv);
    }
  }
}

// Skinny tile (16 rows of x, 16 NT channels): one v_mfma_f32_16x16x32_bf16
// per 32 k and 16 channels, x as the A operand (row m = lane % 16), the
// widened int8 weights as B (channel n = lane % 16), so a lane keeps one
// 16 x 16 accumulator tile per 16 channels instead of the 4 x 4 x 4 tile's 16
// k-slice partials, and each matrix instruction does 8x the work. The k order
// inside a step is free as long as x and the weights use the same one: lane
// group g = lane / 16 of instruction (h, half) takes k = 256 step + 64 h +
// 16 g + 8 half + e (e = 0..7), so a lane reads 16 contiguous weight bytes of
// its channel and 32 contiguous x bytes of its row.
//
// The weights arrive in the fast streaming shape, 4 rows x 256 bytes per wave
// instruction, by buffer loads that write LDS directly, into a per-wave
// double-buffered slot (no barrier: no other wave reads it); each 16-byte
// chunk c of row r sits at slot c ^ (r % 16), so the MFMA-order reads of 16
// rows hit distinct banks. x comes into registers. W waves split K into
// 256-byte steps; the next step's loads are in flight while one is multiplied.
template <int W, int NT>
struct SkLds {
  uint8_t w[W][2][16 * NT * 256];  // per wave, two step slots of 16 NT rows x 256 B
  f32x4 red[W][NT][64];
};

// s_waitcnt vmcnt(N) with expcnt / lgkmcnt left at their maxima (N < 64).
template <int N>
__device__ __forceinline__ void sk_wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

template <int W, int NT>
__device__ __forceinline__ void w8a16_tile_sk(const Tile &t, SkLds<W, NT> &sm) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int64_t K = t.K;
  const int64_t nrows = t.N - t.n0 < 16 * NT ? t.N - t.n0 : 16 * NT;
  const int64_t mrows = t.M - t.m0 < 16 ? t.M - t.m0 : 16;
  const __amdgpu_buffer_rsrc_t rq = rsrc(t.q + t.n0 * K, (uint32_t)(nrows * K));
  const __amdgpu_buffer_rsrc_t rx = rsrc(t.x + t.m0 * K, (uint32_t)(mrows * K * 2));
  const int nst = (int)((K + 255) >> 8);
  const int cnt = wave < nst ? (nst - wave + W - 1) / W : 0;
  // weight DMA: instruction i of a step covers rows 4 i .. 4 i + 3; lane l
  // writes row 4 i + l / 16, slot l % 16 with chunk (l % 16) ^ (row % 16)
  const int drow = lane >> 4, dslot = lane & 15;
  const uint32_t xlane = 2u * (uint32_t)(r * K + 16 * g);  // row r, elements 16 g
  const uint32_t lds0 = (uint32_t)(uintptr_t)&sm.w[wave][0][0];

  f32x4 acc[NT];
#pragma unroll
  for (int c = 0; c < NT; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};

  constexpr int NV = 4 * NT + 8;  // vector memory instructions per step
  auto fetch = [&](int i, int slot, i32x4 (*x_)[2]) {
    const int st = wave + W * i;
    const bool valid = i < cnt;  // uniform
    const __amdgpu_buffer_rsrc_t rqv = rq;
#pragma unroll
    for (int d = 0; d < 4 * NT; ++d) {
      const int row = 4 * d + drow;
      const int c = dslot ^ (row & 15);
      const bool kin = valid && (256 * st + 16 * c) < K;
      const int qo = kin ? (int)((uint32_t)row * (uint32_t)K + 256u * st + 16u * c) : OOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rqv,
          (lds_void *)(uintptr_t)__builtin_amdgcn_readfirstlane(lds0 + (uint32_t)slot * (16 * NT * 256) +
                                                                 1024u * d),
          16, qo, 0, 0, 0);
    }
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const bool kin = valid && (256 * st + 64 * h + 16 * g) < K;
      const int xo = kin ? (int)(xlane + 512u * st + 128u * h) : OOB;
      x_[h][0] = __builtin_amdgcn_raw_buffer_load_b128(rx, xo, 0, 0);
      x_[h][1] = __builtin_amdgcn_raw_buffer_load_b128(rx, xo + 16, 0, 0);
    }
  };
  auto mul = [&](int slot, i32x4 (*x_)[2]) {
    const uint8_t *wl = &sm.w[wave][slot][0];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      i32x4 wq[NT];
#pragma unroll
      for (int c = 0; c < NT; ++c) {
        const int row = 16 * c + r;
        wq[c] = *reinterpret_cast<const i32x4 *>(wl + 256 * row + 16 * ((4 * h + g) ^ r));
      }
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const bf16x8 a = __builtin_bit_cast(bf16x8, x_[h][half]);
#pragma unroll
        for (int c = 0; c < NT; ++c) {
          const s16x4 lo = widen4(wq[c][2 * half]), hi = widen4(wq[c][2 * half + 1]);
          const i32x2 l2 = __builtin_bit_cast(i32x2, lo), h2 = __builtin_bit_cast(i32x2, hi);
          const bf16x8 b = __builtin_bit_cast(bf16x8, i32x4{l2[0], l2[1], h2[0], h2[1]});
          acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[c], 0, 0, 0);
        }
      }
    }
  };

  // Ping-pong over the two slots; a step past the wave's last loads zeros, so
  // the loop needs no early exit. Before a step is read, everything but the
  // following step's NV loads has landed (loads complete in order).
  i32x4 x0[4][2], x1[4][2];
  fetch(0, 0, x0);
  for (int b = 0; b < cnt; b += 2) {
    fetch(b + 1, 1, x1);
    sk_wait_vm<NV>();
    __builtin_amdgcn_sched_barrier(0);
    mul(0, x0);
    __builtin_amdgcn_sched_barrier(0);
    fetch(b + 2, 0, x0);
    sk_wait_vm<NV>();
    __builtin_amdgcn_sched_barrier(0);
    mul(1, x1);
    __builtin_amdgcn_sched_barrier(0);
  }
  sk_wait_vm<0>();

  // waves meet in LDS; wave 0 lane l holds rows 4 g + v of channel 16 c + r
  if constexpr (W > 1) {
#pragma unroll
    for (int c = 0; c < NT; ++c) sm.red[wave][c][lane] = acc[c];
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int c = 0; c < NT; ++c)
#pragma unroll
      for (int w = 1; w < W; ++w) acc[c] += sm.red[w][c][lane];
  }
#pragma unroll
  for (int c = 0; c < NT; ++c) {
    const int64_t n = t.n0 + 16 * c + r;
    if (n >= t.N) continue;
    const float s = t.scale[n];
    const float bv = t.bias ? bf16_to_f32(t.bias[n]) : 0.0f;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t mm = t.m0 + 4 * g + v;
      if (mm < t.M) t.y[mm * t.N + n] = f32_to_bf16_rne(s * acc[c][v] + bv);
    }
  }
}

template <int TG, int MB>
constexpr int batch_steps() {
  return TG * MB <= 8 ? 2 : 1;
}

// Single-row GEMV for long rows (M = 1, K >= kW8A16ContigMinK), contiguous form.
// A workgroup owns 8 output channels and its W waves split K into W
// contiguous ranges (multiples of 16 bytes). A wave reads its range of the 8
// rows as 1 KB pieces, each one row's 1024 contiguous bytes (64 lanes x 16 B):
// on gfx950 that streams from HBM faster than the 4 rows x 256 B shape of the
// other tiles. x for the wave's range comes into registers once, as fp32 (16
// values per lane and piece), and serves all 8 rows; each weight byte is
// widened (sign-extending convert) and fused into a per-row fp32 accumulator
// (int8 x bf16 products are exact in fp32). Loads go in batches of 4 with the
// next batch in flight while one is used. The 8 rows' lane partials are summed
// by a transposing butterfly (3 exchange steps halve the values a lane carries,
// 3 more finish the sum), the waves' sums meet in LDS.
template <int W, int P, int B = 4>
__global__ __launch_bounds__(64 * W) void k_w8a16_m1c(const uint16_t *__restrict__ x, int64_t K,
                                                       const int8_t *__restrict__ q,
                                                       const float *__restrict__ scale,
                                                       const uint16_t *__restrict__ bias,
                                                       int64_t N, uint16_t *__restrict__ y) {
  constexpr int R = 8;           // channels per workgroup
  constexpr int NL = R * P;      // weight loads per wave
  constexpr int NB = (NL + B - 1) / B;
  __shared__ float red[W][R];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t n0 = (int64_t)blockIdx.x * R;
  const int64_t nrows = N - n0 < R ? N - n0 : R;
  const int64_t kw = ((K + W - 1) / W + 15) / 16 * 16;
  const int64_t k0 = wave * kw;
  const int64_t k1 = K < k0 + kw ? K : k0 + kw;
  const __amdgpu_buffer_rsrc_t rq = rsrc(q + n0 * K, (uint32_t)(nrows * K));
  const __amdgpu_buffer_rsrc_t rx = rsrc(x, (uint32_t)(2 * K));

  // piece p of this wave: lane -> k = k0 + 1024 p + 16 lane .. + 16 (zeros past k1)
  int kk[P];
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int64_t k = k0 + 1024 * p + 16 * lane;
    kk[p] = k < k1 ? (int)k : -1;
  }
  auto issue = [&](int b, i32x4 *dst) {
#pragma unroll
    for (int u = 0; u < B; ++u) {
      const int L = b * B + u;
      if (L < NL) {
        const int r = L % R, p = L / R;
        const int off = kk[p] >= 0 ? (int)((uint32_t)r * (uint32_t)K + (uint32_t)kk[p]) : OOB;
        dst[u] = __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 2);
      }
    }
  };

  i32x4 wb0[B], wb1[B];
  issue(0, wb0);
  i32x4 xr[P][2];
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int off = kk[p] >= 0 ? 2 * kk[p] : OOB;
    xr[p][0] = __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0);
    xr[p][1] = __builtin_amdgcn_raw_buffer_load_b128(rx, off >= 0 && off != OOB ? off + 16 : OOB, 0, 0);
  }
  if (NB > 1) issue(1, wb1);
  float xf[P][16];
#pragma unroll
  for (int p = 0; p < P; ++p)
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t d = (uint32_t)xr[p][h][i];
        xf[p][8 * h + 2 * i] = __uint_as_float(d << 16);
        xf[p][8 * h + 2 * i + 1] = __uint_as_float(d & 0xffff0000u);
      }

  float acc[R][2];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r][0] = acc[r][1] = 0.0f;
  auto consume = [&](int b, const i32x4 *src) {
#pragma unroll
    for (int u = 0; u < B; ++u) {
      const int L = b * B + u;
      if (L < NL) {
        const int r = L % R, p = L / R;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int wv = src[u][e];
#pragma unroll
          for (int i = 0; i < 4; ++i)
            acc[r][i & 1] = fmaf((float)(int8_t)(wv >> (8 * i)), xf[p][4 * e + i], acc[r][i & 1]);
        }
      }
    }
  };
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    __builtin_amdgcn_sched_barrier(0);
    consume(b, (b & 1) ? wb1 : wb0);
    __builtin_amdgcn_sched_barrier(0);
    if (b + 2 < NB) issue(b + 2, (b & 1) ? wb1 : wb0);
  }

  // transposing butterfly: the lane-half swaps leave rows 0-3 in the low half
  // and 4-7 in the high half (4 values each), then 2 per row pair, and a row
  // mirror 1 (the row of lane >> 3); half mirror and two quad exchanges
  // finish the sum over the 8 lanes of that row
  float v[R];
#pragma unroll
  for (int r = 0; r < R; ++r) v[r] = acc[r][0] + acc[r][1];
  float t4[4], t2[2];
#pragma unroll
  for (int j = 0; j < 4; ++j) t4[j] = swap32_sum(v[j], v[4 + j]);
#pragma unroll
  for (int j = 0; j < 2; ++j) t2[j] = swap16_sum(t4[j], t4[2 + j]);
  const bool h3 = lane & 8;
  float sum = (h3 ? t2[1] : t2[0]) + dpp_f32<kDppRowMirror>(h3 ? t2[0] : t2[1]);
  sum += dpp_f32<kDppRowHalfMirror>(sum);
  sum += dpp_f32<kDppQuadXor2>(sum);
  sum += dpp_f32<kDppQuadXor1>(sum);
  if constexpr (W > 1) {
    if ((lane & 7) == 0) red[wave][lane >> 3] = sum;
    __syncthreads();
    if (wave != 0 || lane >= R) return;
    sum = red[0][lane];
#pragma unroll
    for (int w = 1; w < W; ++w) sum += red[w][lane];
  } else {
    if ((lane & 7) != 0) return;
  }
  const int row = W > 1 ? lane : lane >> 3;
  const int64_t n = n0 + row;
  if (n >= N) return;
  const float bv = bias ? bf16_to_f32(bias[n]) : 0.0f;
  y[n] = f32_to_bf16_rne(scale[n] * sum + bv);
}

// Grouped single-row GEMVs in the contiguous form of k_w8a16_m1c (1 KB row
// pieces, lane l reading bytes 16 l .. 16 l + 15 of a piece). A workgroup has
// 4 waves. For a problem with K <= 1024 each wave takes its own 8 channels and
// their whole rows, one piece each (the lanes past K read nothing); for
// 1024 < K <= 4096 the workgroup takes 8 channels and wave w piece w of each
// row (a wave past the last piece idles), the waves' sums meeting in LDS.
// Every row is read once and no byte past its end, where the 4 rows x 256 B
// steps of the single-row tile over-read rows whose length is not a multiple
// of 256. x comes straight from memory (the waves of a workgroup read the
// same bytes of it, which the L1 serves) into fp32 registers.
template <int B>
__device__ __forceinline__ void m1p_body(const W8A16GroupEntry &e, int local) {
  constexpr int W = 4, R = 8, NB = (R + B - 1) / B;
  __shared__ float red[W][R];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t K = e.K, N = e.N;
  const bool split = K > 1024;  // uniform
  const int64_t n0 = split ? (int64_t)local * R : ((int64_t)local * W + wave) * R;
  const int64_t k0 = split ? 1024LL * wave : 0;
  const int64_t rem = N - n0;
  const int64_t nrows = rem <= 0 ? 0 : (rem < R ? rem : R);
  const bool active = nrows > 0 && k0 < K;  // uniform
  const __amdgpu_buffer_rsrc_t rq = rsrc(nrows > 0 ? e.q + n0 * K : e.q, (uint32_t)(nrows * K));
  const __amdgpu_buffer_rsrc_t rx = rsrc(e.x, (uint32_t)(2 * K));
  const int64_t kl = k0 + 16 * lane;
  const int kk = kl < K ? (int)kl : -1;

  float acc[R][2];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r][0] = acc[r][1] = 0.0f;
  if (active) {
    auto issue = [&](int b, i32x4 *dst) {
#pragma unroll
      for (int u = 0; u < B; ++u) {
        const int r = b * B + u;
        if (r < R) {
          const int off = kk >= 0 ? (int)((uint32_t)r * (uint32_t)K + (uint32_t)kk) : OOB;
          dst[u] = __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 2);
        }
      }
    };
    i32x4 wb0[B], wb1[B];
    issue(0, wb0);
    const int xo = kk >= 0 ? 2 * kk : OOB;
    const i32x4 xr0 = __builtin_amdgcn_raw_buffer_load_b128(rx, xo, 0, 0);
    const i32x4 xr1 = __builtin_amdgcn_raw_buffer_load_b128(rx, kk >= 0 ? xo + 16 : OOB, 0, 0);
    if (NB > 1) issue(1, wb1);
    float xf[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      xf[2 * i] = __uint_as_float((uint32_t)xr0[i] << 16);
      xf[2 * i + 1] = __uint_as_float((uint32_t)xr0[i] & 0xffff0000u);
      xf[8 + 2 * i] = __uint_as_float((uint32_t)xr1[i] << 16);
      xf[8 + 2 * i + 1] = __uint_as_float((uint32_t)xr1[i] & 0xffff0000u);
    }
    auto consume = [&](int b, const i32x4 *src) {
#pragma unroll
      for (int u = 0; u < B; ++u) {
        const int r = b * B + u;
        if (r < R) {
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int wv = src[u][c];
#pragma unroll
            for (int i = 0; i < 4; ++i)
              acc[r][i & 1] = fmaf((float)(int8_t)(wv >> (8 * i)), xf[4 * c + i], acc[r][i & 1]);
          }
        }
      }
    };
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      __builtin_amdgcn_sched_barrier(0);
      consume(b, (b & 1) ? wb1 : wb0);
      __builtin_amdgcn_sched_barrier(0);
      if (b + 2 < NB) issue(b + 2, (b & 1) ? wb1 : wb0);
    }
  }

  // the transposing butterfly of k_w8a16_m1c: lane l ends with the sum of row l >> 3
  float v[R];
#pragma unroll
  for (int r = 0; r < R; ++r) v[r] = acc[r][0] + acc[r][1];
  float t4[4], t2[2];
#pragma unroll
  for (int j = 0; j < 4; ++j) t4[j] = swap32_sum(v[j], v[4 + j]);
#pragma unroll
  for (int j = 0; j < 2; ++j) t2[j] = swap16_sum(t4[j], t4[2 + j]);
  const bool h3 = lane & 8;
  float sum = (h3 ? t2[1] : t2[0]) + dpp_f32<kDppRowMirror>(h3 ? t2[0] : t2[1]);
  sum += dpp_f32<kDppRowHalfMirror>(sum);
  sum += dpp_f32<kDppQuadXor2>(sum);
  sum += dpp_f32<kDppQuadXor1>(sum);
  int row;
  if (split) {
    if ((lane & 7) == 0) red[wave][lane >> 3] = sum;
    __syncthreads();
    if (wave != 0 || lane >= R) return;
    sum = red[0][lane];
#pragma unroll
    for (int w = 1; w < W; ++w) sum += red[w][lane];
    row = lane;
  } else {
    if ((lane & 7) != 0) return;
    row = lane >> 3;
  }
  const int64_t n = n0 + row;
  if (n >= N) return;
  const float bv = e.bias ? bf16_to_f32(e.bias[n]) : 0.0f;
  e.y[n] = f32_to_bf16_rne(e.scale[n] * sum + bv);
}

template <int B>
__global__ __launch_bounds__(256) void k_w8a16_m1p_grouped(const W8A16GroupEntry *__restrict__ tab,
                                                           int count) {
  const int blk = blockIdx.x;
  int lo = 0, hi = count - 1;
  while (lo < hi) {  // last entry with begin <= blk
    const int mid = (lo + hi + 1) >> 1;
    if (tab[mid].blk_begin <= blk) lo = mid;
    else hi = mid - 1;
  }
  const W8A16GroupEntry &e = tab[lo];
  m1p_body<B>(e, blk - e.blk_begin);
}

// The same for a group of at most kW8A16InlineMax problems whose entries come
// by value in the kernel arguments: the workgroup picks its entry with uniform
// selects and issues its weight loads without first reading a table from
// memory (two dependent round trips that a launch of a few MB, as in a decode
// step whose launches wait on each other, would otherwise pay before its
// weight stream starts).
template <int B, int NI>
__global__ __launch_bounds__(256) void k_w8a16_m1p_inline(W8A16InlineGroup g) {
  const int blk = blockIdx.x;
  W8A16GroupEntry e = g.e[0];
#pragma unroll
  for (int i = 1; i < NI; ++i)
    if (g.e[i].blk_begin <= blk) e = g.e[i];
  m1p_body<B>(e, blk - e.blk_begin);
}

// A few rows of x (2 <= M <= 4), contiguous form: the pieces and the wave
// split of k_w8a16_m1c, with MR rows of x in registers as bf16 pairs and each
// weight dword widened once (exact) and multiplied into the MR rows by
// v_dot2_f32_bf16 (two products, fp32 accumulate). The R x MR lane partials
// (R = 8 channels) go through the same kind of transposing butterfly.
// a.lo * b.lo + a.hi * b.hi + c (bf16 pairs, fp32 accumulate), in the
// three-operand VOP3P form: chains of the two-operand accumulate form that
// the compiler picks for the builtin (v_dot2c_f32_bf16) gave wrong sums here.
__device__ __forceinline__ float dot2_bf16(int a, int b, float c) {
  float d;
  asm volatile("v_dot2_f32_bf16 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "v"(c));
  return d;
}
template <int W, int P, int MR>
__global__ __launch_bounds__(64 * W) void k_w8a16_mfew(const uint16_t *__restrict__ x, int64_t M,
                                                        int64_t K, const int8_t *__restrict__ q,
                                                        const float *__restrict__ scale,
                                                        const uint16_t *__restrict__ bias,
                                                        int64_t N, uint16_t *__restrict__ y) {
  constexpr int R = 8;           // channels per workgroup
  constexpr int NL = R * P;      // weight loads per wave
  constexpr int B = 4;           // loads per batch
  constexpr int NB = (NL + B - 1) / B;
  constexpr int V = R * MR;      // partial sums per lane
  static_assert(V == 16 || V == 32, "MR in {2, 4}");
  __shared__ float red[W][V];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t n0 = (int64_t)blockIdx.x * R;
  const int64_t nrows = N - n0 < R ? N - n0 : R;
  const int64_t kw = ((K + W - 1) / W + 15) / 16 * 16;
  const int64_t k0 = wave * kw;
  const int64_t k1 = K < k0 + kw ? K : k0 + kw;
  const __amdgpu_buffer_rsrc_t rq = rsrc(q + n0 * K, (uint32_t)(nrows * K));
  const __amdgpu_buffer_rsrc_t rx = rsrc(x, (uint32_t)(2 * K * M));

  int kk[P];
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int64_t k = k0 + 1024 * p + 16 * lane;
    kk[p] = k < k1 ? (int)k : -1;
  }
  auto issue = [&](int b, i32x4 *dst) {
#pragma unroll
    for (int u = 0; u < B; ++u) {
      const int L = b * B + u;
      if (L < NL) {
        const int r = L % R, p = L / R;
        const int off = kk[p] >= 0 ? (int)((uint32_t)r * (uint32_t)K + (uint32_t)kk[p]) : OOB;
        dst[u] = __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 2);
      }
    }
  };

  i32x4 wb0[B], wb1[B];
  issue(0, wb0);
  i32x4 xr[P][MR][2];  // bf16 pairs: 16 values per lane, piece and row (rows past M: zero)
#pragma unroll
  for (int p = 0; p < P; ++p)
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      const bool in = kk[p] >= 0 && m < M;
      const int off = in ? 2 * (m * (int)K + kk[p]) : OOB;
      xr[p][m][0] = __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0);
      xr[p][m][1] = __builtin_amdgcn_raw_buffer_load_b128(rx, in ? off + 16 : OOB, 0, 0);
    }
  if (NB > 1) issue(1, wb1);

  float acc[R][MR];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < MR; ++m) acc[r][m] = 0.0f;
  auto consume = [&](int b, const i32x4 *src) {
#pragma unroll
    for (int u = 0; u < B; ++u) {
      const int L = b * B + u;
      if (L < NL) {
        const int r = L % R, p = L / R;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // weights k = 4e .. 4e + 3 of the lane's 16, as two bf16 pairs
          const i32x2 w2 = __builtin_bit_cast(i32x2, widen4(src[u][e]));
#pragma unroll
          for (int m = 0; m < MR; ++m) {
            const i32x4 xv = xr[p][m][e >> 1];
            const int xa = xv[2 * (e & 1)], xb = xv[2 * (e & 1) + 1];
            acc[r][m] = dot2_bf16(xa, w2[0], acc[r][m]);
            acc[r][m] = dot2_bf16(xb, w2[1], acc[r][m]);
          }
        }
      }
    }
  };
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    __builtin_amdgcn_sched_barrier(0);
    consume(b, (b & 1) ? wb1 : wb0);
    __builtin_amdgcn_sched_barrier(0);
    if (b + 2 < NB) issue(b + 2, (b & 1) ? wb1 : wb0);
  }

  // transposing butterfly over lane bits 5, 4, 3, 2 (and 1 for V = 32), then
  // plain sums; lane l ends with value index l >> (6 - log2 V)
  constexpr int LV = V == 16 ? 4 : 5;
  float t[V];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < MR; ++m) t[MR * r + m] = acc[r][m];
#pragma unroll
  for (int j = 0; j < V / 2; ++j) t[j] = swap32_sum(t[j], t[V / 2 + j]);
#pragma unroll
  for (int j = 0; j < V / 4; ++j) t[j] = swap16_sum(t[j], t[V / 4 + j]);
  const bool b3 = lane & 8, b2 = lane & 4, b1 = lane & 2;
#pragma unroll
  for (int j = 0; j < V / 8; ++j) {
    const float keep = b3 ? t[V / 8 + j] : t[j], send = b3 ? t[j] : t[V / 8 + j];
    t[j] = keep + dpp_f32<kDppRowMirror>(send);
  }
#pragma unroll
  for (int j = 0; j < V / 16; ++j) {
    const float keep = b2 ? t[V / 16 + j] : t[j], send = b2 ? t[j] : t[V / 16 + j];
    t[j] = keep + dpp_f32<kDppRowHalfMirror>(send);
  }
  float sum;
  if constexpr (LV == 4) {
    sum = t[0] + dpp_f32<kDppQuadXor2>(t[0]);
  } else {
    const float keep = b1 ? t[1] : t[0], send = b1 ? t[0] : t[1];
    sum = keep + dpp_f32<kDppQuadXor2>(send);
  }
  sum += dpp_f32<kDppQuadXor1>(sum);
  const int idx = lane >> (6 - LV);  // = MR r + m
  const bool lead = (lane & ((64 >> LV) - 1)) == 0;
  if constexpr (W > 1) {
    if (lead) red[wave][idx] = sum;
    __syncthreads();
    if (wave != 0 || lane >= V) return;
    sum = red[0][lane];
#pragma unroll
    for (int w = 1; w < W; ++w) sum += red[w][lane];
    const int r = lane / MR, m = lane % MR;
    const int64_t n = n0 + r;
    if (m >= M || n >= N) return;
    const float bv = bias ? bf16_to_f32(bias[n]) : 0.0f;
    y[m * N + n] = f32_to_bf16_rne(scale[n] * sum + bv);
  } else {
    if (!lead) return;
    const int r = idx / MR, m = idx % MR;
    const int64_t n = n0 + r;
    if (m >= M || n >= N) return;
    const float bv = bias ? bf16_to_f32(bias[n]) : 0.0f;
    y[m * N + n] = f32_to_bf16_rne(scale[n] * sum + bv);
  }
}

constexpr int M1_TG = 2;  // single-row tile: 8 channels per wave tile
constexpr int M1_U = 2;   // steps per fetched batch

// Grouped launch: blocks [begin, begin + nblk * mblk) of the grid belong to
// problem p, n-block fastest. The table is read through the scalar cache.
__device__ __forceinline__ Tile group_tile(const W8A16GroupEntry *__restrict__ tab, int count,
                                           int64_t rows) {
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
  return Tile{e.x, e.q, e.scale, e.bias, e.y, e.M, e.N, e.K, (int64_t)nb * rows, (int64_t)mb * 16};
}

template <int W, int TG, int MB>
__global__ __launch_bounds__(64 * W) void k_w8a16(const uint16_t *__restrict__ x, int64_t M,
                                                  int64_t K, const int8_t *__restrict__ q,
                                                  const float *__restrict__ scale,
                                                  const uint16_t *__restrict__ bias, int64_t N,
                                                  uint16_t *__restrict__ y) {
  __shared__ Red<W, TG, MB> red;
  const Tile t{x, q, scale, bias, y, M, N, K, (int64_t)blockIdx.x * 4 * TG,
               (int64_t)blockIdx.y * 16};
  w8a16_tile<W, TG, MB, batch_steps<TG, MB>()>(t, red);
}

template <int W, int TG, int MB>
__global__ __launch_bounds__(64 * W) void k_w8a16_grouped(const W8A16GroupEntry *__restrict__ tab,
                                                          int count) {
  __shared__ Red<W, TG, MB> red;
  w8a16_tile<W, TG, MB, batch_steps<TG, MB>()>(group_tile(tab, count, 4 * TG), red);
}

// Skinny tile (M <= 16): 16 NT channels x 16 rows per workgroup of W waves.
template <int W, int NT>
__global__ __launch_bounds__(64 * W) void k_w8a16_sk(const uint16_t *__restrict__ x, int64_t M,
                                                     int64_t K, const int8_t *__restrict__ q,
                                                     const float *__restrict__ scale,
                                                     const uint16_t *__restrict__ bias, int64_t N,
                                                     uint16_t *__restrict__ y) {
  __shared__ __attribute__((aligned(16))) SkLds<W, NT> sm;
  const Tile t{x, q, scale, bias, y, M, N, K, (int64_t)blockIdx.x * 16 * NT,
               (int64_t)blockIdx.y * 16};
  w8a16_tile_sk<W, NT>(t, sm);
}

template <int W, int NT>
__global__ __launch_bounds__(64 * W) void k_w8a16_sk_grouped(const W8A16GroupEntry *__restrict__ tab,
                                                             int count) {
  __shared__ __attribute__((aligned(16))) SkLds<W, NT> sm;
  w8a16_tile_sk<W, NT>(group_tile(tab, count, 16 * NT), sm);
}

// Skinny tile with x shared through LDS (row blocks of 16, N >= kW8A16ShareMinN).
// The WC waves of one of the workgroup's WK K ranges take 16 channels each over
// the same steps, so a 256-k step of x (16 rows x 512 B) comes from L2 once per
// WC waves instead of once per wave (with 16-channel tiles the x reads of the
// skinny tile above are twice its weight bytes). Each wave of a range copies
// 8 / WC of the step's 1 KB pieces into the range's LDS slot by buffer loads
// that write LDS, row r's 16-byte chunk c at slot c ^ r (16 rows' chunk c then
// lie in 16 distinct bank groups); the waves meet at a workgroup barrier once
// the step has landed and again before its slot is refilled. Weights arrive as
// in the skinny tile (4 rows x 256 B per load into per-wave slots), and the k
// order within a step is the same. The K ranges' sums meet in LDS.
template <int WC, int WK>
struct ShLds {
  uint8_t w[WC * WK][2][16 * 256];  // per wave, two step slots of 16 rows x 256 B
  uint8_t x[WK][2][16 * 512];       // per K range, two step slots of 16 rows x 512 B
  f32x4 red[WC * WK][64];
};

// part == nullptr: the whole K, y written. Else split blockIdx.z takes steps
// [z spl, (z + 1) spl) and writes its unscaled sums to part[z][M][N] (fp32).
template <int WC, int WK>
__global__ __launch_bounds__(64 * WC * WK) void k_w8a16_sksh(const uint16_t *__restrict__ x, int64_t M,
                                                             int64_t K, const int8_t *__restrict__ q,
                                                             const float *__restrict__ scale,
                                                             const uint16_t *__restrict__ bias,
                                                             int64_t N, uint16_t *__restrict__ y,
                                                             float *__restrict__ part, int spl) {
  static_assert(8 % WC == 0, "x pieces split over a range's waves");
  __shared__ __attribute__((aligned(16))) ShLds<WC, WK> sm;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wc = wave % WC, wk = wave / WC;
  const int r = lane & 15, g = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * (16 * WC) + 16 * wc;
  const int64_t m0 = (int64_t)blockIdx.y * 16;
  const int64_t nrows = N - n0 <= 0 ? 0 : (N - n0 < 16 ? N - n0 : 16);
  const int64_t mrows = M - m0 < 16 ? M - m0 : 16;
  const __amdgpu_buffer_rsrc_t rq = rsrc(nrows > 0 ? q + n0 * K : q, (uint32_t)(nrows * K));
  const __amdgpu_buffer_rsrc_t rx = rsrc(x + m0 * K, (uint32_t)(mrows * K * 2));
  const int nst = (int)((K + 255) >> 8);
  const int s0 = part ? (int)blockIdx.z * spl : 0;
  const int s1 = part ? (s0 + spl < nst ? s0 + spl : nst) : nst;
  // range wk takes steps s0 + wk, s0 + wk + WK, ...; every wave runs the same
  // number of steps (for the barriers), steps past its range load zeros
  const int cnt = (s1 - s0 + WK - 1) / WK;
  const int drow = lane >> 4, dslot = lane & 15;
  const uint32_t lw0 = (uint32_t)(uintptr_t)&sm.w[wave][0][0];
  const uint32_t lx0 = (uint32_t)(uintptr_t)&sm.x[wk][0][0];

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  constexpr int XP = 8 / WC;  // x pieces a wave copies per step
  constexpr int NV = 4 + XP;  // vector memory instructions per step and wave
  auto fetch = [&](int i, int slot) {
    const int st = s0 + wk + WK * i;
    const bool valid = st < s1;  // uniform
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const int row = 4 * d + drow;
      const int c = dslot ^ row;
      const bool kin = valid && (256 * st + 16 * c) < K;
      const int qo = kin ? (int)((uint32_t)row * (uint32_t)K + 256u * st + 16u * c) : OOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rq, (lds_void *)(uintptr_t)__builtin_amdgcn_readfirstlane(lw0 + (uint32_t)slot * 4096u + 1024u * d),
          16, qo, 0, 0, 0);
    }
    // piece p holds x rows 2 p and 2 p + 1: lane l writes row 2 p + l / 32, slot l % 32
#pragma unroll
    for (int u = 0; u < XP; ++u) {
      const int p = wc * XP + u;
      const int row = 2 * p + (lane >> 5), c = (lane & 31) ^ row;
      const bool kin = valid && row < mrows && (256 * st + 8 * c) < K;
      const int xo = kin ? (int)((uint32_t)row * (uint32_t)(2 * K) + 512u * st + 16u * c) : OOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rx, (lds_void *)(uintptr_t)__builtin_amdgcn_readfirstlane(lx0 + (uint32_t)slot * 8192u + 1024u * p),
          16, xo, 0, 0, 0);
    }
  };
  auto mul = [&](int slot) {
    const uint8_t *wl = &sm.w[wave][slot][0];
    const uint8_t *xl = &sm.x[wk][slot][0];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const i32x4 wq = *reinterpret_cast<const i32x4 *>(wl + 256 * r + 16 * ((4 * h + g) ^ r));
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        // row r, k = 64 h + 16 g + 8 half .. + 7: x chunk 8 h + 2 g + half
        const int cx = 8 * h + 2 * g + half;
        const bf16x8 a = *reinterpret_cast<const bf16x8 *>(xl + 512 * r + 16 * (cx ^ r));
        const s16x4 lo = widen4(wq[2 * half]), hi = widen4(wq[2 * half + 1]);
        const i32x2 l2 = __builtin_bit_cast(i32x2, lo), h2 = __builtin_bit_cast(i32x2, hi);
        const bf16x8 b = __builtin_bit_cast(bf16x8, i32x4{l2[0], l2[1], h2[0], h2[1]});
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
      }
    }
  };

  // Step b's loads are out when it starts: wait until only the next step's
  // remain (this wave's parts of step b have landed), meet the other waves
  // (theirs too), multiply, then meet again once every wave has read the slot
  // before it is refilled.
  fetch(0, 0);
  for (int b = 0; b < cnt; b += 2) {
    fetch(b + 1, 1);
    sk_wait_vm<NV>();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    mul(0);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // this wave's LDS reads done
    __builtin_amdgcn_s_barrier();
    fetch(b + 2, 0);
    sk_wait_vm<NV>();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    mul(1);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_s_barrier();
  }
  sk_wait_vm<0>();

  // the ranges' sums meet in LDS (added in the order of the range);
  // lane l of wave (0, wc) holds rows 4 g + v of channel n0 + r
  if constexpr (WK > 1) {
    sm.red[wave][lane] = acc;
    __syncthreads();
    if (wk != 0) return;
#pragma unroll
    for (int k = 1; k < WK; ++k) acc += sm.red[k * WC + wc][lane];
  }
  const int64_t n = n0 + r;
  if (n >= N) return;
  if (part) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t mm = m0 + 4 * g + v;
      if (mm < M) part[((int64_t)blockIdx.z * M + mm) * N + n] = acc[v];
    }
    return;
  }
  const float s = scale[n];
  const float bv = bias ? bf16_to_f32(bias[n]) : 0.0f;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int64_t mm = m0 + 4 * g + v;
    if (mm < M) y[mm * N + n] = f32_to_bf16_rne(s * acc[v] + bv);
  }
}

// Single-row tile; dynamic LDS holds x when XL.
template <int W, int CW, bool XL>
__global__ __launch_bounds__(64 * W * CW, 4) void k_w8a16_m1(const uint16_t *__restrict__ x,
                                                          int64_t K,
                                                          const int8_t *__restrict__ q,
                                                          const float *__restrict__ scale,
                                                          const uint16_t *__restrict__ bias,
                                                          int64_t N, uint16_t *__restrict__ y) {
  __shared__ Red<W * CW, M1_TG, 0> red;
  extern __shared__ __attribute__((aligned(16))) uint8_t xs[];
  const Tile t{x, q, scale, bias, y, 1, N, K, (int64_t)blockIdx.x * 4 * M1_TG * CW, 0};
  w8a16_tile_m1<W, CW, M1_TG, M1_U, XL>(t, red, xs);
}

template <int W, int CW, bool XL>
__global__ __launch_bounds__(64 * W * CW, 4) void k_w8a16_m1_grouped(
    const W8A16GroupEntry *__restrict__ tab, int count) {
  __shared__ Red<W * CW, M1_TG, 0> red;
  extern __shared__ __attribute__((aligned(16))) uint8_t xs[];
  w8a16_tile_m1<W, CW, M1_TG, M1_U, XL>(group_tile(tab, count, 4 * M1_TG * CW), red, xs);
}

template <int TG, int MB>
void launch_single(int W, dim3 grid, hipStream_t st, const uint16_t *x, int64_t M, int64_t K,
                   const int8_t *q, const float *scale, const uint16_t *bias, int64_t N,
                   uint16_t *y) {
  switch (W) {
#define AQL_W(w)                                                                              \
  case w:                                                                                     \
    hipLaunchKernelGGL((k_w8a16<w, TG, MB>), grid, dim3(64 * w), 0, st, x, M, K, q, scale, bias, \
                       N, y);                                                                 \
    break;
    AQL_W(16) AQL_W(8) AQL_W(4) AQL_W(2) default : AQL_W(1)
#undef AQL_W
  }
}

template <int TG, int MB>
void launch_group(int W, int blocks, hipStream_t st, const W8A16GroupEntry *tab, int count) {
  const dim3 grid((unsigned)blocks);
  switch (W) {
#define AQL_W(w)                                                                            \
  case w:                                                                                   \
    hipLaunchKernelGGL((k_w8a16_grouped<w, TG, MB>), grid, dim3(64 * w), 0, st, tab, count); \
    break;
    AQL_W(16) AQL_W(8) AQL_W(4) AQL_W(2) default : AQL_W(1)
#undef AQL_W
  }
}

template <int NT>
void launch_sk_single(int W, dim3 grid, hipStream_t st, const uint16_t *x, int64_t M, int64_t K,
                      const int8_t *q, const float *scale, const uint16_t *bias, int64_t N,
                      uint16_t *y) {
  switch (W) {
#define AQL_W(w)                                                                              \
  case w:                                                                                     \
    hipLaunchKernelGGL((k_w8a16_sk<w, NT>), grid, dim3(64 * w), 0, st, x, M, K, q, scale, bias, \
                       N, y);                                                                 \
    break;
    AQL_W(8) AQL_W(4) AQL_W(2) AQL_W(1)
#undef AQL_W
    default:  // 16 waves (32 channels would not fit the registers of 1024 threads)
      hipLaunchKernelGGL((k_w8a16_sk<NT == 1 ? 16 : 8, NT>), grid, dim3(NT == 1 ? 1024 : 512), 0,
                         st, x, M, K, q, scale, bias, N, y);
      break;
  }
}

template <int NT>
void launch_sk_group(int W, int blocks, hipStream_t st, const W8A16GroupEntry *tab, int count) {
  const dim3 grid((unsigned)blocks);
  switch (W) {
#define AQL_W(w)                                                                               \
  case w:                                                                                      \
    hipLaunchKernelGGL((k_w8a16_sk_grouped<w, NT>), grid, dim3(64 * w), 0, st, tab, count);     \
    break;
    AQL_W(8) AQL_W(4) AQL_W(2) AQL_W(1)
#undef AQL_W
    default:  // 16 waves
      hipLaunchKernelGGL((k_w8a16_sk_grouped<NT == 1 ? 16 : 8, NT>), grid,
                         dim3(NT == 1 ? 1024 : 512), 0, st, tab, count);
      break;
  }
}

template <int TG>
void launch_single_tg(int MB, int W, dim3 grid, hipStream_t st, const uint16_t *x, int64_t M,
                      int64_t K, const int8_t *q, const float *scale, const uint16_t *bias,
                      int64_t N, uint16_t *y) {
  switch (MB) {
    case 1: launch_single<TG, 1>(W, grid, st, x, M, K, q, scale, bias, N, y); break;
    case 2: launch_single<TG, 2>(W, grid, st, x, M, K, q, scale, bias, N, y); break;
    default: launch_single<TG, 4>(W, grid, st, x, M, K, q, scale, bias, N, y); break;
  }
}

template <int TG>
void launch_group_tg(int MB, int W, int blocks, hipStream_t st, const W8A16GroupEntry *tab,
                     int count) {
  switch (MB) {
    case 1: launch_group<TG, 1>(W, blocks, st, tab, count); break;
    case 2: launch_group<TG, 2>(W, blocks, st, tab, count); break;
    default: launch_group<TG, 4>(W, blocks, st, tab, count); break;
  }
}

// Single-row launches: one switch over (W, CW, XL) serves both kernels; F is
// called with the kernel's template arguments as constants.
template <typename F>
void m1_dispatch(int W, int CW, bool XL, F f) {
#define AQL_M1(w, c)                                                     \
  if (W == w && CW == c) {                                               \
    if (XL) f(std::integral_constant<int, w>{}, std::integral_constant<int, c>{}, \
              std::true_type{});                                         \
    else f(std::integral_constant<int, w>{}, std::integral_constant<int, c>{},    \
           std::false_type{});                                           \
    return;                                                              \
  }
  AQL_M1(1, 1) AQL_M1(1, 2) AQL_M1(1, 4) AQL_M1(2, 1) AQL_M1(2, 2) AQL_M1(2, 4)
  AQL_M1(4, 1) AQL_M1(4, 2) AQL_M1(4, 4) AQL_M1(8, 1) AQL_M1(8, 2)
#undef AQL_M1
}

bool m1_shape_ok(const W8A16Shape &sh) {
  const int w = sh.waves, c = sh.cgroups;
  return (w == 1 || w == 2 || w == 4 || w == 8) && (c == 1 || c == 2 || c == 4) && w * c <= 16 &&
         sh.xlds >= 0 && sh.xlds <= kW8A16MaxXlds && sh.xlds % 1024 == 0;
}

}  // namespace

// Launch shape, from a sweep of tile rows x waves on the 7B MLP shapes and the
// SmolVLM decode sweep: streaming is fastest with few waves per workgroup and
// enough wave-tiles in flight: for the single-row tile about 3000 (8-channel
// tiles; waves split K only while the tiles alone fall short; about 1000 for
// rows of 8 KiB and more, measured on K = 8192, 12288 and 14336), for larger M
// about 768 (8-channel tiles for M <= 2, 16 otherwise). The single-row tile
// reads x from LDS whenever 2 K fits the budget (one 1 KiB load per wave
// instruction instead of 512 bytes per step and wave), and pairs wave tiles in
// a workgroup only when the grid is large: sharing x then saves L2 reads, while
// on smaller grids the halved workgroup count costs more than it saves.
W8A16Shape w8a16_shape(int64_t M, int64_t N, int64_t K) {
  W8A16Shape s;
  const int64_t nst = (K + 255) / 256;  // 256-byte K steps
  if (M >= kW8A16SkinnyMinM) {
    // skinny tile: 16 rows x 16 NT channels on 16x16x32 MFMAs
    s.mblocks = kW8A16Skinny;
    s.tgroups = N >= 8192 ? 8 : 4;
    const int64_t tiles = ((N + 4 * s.tgroups - 1) / (4 * s.tgroups)) * ((M + 15) / 16);
    int W = 1;
    // waves split K while the grid holds fewer than ~1024 wave tiles and each
    // wave keeps at least 8 steps (shorter loops pay their fill and drain)
    const int wmax = s.tgroups == 8 ? 8 : 16;  // 1024 threads leave too few registers for 32 channels
    while (W < wmax && tiles * W < 1024 && 16 * W <= nst) W <<= 1;
    s.waves = W;
    return s;
  }
  s.mblocks = M == 1 ? 0 : (M <= 4 ? 1 : (M <= 8 ? 2 : 4));
  s.tgroups = M <= 2 ? 2 : 4;
  const int64_t tiles = ((N + 4 * s.tgroups - 1) / (4 * s.tgroups)) * ((M + 15) / 16);
  // long rows (K >= 8 KiB) stream best from fewer, longer waves (~1024 wave
  // tiles), with two wave tiles sharing a workgroup's copy of x once waves
  // split K
  const bool long_k = M == 1 && nst >= 32;
  const int64_t want = M == 1 ? (long_k ? 1024 : 3072) : 768;
  const int wmax = M == 1 ? 8 : 16;
  int W = 1;
  while (W < wmax && tiles * W < want && W * (M == 1 ? 2 : 4) <= nst) W <<= 1;
  s.waves = W;
  if (M == 1) {
    s.cgroups = long_k ? (W >= 2 ? 2 : 1) : (tiles * W >= 8192 ? 2 : 1);
    s.xlds = w8a16_xlds_bytes(K);
  }
  return s;
}

int w8a16_xlds_bytes(int64_t K) {
  const int64_t b = (2 * K + 1023) / 1024 * 1024;
  return b <= kW8A16MaxXlds ? (int)b : 0;
}

hipError_t launch_w8a16_shape(const W8A16Shape &sh, const uint16_t *x, int64_t M, int64_t K,
                              const int8_t *q, const float *scale, const uint16_t *bias,
                              int64_t N, uint16_t *y, hipStream_t st) {
  if (sh.mblocks == 0) {
    if (M != 1 || !m1_shape_ok(sh) || (sh.xlds && sh.xlds < 2 * K)) return hipErrorInvalidValue;
    const int64_t rows = 4 * M1_TG * sh.cgroups;
    const dim3 grid((unsigned)((N + rows - 1) / rows)), block(64 * sh.waves * sh.cgroups);
    m1_dispatch(sh.waves, sh.cgroups, sh.xlds > 0, [&](auto w, auto c, auto xl) {
      hipLaunchKernelGGL((k_w8a16_m1<decltype(w)::value, decltype(c)::value, decltype(xl)::value>),
                         grid, block, sh.xlds, st, x, K, q, scale, bias, N, y);
    });
    return hipGetLastError();
  }
  const int64_t rows = 4 * sh.tgroups;
  const dim3 grid((unsigned)((N + rows - 1) / rows), (unsigned)((M + 15) / 16));
  if (sh.mblocks == kW8A16Skinny) {
    if (sh.tgroups == 8) launch_sk_single<2>(sh.waves, grid, st, x, M, K, q, scale, bias, N, y);
    else launch_sk_single<1>(sh.waves, grid, st, x, M, K, q, scale, bias, N, y);
    return hipGetLastError();
  }
  switch (sh.tgroups) {
    case 1: launch_single_tg<1>(sh.mblocks, sh.waves, grid, st, x, M, K, q, scale, bias, N, y); break;
    case 2: launch_single_tg<2>(sh.mblocks, sh.waves, grid, st, x, M, K, q, scale, bias, N, y); break;
    default: launch_single_tg<4>(sh.mblocks, sh.waves, grid, st, x, M, K, q, scale, bias, N, y); break;
  }
  return hipGetLastError();
}

hipError_t launch_w8a16_m1c(const uint16_t *x, int64_t K, const int8_t *q, const float *scale,
                            const uint16_t *bias, int64_t N, uint16_t *y, hipStream_t st) {
  if (K < kW8A16ContigMinK || K > kW8A16ContigMaxK || K % 16) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((N + 7) / 8));
  // 4 waves split K, each with one or two pieces of 1 KB per row; one piece
  // per row is consumed in batches of 2 loads (K = 4096, N = 14336: 10.66 us
  // against 10.81 with batches of 4; a single launch of the read-only probe
  // over the same 58.7 MB takes 10.39 us). A grid of at most one workgroup a
  // CU is bound by latency, not by the stream: its 8 loads go out at once.
  if (K <= 4096 && grid.x <= 256)
    hipLaunchKernelGGL((k_w8a16_m1c<4, 1, 8>), grid, dim3(256), 0, st, x, K, q, scale, bias, N, y);
  else if (K <= 4096)
    hipLaunchKernelGGL((k_w8a16_m1c<4, 1, 2>), grid, dim3(256), 0, st, x, K, q, scale, bias, N, y);
  else
    hipLaunchKernelGGL((k_w8a16_m1c<4, 2>), grid, dim3(256), 0, st, x, K, q, scale, bias, N, y);
  return hipGetLastError();
}

hipError_t launch_w8a16_m1p_grouped(const W8A16GroupEntry *dev_tab, const W8A16GroupEntry *host_tab,
                                    int count, int total_blocks, hipStream_t st) {
  if (host_tab && count >= 1 && count <= kW8A16InlineMax) {
    W8A16InlineGroup g = {};
    for (int i = 0; i < count; ++i) g.e[i] = host_tab[i];
    switch (count) {
      case 1: hipLaunchKernelGGL((k_w8a16_m1p_inline<4, 1>), dim3((unsigned)total_blocks), dim3(256), 0, st, g); break;
      case 2: hipLaunchKernelGGL((k_w8a16_m1p_inline<4, 2>), dim3((unsigned)total_blocks), dim3(256), 0, st, g); break;
      case 3: hipLaunchKernelGGL((k_w8a16_m1p_inline<4, 3>), dim3((unsigned)total_blocks), dim3(256), 0, st, g); break;
      default: hipLaunchKernelGGL((k_w8a16_m1p_inline<4, 4>), dim3((unsigned)total_blocks), dim3(256), 0, st, g); break;
    }
    return hipGetLastError();
  }
  hipLaunchKernelGGL((k_w8a16_m1p_grouped<4>), dim3((unsigned)total_blocks), dim3(256), 0, st,
                     dev_tab, count);
  return hipGetLastError();
}

hipError_t launch_w8a16_mfew(const uint16_t *x, int64_t M, int64_t K, const int8_t *q,
                             const float *scale, const uint16_t *bias, int64_t N, uint16_t *y,
                             hipStream_t st) {
  if (M < 2 || M > kW8A16FewMaxM || K < kW8A16FewMinK || K > kW8A16FewMaxK || K % 16)
    return hipErrorInvalidValue;
  const dim3 grid((unsigned)((N + 7) / 8));
  auto go = [&](auto kern, int W) {
    hipLaunchKernelGGL(kern, grid, dim3(64 * W), 0, st, x, M, K, q, scale, bias, N, y);
  };
  // waves split K so that each keeps one or two pieces of 1 KB per row
  if (M == 2) {
    if (K <= 4096) go(k_w8a16_mfew<4, 1, 2>, 4);
    else if (K <= 8192) go(k_w8a16_mfew<4, 2, 2>, 4);
    else go(k_w8a16_mfew<8, 2, 2>, 8);
  } else {
    if (K <= 4096) go(k_w8a16_mfew<4, 1, 4>, 4);
    else if (K <= 8192) go(k_w8a16_mfew<4, 2, 4>, 4);
    else go(k_w8a16_mfew<8, 2, 4>, 8);
  }
  return hipGetLastError();
}

int w8a16_skinny_splits(int64_t M, int64_t N, int64_t K) {
  if (M < 12 || M >= 64 || N >= kW8A16ShareMinN || K < 8192) return 1;
  const int64_t tiles = ((N + 63) / 64) * ((M + 15) / 16);
  return tiles <= 128 ? 4 : tiles <= 256 ? 2 : 1;
}

size_t w8a16_skinny_part_bytes(int64_t M, int64_t N, int64_t K) {
  const int S = w8a16_skinny_splits(M, N, K);
  return S > 1 ? (size_t)S * (size_t)M * (size_t)N * 4 : 0;
}

hipError_t launch_w8a16(const uint16_t *x, int64_t M, int64_t K, const int8_t *q,
                        const float *scale, const uint16_t *bias, int64_t N, uint16_t *y,
                        float *part, size_t part_bytes, hipStream_t st) {
  if (M == 1 && K >= kW8A16ContigMinK && K <= kW8A16ContigMaxK)
    return launch_w8a16_m1c(x, K, q, scale, bias, N, y, st);
  if (M >= 2 && M <= kW8A16FewMaxM && K >= kW8A16FewMinK && K <= kW8A16FewMaxK)
    return launch_w8a16_mfew(x, M, K, q, scale, bias, N, y, st);
  if (M >= kW8A16SkinnyMinM && N >= kW8A16ShareMinN) {
    // 64 channels a workgroup; one K range for rows of up to 4 KiB once there
    // are 192 workgroups a row block, else two (M = 16: K = 4096, N = 14336:
    // 14.2 us against 17.8 for the skinny tile; N = 11008: 13.0 vs 17.0;
    // K = N = 8192: 20.0 vs 22.4)
    const dim3 grid((unsigned)((N + 63) / 64), (unsigned)((M + 15) / 16));
    if (N >= 12288 && K <= 4096)
      hipLaunchKernelGGL((k_w8a16_sksh<4, 1>), grid, dim3(256), 0, st, x, M, K, q, scale, bias, N, y, nullptr, 0);
    else
      hipLaunchKernelGGL((k_w8a16_sksh<4, 2>), grid, dim3(512), 0, st, x, M, K, q, scale, bias, N, y, nullptr, 0);
    return hipGetLastError();
  }
  const int S = w8a16_skinny_splits(M, N, K);
  if (S > 1 && part && part_bytes >= w8a16_skinny_part_bytes(M, N, K)) {
    // Fewer channels: the shared-x form over S ranges of K, each writing its
    // fp32 partial sums, then their sum (M = 16, K = 14336, N = 4096: 16.4 us
    // against 19.1 for the skinny tile; M = 32: 20.5 vs 32.3; rotated weights)
    const int nst = (int)((K + 255) / 256);
    const int spl = (nst + S - 1) / S;
    const int splits = (nst + spl - 1) / spl;
    const dim3 grid((unsigned)((N + 63) / 64), (unsigned)((M + 15) / 16), (unsigned)splits);
    hipLaunchKernelGGL((k_w8a16_sksh<4, 1>), grid, dim3(256), 0, st, x, M, K, q, scale, bias, N, y,
                       part, spl);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_w8a16_splitk_reduce(part, splits, M, N, scale, bias, y, st);
  }
  return launch_w8a16_shape(w8a16_shape(M, N, K), x, M, K, q, scale, bias, N, y, st);
}

hipError_t launch_w8a16_grouped(const W8A16GroupEntry *dev_tab, int count, int total_blocks,
                                const W8A16Shape &sh, hipStream_t st) {
  if (sh.mblocks == 0) {
    if (!m1_shape_ok(sh)) return hipErrorInvalidValue;
    const dim3 grid((unsigned)total_blocks), block(64 * sh.waves * sh.cgroups);
    m1_dispatch(sh.waves, sh.cgroups, sh.xlds > 0, [&](auto w, auto c, auto xl) {
      hipLaunchKernelGGL(
          (k_w8a16_m1_grouped<decltype(w)::value, decltype(c)::value, decltype(xl)::value>), grid,
          block, sh.xlds, st, dev_tab, count);
    });
    return hipGetLastError();
  }
  if (sh.mblocks == kW8A16Skinny) {
    if (sh.tgroups == 8) launch_sk_group<2>(sh.waves, total_blocks, st, dev_tab, count);
    else launch_sk_group<1>(sh.waves, total_blocks, st, dev_tab, count);
    return hipGetLastError();
  }
  switch (sh.tgroups) {
    case 1: launch_group_tg<1>(sh.mblocks, sh.waves, total_blocks, st, dev_tab, count); break;
    case 2: launch_group_tg<2>(sh.mblocks, sh.waves, total_blocks, st, dev_tab, count); break;
    default: launch_group_tg<4>(sh.mblocks, sh.waves, total_blocks, st, dev_tab, count); break;
  }
  return hipGetLastError();
}

}  // namespace aql
