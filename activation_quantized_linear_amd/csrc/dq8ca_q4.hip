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
// Either way every 32-k group's int32 sum is formed exactly by the matrix cores
// and folded into the fp32 accumulator with its group scale right away.
#include <float.h>

#include <type_traits>

#include "dq8ca_q4.h"

namespace aql {
namespace {

typedef __attribute__((address_space(3))) void lds_void;

constexpr int OOB = 0x40000000;  // an offset past any range: buffer loads return 0

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// s_waitcnt vmcnt(n), expcnt and lgkmcnt left at their maxima (n < 64)
constexpr int vmcnt_imm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

__device__ __forceinline__ long unpack_q4x8(uint32_t w) {
  const uint32_t even = (w << 4) & 0xF0F0F0F0u;
  const uint32_t odd = w & 0xF0F0F0F0u;
  return (long)((uint64_t)even | ((uint64_t)odd << 32));
}

// ------------------------------------------------------ streaming (M <= 16)
// Bound by streaming the packed weights and their group scales from HBM. The
// access shape follows the weight-only GEMV: a wave instruction reads 4 weight
// rows x 256 contiguous bytes, so each lane holds 16 bytes = one whole 32-k
// group of one channel (lane % 4 = row, lane / 4 = group within the step),
// plus that group's scale (4 rows x 64 contiguous bytes). The group is
// multiplied where it lands with v_mfma_i32_4x4x4_i8: block b = lane / 4 takes
// k-slices of group b for 4 channels (B column j = lane % 4) against the same
// k-slices of 4 rows of xq (A row i = lane % 4), so after 8 MFMAs lane 4b + j
// holds, for each of its 4 rows, the exact int32 group sum of its own channel.
// The group's code sum comes from the unpacked bytes themselves (8 four-byte
// dot products with ones, cheaper than streaming the stored sums), and the
// zero point and the group scale are folded in right there.
//
// Tile: TG row groups of 4 channels, MB blocks of 4 rows of x, W waves splitting
// K into 512-k steps (256 bytes of nibbles); batches of U steps ping-pong.
namespace {
template <int W, int TG, int MB>
struct Q4Red {
  f32x4 v[W][TG][MB][4];
};
}  // namespace

template <int W, int TG, int MB, int U>
__global__ __launch_bounds__(64 * W) void k_dq8ca_q4_stream(Q4Args p) {
  __shared__ Q4Red<W, TG, MB> red;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int j = lane & 3, blk = lane >> 2;
  const int64_t K = p.K, G = K / 32, KB = K / 2;  // KB: packed bytes per row
  const int64_t n0 = (int64_t)blockIdx.x * 4 * TG, m0 = (int64_t)blockIdx.y * 16;
  const int64_t nrows = p.N - n0 < 4 * TG ? p.N - n0 : 4 * TG;
  const int64_t mrows = p.M - m0 < 16 ? p.M - m0 : 16;
  const __amdgpu_buffer_rsrc_t rq = rsrc(p.q4 + n0 * KB, (uint32_t)(nrows * KB));
  const __amdgpu_buffer_rsrc_t rg = rsrc(p.gs + n0 * G, (uint32_t)(nrows * G * 4));
  const __amdgpu_buffer_rsrc_t rx = rsrc(p.xq + m0 * K, (uint32_t)(mrows * K));
  const uint32_t qlane = (uint32_t)(j * KB + 16 * blk);
  const uint32_t glane = 4u * (uint32_t)(j * G + blk);
  const uint32_t xlane = (uint32_t)(j * K + 32 * blk);
  const int nst = (int)((KB + 255) >> 8);
  const int cnt = wave < nst ? (nst - wave + W - 1) / W : 0;

  int zpn[MB][4];  // -zp per row (0 past M)
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t mm = m0 + 4 * mb + v;
      zpn[mb][v] = mm < p.M ? -p.xz[mm] : 0;
    }

  f32x4 f[TG][MB];
#pragma unroll
  for (int tg = 0; tg < TG; ++tg)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) f[tg][mb] = f32x4{0.f, 0.f, 0.f, 0.f};

  struct Batch {
    i32x4 q[U][TG];
    float gs[U][TG];
    i32x4 x[U][MB][2];
  };
  auto fetch = [&](int i0, Batch &bt) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u;
      const int st = wave + W * i;
      const bool valid = i < cnt;  // uniform
      // per lane: this lane's group lies before K (only the last step can end early)
      const bool kin = 256 * st + 16 * blk < KB;
      const uint32_t qstep = valid ? 256u * st : (uint32_t)OOB;
      const uint32_t gstep = valid ? 64u * st : (uint32_t)OOB;
      const uint32_t xstep = valid ? 512u * st : (uint32_t)OOB;
#pragma unroll
      for (int tg = 0; tg < TG; ++tg) {
        const int qo = (int)(qlane + (uint32_t)(4 * tg) * (uint32_t)KB + qstep);
        bt.q[u][tg] = __builtin_amdgcn_raw_buffer_load_b128(rq, qo, 0, 2);
        const int go = kin ? (int)(glane + 4u * (uint32_t)(4 * tg) * (uint32_t)G + gstep) : OOB;
        bt.gs[u][tg] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rg, go, 0, 2));
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int xo = kin ? (int)(xlane + (uint32_t)(4 * mb) * (uint32_t)K + xstep) : OOB;
        bt.x[u][mb][0] = __builtin_amdgcn_raw_buffer_load_b128(rx, xo, 0, 0);
        bt.x[u][mb][1] = __builtin_amdgcn_raw_buffer_load_b128(rx, xo + 16, 0, 0);
      }
    }
  };
  auto mul = [&](const Batch &bt) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int tg = 0; tg < TG; ++tg) {
        int wq[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t w = (uint32_t)bt.q[u][tg][e];
          wq[2 * e] = (int)((w << 4) & 0xF0F0F0F0u);  // even k of the 8-k block, as 16 c
          wq[2 * e + 1] = (int)(w & 0xF0F0F0F0u);     // odd k
        }
        // 16 x this lane's group sum of the codes, from the unpacked bytes: the
        // same 8 MFMAs against an all-ones A operand (every row of the result
        // holds the column sums); the matrix cores have room here, the vector
        // ALU of these few waves does not
        i32x4 ts = {0, 0, 0, 0};
#pragma unroll
        for (int d = 0; d < 8; ++d) ts = __builtin_amdgcn_mfma_i32_4x4x4i8(0x01010101, wq[d], ts, 0, 0, 0);
        const int gm16 = ts[0];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          i32x4 t = {0, 0, 0, 0};
#pragma unroll
          for (int d = 0; d < 8; ++d)
            t = __builtin_amdgcn_mfma_i32_4x4x4i8(bt.x[u][mb][d >> 2][d & 3], wq[d], t, 0, 0, 0);
#pragma unroll
          for (int v = 0; v < 4; ++v)  // |zp| <= 128, |gm16| <= 4096: 24-bit product
            f[tg][mb][v] += bt.gs[u][tg] * (float)(t[v] + __mul24(zpn[mb][v], gm16));
        }
      }
  };

  Batch b0, b1;
  fetch(0, b0);
  for (int b = 0; b < cnt; b += 2 * U) {
    fetch(b + U, b1);
    __builtin_amdgcn_sched_barrier(0);
    mul(b0);
    __builtin_amdgcn_sched_barrier(0);
    fetch(b + 2 * U, b0);
    __builtin_amdgcn_sched_barrier(0);
    mul(b1);
    __builtin_amdgcn_sched_barrier(0);
  }

  // Sum over the 16 groups of a step: lanes j, j + 4, ..., j + 60.
#pragma unroll
  for (int tg = 0; tg < TG; ++tg)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int o = 4; o < 64; o <<= 1)
#pragma unroll
        for (int v = 0; v < 4; ++v) f[tg][mb][v] += __shfl_xor(f[tg][mb][v], o);
  if (lane < 4) {
#pragma unroll
    for (int tg = 0; tg < TG; ++tg)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) red.v[wave][tg][mb][j] = f[tg][mb];
  }
  if constexpr (W > 1) __syncthreads();
  if (wave != 0 || lane >= 4 * TG) return;
  const int tg = lane >> 2, jj = lane & 3;
  const int64_t n = n0 + lane;
  if (n >= p.N) return;
  const float bv = p.bias ? p.bias[n] : 0.0f;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    f32x4 sum = red.v[0][tg][mb][jj];
#pragma unroll
    for (int w = 1; w < W; ++w) sum += red.v[w][tg][mb][jj];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t mm = m0 + 4 * mb + v;
      if (mm < p.M) p.y[mm * p.N + n] = p.xs[mm] * (sum[v] * 0.0625f) + bv;
    }
  }
}

// Cross-lane helpers of the few-rows kernel.
template <int CTRL>
__device__ __forceinline__ float q4_dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
// lanes 0-31 get a[l] + a[l + 32], lanes 32-63 get b[l - 32] + b[l]
__device__ __forceinline__ float q4_swap32_sum(float a, float b) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}
// rows 0 and 2 get a's sums with rows 1 and 3, rows 1 and 3 get b's
__device__ __forceinline__ float q4_swap16_sum(float a, float b) {
  const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

// ------------------------------------------- few rows on the matrix cores (M <= 4)
// The weights stream as TG x 4 channel rows x 256 contiguous bytes per wave
// instruction (lane 4 b + j: the whole 32-k group 16 s + b of channel 4 tg + j),
// and every step s of the wave's K is requested, with its group scales, before
// any arithmetic. Group sums are formed on the matrix cores as in the streaming
// kernel: v_mfma_i32_4x4x4_i8 block b multiplies the 4 rows of x codes of its
// group (A row i = lane 4 b + i) by the 4 channels' nibbles of that group
// unpacked as 16 c (B column j = lane 4 b + j), 8 MFMAs of 4 k, and 8 more
// against an all-ones A give 16 x the group's code sum. Lane 4 b + j then holds
// its channel's exact A16 for the 4 rows and folds each with one FMA,
// f += gs * (A16 - zp * gsum16): the vector ALU only unpacks and folds. The 16
// groups of a step (lanes j, j + 4, ..., j + 60) are summed at the end by two
// transposing exchanges (lane bits 5 and 4) and two row-rotation adds (bits 3
// and 2).
//
// The x codes (from the qparams kernel) are copied into LDS first, by buffer
// loads that write LDS, ahead of the weights: row i at i * xpitch (xpitch = 64
// mod 256) holds the first 16 bytes of every group, then the second 16, so that
// the 16 lanes of a read (4 rows x 4 groups) cover distinct banks. (Forming the
// row qparams and codes inside this kernel, every workgroup for itself, measured
// slower: 12.8 vs 8.8 us at M = 4, K = 4096, N = 11008; the workgroups that
// start last find their x reads queued behind the weight stream.)
template <int W, int TG, int NS>
__global__ __launch_bounds__(64 * W) void k_dq8ca_q4_fm(Q4Args p, int xpitch) {
  constexpr int V = 4 * TG;  // partial sums per lane: TG x 4 channels' rows 0..3
  extern __shared__ __attribute__((aligned(16))) uint8_t xl[];  // M rows of xpitch bytes
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int j = lane & 3, blk = lane >> 2;
  const int64_t M = p.M, N = p.N, K = p.K, G = K / 32, KB = K / 2;
  const int64_t n0 = ((int64_t)blockIdx.x * W + wave) * (4 * TG);
  const int64_t rem = N - n0;
  const int64_t nrows = rem <= 0 ? 0 : (rem < 4 * TG ? rem : 4 * TG);
  const __amdgpu_buffer_rsrc_t rq = rsrc(nrows > 0 ? p.q4 + n0 * KB : p.q4, (uint32_t)(nrows * KB));
  const __amdgpu_buffer_rsrc_t rg = rsrc(nrows > 0 ? p.gs + n0 * G : p.gs, (uint32_t)(nrows * G * 4));
  const int nst = (int)((KB + 255) >> 8);  // steps of 512 k (256 packed bytes a row)

  // ---- x codes into LDS first (they gate the arithmetic), then the weights
  {
    const __amdgpu_buffer_rsrc_t rx = rsrc(p.xq, (uint32_t)(M * K));
    const int cpr = (int)((K + 1023) >> 10);  // 1 KB copies per row
    const uint32_t base = (uint32_t)(uintptr_t)xl;
    for (int c = wave; c < (int)M * cpr; c += W) {
      const int i = c / cpr, u = 64 * (c % cpr) + lane;  // unit u: half u / G, group u % G
      const int h = (int)(u / G), g = (int)(u % G);
      const int src = u < 2 * G ? (int)((int64_t)i * K + 32 * g + 16 * h) : OOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rx, (lds_void *)(uintptr_t)__builtin_amdgcn_readfirstlane(base + (uint32_t)(i * xpitch + 1024 * (c % cpr))),
          16, src, 0, 0, 0);
    }
  }
  __asm__ volatile("" ::: "memory");

  i32x4 q[NS][TG];
  float gsv[NS][TG];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    // this lane's group lies before K (steps past the last, or the lanes of a
    // last step past K, read 0: zero codes and a zero group scale add nothing)
    const bool kin = s < nst && 256 * s + 16 * blk < KB;
#pragma unroll
    for (int tg = 0; tg < TG; ++tg) {
      const uint32_t row = (uint32_t)(4 * tg + j);
      q[s][tg] = __builtin_amdgcn_raw_buffer_load_b128(
          rq, kin ? (int)(row * (uint32_t)KB + 256u * s + 16u * blk) : OOB, 0, 2);
      gsv[s][tg] = __builtin_bit_cast(
          float, __builtin_amdgcn_raw_buffer_load_b32(
                     rg, kin ? (int)(4u * (row * (uint32_t)G + 16u * s + blk)) : OOB, 0, 2));
    }
  }
  // the copies of x were issued before the 2 TG NS weight loads: wait for them
  // only, then for the other waves' copies
  static_assert(2 * TG * NS < 64, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * TG * NS));
  // row scales and -zp (0 past M) by scalar loads: a vector load here would
  // wait for every weight load
  const __attribute__((address_space(4))) int32_t *xzc =
      (const __attribute__((address_space(4))) int32_t *)(uintptr_t)p.xz;
  const __attribute__((address_space(4))) float *xsc =
      (const __attribute__((address_space(4))) float *)(uintptr_t)p.xs;
  int zpn[4];
  float sc[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int v = xzc[r < M ? r : 0];
    sc[r] = xsc[r < M ? r : 0];
    zpn[r] = r < M ? -v : 0;
  }
  __builtin_amdgcn_s_barrier();
  // rows of x past M read row 0 (their sums are never written)
  const char *xrow = reinterpret_cast<const char *>(xl) + (j < M ? j : 0) * xpitch + 16 * blk;

  float t[V];
#pragma unroll
  for (int i = 0; i < V; ++i) t[i] = 0.0f;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    if (s >= nst) continue;  // uniform
    i32x4 xv[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
      xv[h] = *reinterpret_cast<const i32x4 *>(xrow + h * 16 * (int)G + 256 * s);
#pragma unroll
    for (int tg = 0; tg < TG; ++tg) {
      int wq[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t w = (uint32_t)q[s][tg][e];
        wq[2 * e] = (int)((w << 4) & 0xF0F0F0F0u);  // k = 8e + 0, 2, 4, 6, as 16 c
        wq[2 * e + 1] = (int)(w & 0xF0F0F0F0u);     // k = 8e + 1, 3, 5, 7
      }
      i32x4 cs = {0, 0, 0, 0}, a = {0, 0, 0, 0};
#pragma unroll
      for (int d = 0; d < 8; ++d) cs = __builtin_amdgcn_mfma_i32_4x4x4i8(0x01010101, wq[d], cs, 0, 0, 0);
#pragma unroll
      for (int d = 0; d < 8; ++d)
        a = __builtin_amdgcn_mfma_i32_4x4x4i8(xv[d >> 2][d & 3], wq[d], a, 0, 0, 0);
#pragma unroll
      for (int v = 0; v < 4; ++v)  // |zp| <= 128 and |gsum16| <= 4096: a 24-bit product
        t[4 * tg + v] += gsv[s][tg] * (float)(a[v] + __mul24(zpn[v], cs[0]));
    }
  }

  // ---- sum over lane bits 5..2 (the 16 groups): the transposing exchanges over
  // bits 5 and 4 halve the values a lane carries, rotations by 8 and 4 lanes
  // within each row of 16 add over bits 3 and 2
#pragma unroll
  for (int i = 0; i < V / 2; ++i) t[i] = q4_swap32_sum(t[i], t[V / 2 + i]);
#pragma unroll
  for (int i = 0; i < V / 4; ++i) t[i] = q4_swap16_sum(t[i], t[V / 4 + i]);
#pragma unroll
  for (int i = 0; i < V / 4; ++i) {
    t[i] += q4_dpp<0x128>(t[i]);  // row_ror:8
    t[i] += q4_dpp<0x124>(t[i]);  // row_ror:4
  }
  if ((lane & 12) != 0) return;
  // lane l holds, for i < TG, value index (l >> 5) V/2 + ((l >> 4) & 1) V/4 + i
#pragma unroll
  for (int i = 0; i < TG; ++i) {
    const int idx = (lane >> 5) * (V / 2) + ((lane >> 4) & 1) * (V / 4) + i;
    const int tg = idx >> 2, m = idx & 3;
    const int64_t n = n0 + 4 * tg + j;
    if (m < M && n < N) {
      const float bv = p.bias ? p.bias[n] : 0.0f;
      const float sm = m == 0 ? sc[0] : (m == 1 ? sc[1] : (m == 2 ? sc[2] : sc[3]));
      p.y[m * N + n] = sm * (t[i] * 0.0625f) + bv;
    }
  }
}

// ----------------------------------------------------------------- tiled
// M > 16, on the bf16 matrix cores with exact integer arithmetic. The
// activation operand is d = xq - zp as bf16 (an integer in [-255, 255], exact),
// written by the qparams kernel with each 8-k block in the order the weights
// unpack in; a weight nibble c becomes the bf16 128 + (c + 8) by OR-ing it into
// the mantissa of 128 (also exact). Per 32-k group
// one MFMA with a constant -136 operand gives -136 sum_k d per row, and the
// group's MFMA, accumulating on top of it, gives
//     sum_k d (136 + c) - 136 sum_k d = sum_k (xq - zp) c
// exactly: every product and partial sum is an integer below 2^24, so fp32
// accumulation does not round. The zero point therefore costs no vector op,
// and the per-output, per-group work is one FMA with the group scale (the
// integer path needs a multiply-add for the zero point, a convert and the FMA).
// The correction is per row, so it is formed once per row tile and used as the
// accumulator input of every column tile's MFMA.
//
// Tile: WM x WN waves of (16 TI) x (16 TJ) outputs, times KH waves taking
// alternate groups of each stage of GS groups (32 GS k; their sums meet in LDS
// at the end). Operands go global -> LDS by buffer loads that write LDS (bf16
// d rows of 64 GS bytes with 16-byte chunks XOR-swizzled by (row / 2) mod 8
// or, for GS = 4, row mod 16; nibble rows of 16 GS bytes, one 16-byte chunk a
// group, swizzled by (row / 8) mod 2 or (row / 2) mod 4; 16 bytes of group
// scales per row, of which the stage uses the first GS) into a ring,
// with exact vmcnt waits and a fence-free barrier as in the int8 GEMM. Every
// wave issues the same number of loads per stage; the spare ones zero-fill a
// scratch slot. The output tile is staged in LDS per wave and written as
// whole rows.
template <int TI_, int TJ_, int WM_, int WN_, int KH_, int STAGES_, int GS_ = 2>
struct QT {
  static constexpr int TI = TI_, TJ = TJ_, WM = WM_, WN = WN_, KH = KH_, STAGES = STAGES_;
  // 32-k groups per stage (2 or 4): a stage holds 64 GS bytes of each bf16 d
  // row (4 GS chunks of 16 B), 16 GS bytes of each nibble row (GS chunks)
  // and 4 GS bytes of each row's group scales (a 16-byte load)
  static constexpr int GS = GS_;
  static_assert(GS == 2 || GS == 4, "groups per stage");
  static constexpr int RA = 16 / GS, RB = 64 / GS;  // rows per 1 KB load of d / nibbles
  static constexpr int NW = WM * WN * KH;
  static constexpr int BM = 16 * TI * WM, BN = 16 * TJ * WN;
  // loads per stage of each kind, rounded up to a multiple of the wave count
  // so that a wave's q-th load is of one kind on every wave (the extra loads
  // fetch rows past the tile: the range check makes them zero, and their LDS
  // rows are never read)
  static constexpr int QA = ((BM + RA - 1) / RA + NW - 1) / NW;  // bf16 d: RA rows x 64 GS B
  static constexpr int QB = ((BN + RB - 1) / RB + NW - 1) / NW;  // nibbles: RB rows x 16 GS B
  static constexpr int QG = ((BN + 63) / 64 + NW - 1) / NW;   // scales: 64 rows x 16 B
  static constexpr int NL = QA + QB + QG;
  static constexpr int A_BYTES = QA * NW * 1024, B_BYTES = QB * NW * 1024, G_BYTES = QG * NW * 1024;
  static constexpr int B_OFF = A_BYTES, G_OFF = A_BYTES + B_BYTES;
  static constexpr int STAGE = A_BYTES + B_BYTES + G_BYTES;
  static constexpr int RING = STAGES * STAGE;
  static constexpr int OUT_LD = 16 * TJ + 4;  // words per staged output row
  static constexpr int OUT_WAVE = 16 * TI * OUT_LD * 4;
  static_assert((KH == 1 || KH == 2 || KH == 4) && GS % KH == 0, "group split");
  static constexpr int XCH = (KH - 1) * WM * WN * 64 * TI * TJ * 16;  // partial sums of kh > 0
  static constexpr int EPI = XCH + WM * WN * OUT_WAVE;
  static constexpr int LDS = RING > EPI ? RING : EPI;
};
// The smaller tiles take stages of 4 groups, one group to each of 4 waves
// that all cover the whole tile (its nibbles are unpacked once per group), and
// keep 3 stages in flight.
using QTL = QT<4, 4, 2, 2, 1, 3>;     // 128 x 128, large M
using QTW = QT<4, 3, 2, 2, 1, 2>;     // 128 x 96, 2 stages
using QTM = QT<4, 4, 1, 1, 4, 3, 4>;  // 64 x 64
using QTN = QT<4, 3, 1, 1, 4, 3, 4>;  // 64 x 48
using QTP = QT<2, 3, 1, 2, 4, 3, 4>;  // 32 x 96
using QTR = QT<2, 3, 1, 1, 4, 3, 4>;  // 32 x 48
using QTQ = QT<4, 3, 1, 2, 4, 3, 4>;  // 64 x 96

__device__ __forceinline__ bf16x8 bf16x8_splat(uint32_t bits) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const uint32_t d = bits | (bits << 16);
  return __builtin_bit_cast(bf16x8, u32x4{d, d, d, d});
}

// 8 nibbles of one lane (k = 0..7 of its 8-k slice, k even in the low nibble
// of each byte) -> bf16 136 + c in the order k = 0,4,1,5,2,6,3,7: dword i holds
// nibbles i and i + 4, which one shift and one mask-xor pull out together.
// Flipping bit 3 of a two's-complement nibble adds 8 (mod 16), so c + 8 comes
// from the same xor that sets the high byte 0x43: (raw & 0xF) ^ 0x4308 =
// 0x4300 | (c + 8), the bf16 128 + (c + 8).
__device__ __forceinline__ bf16x8 nib_bf16x8(uint32_t w) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = ((w >> (4 * i)) & 0x000F000Fu) ^ 0x43084308u;
  return __builtin_bit_cast(bf16x8, r);
}

// XOR swizzles of the 16-byte chunks of a stage's rows in LDS: d rows of
// 4 GS chunks (conflict-free 16-byte fragment reads over 16 rows), nibble rows
// of GS chunks
template <int GS>
__device__ __forceinline__ int q4_swz_a(int row) { return GS == 2 ? (row >> 1) & 7 : row & 15; }
template <int GS>
__device__ __forceinline__ int q4_swz_b(int row) { return GS == 2 ? (row >> 3) & 1 : (row >> 1) & 3; }

template <int TI_, int TJ_, int WM_, int WN_, int KH_, int STAGES_, int GS_>
__global__ __launch_bounds__(64 * WM_ * WN_ * KH_, 2) void k_dq8ca_q4_tiled(Q4Args p, int tiles_m,
                                                                            int tiles_n) {
  using C = QT<TI_, TJ_, WM_, WN_, KH_, STAGES_, GS_>;
  constexpr int GS = C::GS, SA = 64 * GS, SB = 16 * GS;  // d and nibble bytes a row per stage
  extern __shared__ __attribute__((aligned(16))) char smem[];
  constexpr int TI = C::TI, TJ = C::TJ, KH = C::KH, NL = C::NL, STAGES = C::STAGES;
  const int nt = tiles_m * tiles_n;
  const int lin = blockIdx.x;
  // Workgroups go to the 8 XCDs round-robin (XCD lin mod 8); XCD x takes the
  // contiguous tile range of its share (the first nt mod 8 XCDs one extra), so
  // the row tiles of a column tile run under one L2 and read its weights once.
  const int xq = nt >> 3, xr = nt & 7, x = lin & 7;
  const int tile = x * xq + (x < xr ? x : xr) + (lin >> 3);
  const int tn = tile / tiles_m, tm = tile % tiles_m;
  const int64_t n0 = (int64_t)tn * C::BN, m0 = (int64_t)tm * C::BM;
  const int64_t M = p.M, N = p.N, K = p.K, G = K / 32, KB = K / 2;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // wave = (kh * WM + wm) * WN + wn
  const int wn = wave % C::WN, wm = (wave / C::WN) % C::WM, kh = wave / (C::WN * C::WM);
  const int r = lane & 15, g4 = lane >> 4;
  const int64_t mval = M - m0 < C::BM ? M - m0 : C::BM;
  const int64_t nval = N - n0 < C::BN ? N - n0 : C::BN;

  // ---- loads: the q-th load of wave w is number l = (q - first q of its
  // kind) * NW + w of that kind: bf16 d (8 rows x 128 B), nibbles (32 rows x
  // 32 B), group scales (64 rows x 16 B). The kind of each q is a compile-time
  // constant, so its descriptor is uniform by construction.
  const __amdgpu_buffer_rsrc_t ra = rsrc(p.xd + m0 * K, (uint32_t)(mval * K * 2));
  const __amdgpu_buffer_rsrc_t rb = rsrc(p.q4 + n0 * KB, (uint32_t)(nval * KB));
  const __amdgpu_buffer_rsrc_t rg = rsrc(p.gs + n0 * G, (uint32_t)(nval * G * 4));
  uint32_t off[NL], lds_off[NL];
  int klim[NL];  // first stage whose bytes for this lane lie past the row
#pragma unroll
  for (int q = 0; q < NL; ++q) {
    if (q < C::QA) {
      const int l = q * C::NW + wave;
      const int row = C::RA * l + lane / (4 * GS), c = (lane % (4 * GS)) ^ q4_swz_a<GS>(row);
      off[q] = (uint32_t)row * (uint32_t)(2 * K) + 16u * c;
      lds_off[q] = (uint32_t)(l * 1024);
      klim[q] = (int)((2 * K - 16 * c + SA - 1) / SA);
    } else if (q < C::QA + C::QB) {
      const int l = (q - C::QA) * C::NW + wave;
      const int row = C::RB * l + lane / GS, c = (lane % GS) ^ q4_swz_b<GS>(row);
      off[q] = (uint32_t)row * (uint32_t)KB + 16u * c;
      lds_off[q] = (uint32_t)(C::B_OFF + l * 1024);
      klim[q] = (int)((KB - 16 * c + SB - 1) / SB);
    } else {
      const int l = (q - C::QA - C::QB) * C::NW + wave;
      const int row = 64 * l + lane;
      off[q] = (uint32_t)row * (uint32_t)(G * 4);
      lds_off[q] = (uint32_t)(C::G_OFF + l * 1024);
      klim[q] = (int)((G + GS - 1) / GS);
    }
  }
  const uint32_t lds_base = (uint32_t)(uintptr_t)smem;
  const int nk = (int)((K + 32 * GS - 1) / (32 * GS));
  // The first nf stages lie inside every row for every load (d and nibbles up
  // to the last stage; the 16-byte group-scale load up to stage (G - 4) / GS):
  // their offset along the row is uniform and goes in the scalar offset, with
  // no per-lane range test. Later stages test each lane.
  auto issue_as = [&](int kt, auto full) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < NL; ++q) {
      const uint32_t kstep = q < C::QA ? (uint32_t)SA : (q < C::QA + C::QB ? (uint32_t)SB : 4u * GS);
      const uint32_t dst = lds_base + lds_off[q] + (uint32_t)((kt % STAGES) * C::STAGE);
      lds_void *d = (lds_void *)(uintptr_t)__builtin_amdgcn_readfirstlane(dst);
      const __amdgpu_buffer_rsrc_t rs = q < C::QA ? ra : (q < C::QA + C::QB ? rb : rg);
      if constexpr (decltype(full)::value) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, d, 16, (int)off[q], (int)(kstep * (uint32_t)kt), 0, 0);
      } else {
        const int o = kt < klim[q] ? (int)(off[q] + kstep * (uint32_t)kt) : OOB;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, d, 16, o, 0, 0, 0);
      }
    }
  };
  const int nf = G >= 4 ? min(nk - 1, (int)(G - 4) / GS + 1) : 0;
  auto issue_full = [&](int kt) { issue_as(kt, std::true_type{}); };
  auto issue_tail = [&](int kt) { issue_as(kt, std::false_type{}); };

  f32x4 f[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) f[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int kt) __attribute__((always_inline)) {
    const char *st = smem + (kt % STAGES) * C::STAGE;
    const bf16x8 bneg = bf16x8_splat(0xC308u);  // -136 in every element
#pragma unroll
    for (int x = 0; x < GS / KH; ++x) {
      const int gg = kh + KH * x;  // group within the stage
      if (GS * kt + gg < (int)G) { // uniform: the last stage may hold fewer groups
        bf16x8 a[TI], b[TJ];
        f32x4 corr[TI];
        float gsv[TJ];
#pragma unroll
        for (int i = 0; i < TI; ++i) {
          const int R = wm * 16 * TI + 16 * i + r;
          const int c = 4 * gg + g4;
          a[i] = *reinterpret_cast<const bf16x8 *>(st + R * SA + 16 * (c ^ q4_swz_a<GS>(R)));
        }
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
          const int R = wn * 16 * TJ + 16 * j + r;
          const uint32_t w = *reinterpret_cast<const uint32_t *>(
              st + C::B_OFF + R * SB + 16 * (gg ^ q4_swz_b<GS>(R)) + 4 * g4);
          b[j] = nib_bf16x8(w);
          gsv[j] = *reinterpret_cast<const float *>(st + C::G_OFF + R * 16 + 4 * gg);
        }
        __builtin_amdgcn_s_setprio(1);  // MFMA run at raised wave priority
#pragma unroll
        for (int i = 0; i < TI; ++i)
          corr[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], bneg, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        // Row by row: the FMAs that fold row i - 1's group sums into f go
        // between row i's MFMAs (whose results they do not need), so the
        // vector ALU and the matrix core work side by side.
        f32x4 tp[TJ], tc[TJ];
#pragma unroll
        for (int i = 0; i < TI; ++i) {
#pragma unroll
          for (int j = 0; j < TJ; ++j)
            tc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], corr[i], 0, 0, 0);
          if (i > 0) {
#pragma unroll
            for (int j = 0; j < TJ; ++j)
#pragma unroll
              for (int v = 0; v < 4; ++v) f[i - 1][j][v] = __builtin_fmaf(gsv[j], tp[j][v], f[i - 1][j][v]);
          }
#pragma unroll
          for (int j = 0; j < TJ; ++j) tp[j] = tc[j];
        }
#pragma unroll
        for (int j = 0; j < TJ; ++j)
#pragma unroll
          for (int v = 0; v < 4; ++v) f[TI - 1][j][v] = __builtin_fmaf(gsv[j], tp[j][v], f[TI - 1][j][v]);
        __builtin_amdgcn_s_setprio(0);
        // issue order: the fragment reads, the corrections with the unpacking
        // between them, then per row its MFMAs each followed by 4 of the
        // previous row's FMAs
        __builtin_amdgcn_sched_group_barrier(0x100, TI + 2 * TJ, 0);
#pragma unroll
        for (int i = 0; i < TI; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, (9 * TJ + TI - 1) / TI, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, TJ, 0);
#pragma unroll
        for (int u = 0; u < (TI - 1) * TJ; ++u) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
        }
      }
    }
  };

#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s) {
    if (s < nf) issue_full(s);
    else issue_tail(s);
  }
  int kt = 0;
  static_assert(NL * (STAGES - 2) < 64, "vmcnt immediate");
  auto step = [&](int k, auto full) __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(NL * (STAGES - 2)));
    __builtin_amdgcn_s_barrier();
    issue_as(k + STAGES - 1, full);
    compute(k);
    __builtin_amdgcn_s_waitcnt(0xC07F);
  };
  // steps issuing stages below nf: whole turns of the ring first, so that
  // each step's LDS slot offsets are constants
  for (; kt + 2 * STAGES - 1 <= nf; kt += STAGES) {
#pragma unroll
    for (int u = 0; u < STAGES; ++u) step(kt + u, std::true_type{});
  }
  for (; kt + STAGES - 1 < nf; ++kt) step(kt, std::true_type{});
  for (; kt < nk - (STAGES - 1); ++kt) step(kt, std::false_type{});
#pragma unroll
  for (int t = 0; t < STAGES - 1; ++t) {
    if (kt < nk) {
      // stages issued after stage kt: STAGES - 2 - t
      if (t == 0) __builtin_amdgcn_s_waitcnt(vmcnt_imm(NL * (STAGES - 2)));
      else if (t == 1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(STAGES > 3 ? NL * (STAGES - 3) : 0));
      else if (t == 2) __builtin_amdgcn_s_waitcnt(vmcnt_imm(STAGES > 4 ? NL * (STAGES - 4) : 0));
      else __builtin_amdgcn_s_waitcnt(0x0F70);
      __builtin_amdgcn_s_barrier();
      compute(kt);
      __builtin_amdgcn_s_waitcnt(0xC07F);
    }
    ++kt;
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();  // ring no longer read or written

  // ---- KH > 1: waves kh > 0 hand their sums to kh = 0, which adds them in
  // the order of kh
  const int pw = wm * C::WN + wn;  // plane wave 0 .. WM WN - 1
  if constexpr (KH > 1) {
    f32x4 *xch = reinterpret_cast<f32x4 *>(smem);
    constexpr int PLANE = C::WM * C::WN * TI * TJ * 64;  // f32x4 per kh slot
    if (kh > 0) {
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) xch[(kh - 1) * PLANE + ((pw * TI + i) * TJ + j) * 64 + lane] = f[i][j];
    }
    __syncthreads();
    if (kh == 0) {
#pragma unroll
      for (int h = 1; h < KH; ++h)
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
          for (int j = 0; j < TJ; ++j) f[i][j] += xch[(h - 1) * PLANE + ((pw * TI + i) * TJ + j) * 64 + lane];
    }
  }
  if (kh != 0) return;

  // ---- y = xs[m] f + bias[n], staged per wave: f[i][j] lane holds rows
  // 4 g4 + v, column r of MFMA tile (i, j)
  float *tl = reinterpret_cast<float *>(smem + C::XCH + pw * C::OUT_WAVE);
  const int64_t wm0 = m0 + wm * 16 * TI, wn0 = n0 + wn * 16 * TJ;
  // row scales and bias by range-checked loads, all in flight together (rows
  // past M and columns past N, or no bias, read 0)
  const __amdgpu_buffer_rsrc_t rxs = rsrc(p.xs + m0, (uint32_t)(mval * 4));
  const __amdgpu_buffer_rsrc_t rbi = rsrc(p.bias ? p.bias + n0 : p.xs, p.bias ? (uint32_t)(nval * 4) : 0u);
  float xsv[TI][4], bv[TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int v = 0; v < 4; ++v)
      xsv[i][v] = __builtin_bit_cast(
          float, __builtin_amdgcn_raw_buffer_load_b32(rxs, 4 * (wm * 16 * TI + 16 * i + 4 * g4 + v), 0, 0));
#pragma unroll
  for (int j = 0; j < TJ; ++j)
    bv[j] = __builtin_bit_cast(
        float, __builtin_amdgcn_raw_buffer_load_b32(rbi, 4 * (wn * 16 * TJ + 16 * j + r), 0, 0));
#pragma unroll
  for (int j = 0; j < TJ; ++j)
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        tl[(16 * i + 4 * g4 + v) * C::OUT_LD + 16 * j + r] = xsv[i][v] * f[i][j][v] + bv[j];
  // the wave reads back only what it wrote: no barrier needed beyond the
  // wave's own LDS ordering
  __builtin_amdgcn_s_waitcnt(0xC07F);
  constexpr int CPR = 4 * TJ;  // 16-byte chunks per row
  const bool vec = (N & 3) == 0;
#pragma unroll
  for (int u = lane; u < 16 * TI * CPR; u += 64) {
    const int row = u / CPR, c = u % CPR;
    const int64_t m = wm0 + row, n = wn0 + 4 * c;
    if (m >= M || n >= N) continue;
    const f32x4 val = *reinterpret_cast<const f32x4 *>(tl + row * C::OUT_LD + 4 * c);
    float *dst = p.y + m * N + n;
    if (vec) {
      *reinterpret_cast<f32x4 *>(dst) = val;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (n + e < N) dst[e] = val[e];
    }
  }
}

template <int TG, int MB>
void launch_stream(int W, dim3 grid, const Q4Args &a, hipStream_t st) {
  constexpr int U = TG * MB <= 4 ? 2 : 1;
  switch (W) {
#define AQL_W(w)                                                                              \
  case w: hipLaunchKernelGGL((k_dq8ca_q4_stream<w, TG, MB, U>), grid, dim3(64 * w), 0, st, a); break;
    AQL_W(8) AQL_W(4) AQL_W(2) default : AQL_W(1)
#undef AQL_W
  }
}

template <int TG>
void launch_stream_tg(int MB, int W, dim3 grid, const Q4Args &a, hipStream_t st) {
  switch (MB) {
    case 1: launch_stream<TG, 1>(W, grid, a, st); break;
    case 2: launch_stream<TG, 2>(W, grid, a, st); break;
    default: launch_stream<TG, 4>(W, grid, a, st); break;
  }
}

template <typename C>
void launch_tiled(const Q4Args &a, hipStream_t st) {
  constexpr auto kern = k_dq8ca_q4_tiled<C::TI, C::TJ, C::WM, C::WN, C::KH, C::STAGES, C::GS>;
  const int tiles_m = (int)((a.M + C::BM - 1) / C::BM);
  const int tiles_n = (int)((a.N + C::BN - 1) / C::BN);
  // more than 64 KB of dynamic LDS: raise the function's limit once (a launch
  // the limit does not allow reports its own error)
  static bool attr = false;
  if (!attr) {
    (void)hipFuncSetAttribute((const void *)kern,
                              hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS);
    (void)hipGetLastError();
    attr = true;
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)(tiles_m * tiles_n)), dim3(64 * C::NW),
                     C::LDS, st, a, tiles_m, tiles_n);
}

// Few rows on the matrix cores: 4 waves of 4 channels, all of K in flight (NS
// steps of 512 k). K = 4096, N = 11008: 8.8 us at M = 4 and 8.0 at M = 1,
// against 10.0 and 8.2 for group sums formed by 4-byte dot products on the
// vector ALU (1 KB weight pieces); 2 channel groups a wave or 8 waves a
// workgroup measured slower.
void launch_fm(const Q4Args &a, hipStream_t st) {
  constexpr int W = 4, TG = 1;
  const dim3 grid((unsigned)((a.N + 4 * TG * W - 1) / (4 * TG * W)));
  const int xpitch = (int)((a.K + 1023) / 1024 * 1024 + 64);
  const size_t lds = (size_t)(a.M * xpitch);
#define AQL_FM(ns) hipLaunchKernelGGL((k_dq8ca_q4_fm<W, TG, ns>), grid, dim3(64 * W), lds, st, a, xpitch)
  if (a.K <= 512) AQL_FM(1);
  else if (a.K <= 1024) AQL_FM(2);
  else if (a.K <= 2048) AQL_FM(4);
  else if (a.K <= 4096) AQL_FM(8);
  else AQL_FM(16);
#undef AQL_FM
}

}  // namespace

hipError_t launch_dq8ca_q4(const Q4Args &a, hipStream_t st) {
  if (a.M <= kQ4FewMaxM && a.K <= kQ4FewMaxK) {
    launch_fm(a, st);
  } else if (a.M <= kQ4StreamMaxM) {
    // 8-channel tiles for M <= 2, 16 otherwise; waves per workgroup (splitting
    // K) only while the wave-tiles are fewer than ~384: these waves are short
    // and few, and a K split adds a cross-wave reduction to each
    const int MB = a.M <= 4 ? 1 : (a.M <= 8 ? 2 : 4);
    const int TG = a.M <= 2 ? 2 : 4;
    const int64_t nst = (a.K / 2 + 255) / 256;
    const int64_t tiles = (a.N + 4 * TG - 1) / (4 * TG);
    int W = 1;
    while (W < 8 && tiles * W < 384 && W * 4 <= nst) W <<= 1;
    const dim3 grid((unsigned)tiles, 1);
    if (TG == 2) launch_stream_tg<2>(MB, W, grid, a, st);
    else launch_stream_tg<4>(MB, W, grid, a, st);
  } else {
    // Tile by the rows and the count of 128 x 128 tiles, as measured at
    // K = 4096, N = 11008 with the weights streamed from HBM: 128 x 128 from
    // 2.5 such tiles a CU (277 us at M = 2048 against 294 for 128 x 96),
    // 128 x 96 in 2 stages from M = 384 (70.4 vs 74.9 us for 64 x 48 at
    // M = 384, 75.3 vs 84.2 for 128 x 128 at M = 512); below that 32 x 48 up
    // to M = 32 (15.7 us, 26.0 for 64 x 64 tiles with two groups a stage over
    // two waves), 32 x 96 up to M = 64 (19.6 vs 20.9 for 32 x 48), 64 x 48 up
    // to M = 256 (29.7 vs 37.8 at M = 128, 47.1 vs 56.6 at M = 200) and
    // 64 x 64 above (58.2 vs 67.8 at M = 300)
    // 64 x 96 where its tiles fit one round of the 256 CUs and those of 64 x 48
    // do not, the last row tile at least half full (M = 128: 31.2 vs 33.3 us;
    // M = 96 30.3 vs 30.4; M = 80 29.7 vs 29.2; M = 160-200, two rounds of
    // 64 x 96, 54-55 vs 48-52)
    const int64_t tl = ((a.M + QTL::BM - 1) / QTL::BM) * ((a.N + QTL::BN - 1) / QTL::BN);
    const int64_t rt = (a.M + 63) / 64;
    const bool q96 = rt * ((a.N + QTN::BN - 1) / QTN::BN) > 256 &&
                     rt * ((a.N + QTQ::BN - 1) / QTQ::BN) <= 256 && (a.M % 64 == 0 || a.M % 64 >= 32);
    if (tl >= 640) launch_tiled<QTL>(a, st);
    else if (a.M >= 384) launch_tiled<QTW>(a, st);
    else if (a.M <= 32) launch_tiled<QTR>(a, st);
    else if (a.M <= 64) launch_tiled<QTP>(a, st);
    else if (q96) launch_tiled<QTQ>(a, st);
    else if (a.M <= 256) launch_tiled<QTN>(a, st);
    else launch_tiled<QTM>(a, st);
  }
  return hipGetLastError();
}

}  // namespace aql
