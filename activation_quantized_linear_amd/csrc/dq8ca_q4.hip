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
#include "dq8ca_q4.h"

namespace aql {
namespace {

typedef __attribute__((address_space(3))) void lds_void;

constexpr int OOB = 0x40000000;  // an offset past any range: buffer loads return 0

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                           0x00020000);
}

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
// alternate groups of each 64-k stage (their sums meet in LDS at the end).
// Operands go global -> LDS by buffer loads that write LDS (bf16 d rows of
// 128 B with 16-byte chunks XOR-swizzled by (row / 2) mod 8; nibble rows of
// 32 B with their two group chunks swapped on odd eighths of rows; 16 bytes of
// group scales per row, of which the stage uses the first two) into a ring,
// with exact vmcnt waits and a fence-free barrier as in the int8 GEMM. Every
// wave issues the same number of loads per stage; the spare ones zero-fill a
// scratch slot. The output tile is staged in LDS per wave and written as
// whole rows.
template <int TI_, int TJ_, int WM_, int WN_, int KH_, int STAGES_>
struct QT {
  static constexpr int TI = TI_, TJ = TJ_, WM = WM_, WN = WN_, KH = KH_, STAGES = STAGES_;
  static constexpr int NW = WM * WN * KH;
  static constexpr int BM = 16 * TI * WM, BN = 16 * TJ * WN;
  // loads per stage of each kind, rounded up to a multiple of the wave count
  // so that a wave's q-th load is of one kind on every wave (the extra loads
  // fetch rows past the tile: the range check makes them zero, and their LDS
  // rows are never read)
  static constexpr int QA = (BM * 128 / 1024 + NW - 1) / NW;  // bf16 d: 8 rows x 128 B each
  static constexpr int QB = (BN * 32 / 1024 + NW - 1) / NW;   // nibbles: 32 rows x 32 B
  static constexpr int QG = (BN * 16 / 1024 + NW - 1) / NW;   // scales: 64 rows x 16 B
  static constexpr int NL = QA + QB + QG;
  static constexpr int A_BYTES = QA * NW * 1024, B_BYTES = QB * NW * 1024, G_BYTES = QG * NW * 1024;
  static constexpr int B_OFF = A_BYTES, G_OFF = A_BYTES + B_BYTES;
  static constexpr int STAGE = A_BYTES + B_BYTES + G_BYTES;
  static constexpr int RING = STAGES * STAGE;
  static constexpr int OUT_LD = 16 * TJ + 4;  // words per staged output row
  static constexpr int OUT_WAVE = 16 * TI * OUT_LD * 4;
  static constexpr int XCH = KH == 2 ? WM * WN * 64 * TI * TJ * 16 : 0;  // partial sums of kh = 1
  static constexpr int EPI = XCH + WM * WN * OUT_WAVE;
  static constexpr int LDS = RING > EPI ? RING : EPI;
};
using QTL = QT<4, 4, 2, 2, 1, 3>;  // 128 x 128, large M
using QTS = QT<4, 2, 1, 2, 2, 4>;  // 64 x 64, groups split over two waves

__device__ __forceinline__ bf16x8 bf16x8_splat(uint32_t bits) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const uint32_t d = bits | (bits << 16);
  return __builtin_bit_cast(bf16x8, u32x4{d, d, d, d});
}

// 8 nibbles of one lane (k = 0..7 of its 8-k slice, k even in the low nibble
// of each byte) -> bf16 136 + c in the order k = 0,4,1,5,2,6,3,7: dword i holds
// nibbles i and i + 4, which one shift and one mask-or pull out together.
__device__ __forceinline__ bf16x8 nib_bf16x8(uint32_t w) {
  const uint32_t u = w ^ 0x88888888u;
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = ((u >> (4 * i)) & 0x000F000Fu) | 0x43004300u;
  return __builtin_bit_cast(bf16x8, r);
}

template <int TI_, int TJ_, int WM_, int WN_, int KH_, int STAGES_>
__global__ __launch_bounds__(64 * WM_ * WN_ * KH_, 2) void k_dq8ca_q4_tiled(Q4Args p, int tiles_m,
                                                                            int tiles_n) {
  using C = QT<TI_, TJ_, WM_, WN_, KH_, STAGES_>;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  constexpr int TI = C::TI, TJ = C::TJ, KH = C::KH, NL = C::NL, STAGES = C::STAGES;
  const int nt = tiles_m * tiles_n;
  const int lin = blockIdx.x;
  int tile = lin;
  if ((nt & 7) == 0) tile = (lin & 7) * (nt >> 3) + (lin >> 3);
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
      const int row = 8 * l + (lane >> 3), c = (lane & 7) ^ ((row >> 1) & 7);
      off[q] = (uint32_t)row * (uint32_t)(2 * K) + 16u * c;
      lds_off[q] = (uint32_t)(l * 1024);
      klim[q] = (int)((2 * K - 16 * c + 127) / 128);
    } else if (q < C::QA + C::QB) {
      const int l = (q - C::QA) * C::NW + wave;
      const int row = 32 * l + (lane >> 1), c = (lane & 1) ^ ((row >> 3) & 1);
      off[q] = (uint32_t)row * (uint32_t)KB + 16u * c;
      lds_off[q] = (uint32_t)(C::B_OFF + l * 1024);
      klim[q] = (int)((KB - 16 * c + 31) / 32);
    } else {
      const int l = (q - C::QA - C::QB) * C::NW + wave;
      const int row = 64 * l + lane;
      off[q] = (uint32_t)row * (uint32_t)(G * 4);
      lds_off[q] = (uint32_t)(C::G_OFF + l * 1024);
      klim[q] = (int)((G + 1) / 2);
    }
  }
  const uint32_t lds_base = (uint32_t)(uintptr_t)smem;
  auto issue = [&](int kt) {
#pragma unroll
    for (int q = 0; q < NL; ++q) {
      const uint32_t kstep = q < C::QA ? 128u : (q < C::QA + C::QB ? 32u : 8u);
      const uint32_t dst = lds_base + lds_off[q] + (uint32_t)((kt % STAGES) * C::STAGE);
      const int o = kt < klim[q] ? (int)(off[q] + kstep * (uint32_t)kt) : OOB;
      lds_void *d = (lds_void *)(uintptr_t)__builtin_amdgcn_readfirstlane(dst);
      const __amdgpu_buffer_rsrc_t rs = q < C::QA ? ra : (q < C::QA + C::QB ? rb : rg);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, d, 16, o, 0, 0, 0);
    }
  };

  f32x4 f[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) f[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int kt) {
    const char *st = smem + (kt % STAGES) * C::STAGE;
    const bf16x8 bneg = bf16x8_splat(0xC308u);  // -136 in every element
#pragma unroll
    for (int x = 0; x < 2 / KH; ++x) {
      const int gg = kh + KH * x;  // group within the stage
      if (2 * kt + gg < G) {       // uniform: the last stage may hold one group
        bf16x8 a[TI], b[TJ];
        f32x4 corr[TI];
        float gsv[TJ];
#pragma unroll
        for (int i = 0; i < TI; ++i) {
          const int R = wm * 16 * TI + 16 * i + r;
          const int c = 4 * gg + g4;
          a[i] = *reinterpret_cast<const bf16x8 *>(st + R * 128 + 16 * (c ^ ((R >> 1) & 7)));
        }
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
          const int R = wn * 16 * TJ + 16 * j + r;
          const uint32_t w = *reinterpret_cast<const uint32_t *>(
              st + C::B_OFF + R * 32 + 16 * (gg ^ ((R >> 3) & 1)) + 4 * g4);
          b[j] = nib_bf16x8(w);
          gsv[j] = *reinterpret_cast<const float *>(st + C::G_OFF + R * 16 + 4 * gg);
        }
        __builtin_amdgcn_s_setprio(1);  // MFMA run at raised wave priority
#pragma unroll
        for (int i = 0; i < TI; ++i)
          corr[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], bneg, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
          for (int j = 0; j < TJ; ++j) {
            const f32x4 t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], corr[i], 0, 0, 0);
#pragma unroll
            for (int v = 0; v < 4; ++v) f[i][j][v] = __builtin_fmaf(gsv[j], t[v], f[i][j][v]);
          }
        __builtin_amdgcn_s_setprio(0);
      }
    }
  };

  const int nk = (int)((K + 63) / 64);
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s) issue(s);
  int kt = 0;
  static_assert(NL * (STAGES - 2) < 16, "vmcnt immediate");
  for (; kt < nk - (STAGES - 1); ++kt) {
    __builtin_amdgcn_s_waitcnt(0x0F70 | (NL * (STAGES - 2)));
    __builtin_amdgcn_s_barrier();
    issue(kt + STAGES - 1);
    compute(kt);
    __builtin_amdgcn_s_waitcnt(0xC07F);
  }
#pragma unroll
  for (int t = 0; t < STAGES - 1; ++t) {
    if (kt < nk) {
      // stages issued after stage kt: STAGES - 2 - t
      if (t == 0) __builtin_amdgcn_s_waitcnt(0x0F70 | (NL * (STAGES - 2)));
      else if (t == 1) __builtin_amdgcn_s_waitcnt(0x0F70 | (STAGES > 3 ? NL * (STAGES - 3) : 0));
      else if (t == 2) __builtin_amdgcn_s_waitcnt(0x0F70 | (STAGES > 4 ? NL * (STAGES - 4) : 0));
      else __builtin_amdgcn_s_waitcnt(0x0F70);
      __builtin_amdgcn_s_barrier();
      compute(kt);
      __builtin_amdgcn_s_waitcnt(0xC07F);
    }
    ++kt;
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();  // ring no longer read or written

  // ---- KH = 2: waves kh = 1 hand their sums to kh = 0
  const int pw = wm * C::WN + wn;  // plane wave 0 .. WM WN - 1
  if constexpr (KH == 2) {
    f32x4 *xch = reinterpret_cast<f32x4 *>(smem);
    if (kh == 1) {
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) xch[((pw * TI + i) * TJ + j) * 64 + lane] = f[i][j];
    }
    __syncthreads();
    if (kh == 0) {
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) f[i][j] += xch[((pw * TI + i) * TJ + j) * 64 + lane];
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
  constexpr auto kern = k_dq8ca_q4_tiled<C::TI, C::TJ, C::WM, C::WN, C::KH, C::STAGES>;
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

}  // namespace

hipError_t launch_dq8ca_q4(const Q4Args &a, hipStream_t st) {
  if (a.M <= kQ4StreamMaxM) {
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
    // 128 x 128 tiles once they give every CU a few; else 64 x 64 tiles with
    // the groups split over two waves
    const int64_t tl = ((a.M + QTL::BM - 1) / QTL::BM) * ((a.N + QTL::BN - 1) / QTL::BN);
    if (tl >= 512) launch_tiled<QTL>(a, st);
    else launch_tiled<QTS>(a, st);
  }
  return hipGetLastError();
}

}  // namespace aql
