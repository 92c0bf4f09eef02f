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
#include "common.h"

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
// Bound by streaming the packed weights (and their group scales and sums) from
// HBM. The access shape follows the weight-only GEMV: a wave instruction reads
// 4 weight rows x 256 contiguous bytes, so each lane holds 16 bytes = one whole
// 32-k group of one channel (lane % 4 = row, lane / 4 = group within the step),
// plus that group's scale and sum (4 rows x 64 contiguous bytes each). The
// group is multiplied where it lands with v_mfma_i32_4x4x4_i8: block b = lane / 4
// takes k-slices of group b for 4 channels (B column j = lane % 4) against the
// same k-slices of 4 rows of xq (A row i = lane % 4), so after 8 MFMAs lane
// 4b + j holds, for each of its 4 rows, the exact int32 group sum of its own
// channel: the zero point and the group scale are folded in right there.
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
  const __amdgpu_buffer_rsrc_t rm = rsrc(p.gsum + n0 * G, (uint32_t)(nrows * G * 4));
  const __amdgpu_buffer_rsrc_t rx = rsrc(p.xq + m0 * K, (uint32_t)(mrows * K));
  const uint32_t qlane = (uint32_t)(j * KB + 16 * blk);
  const uint32_t glane = 4u * (uint32_t)(j * G + blk);
  const uint32_t xlane = (uint32_t)(j * K + 32 * blk);
  const int nst = (int)((KB + 255) >> 8);
  const int cnt = wave < nst ? (nst - wave + W - 1) / W : 0;

  int zp16[MB][4];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t mm = m0 + 4 * mb + v;
      zp16[mb][v] = mm < p.M ? -16 * p.xz[mm] : 0;
    }

  f32x4 f[TG][MB];
#pragma unroll
  for (int tg = 0; tg < TG; ++tg)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) f[tg][mb] = f32x4{0.f, 0.f, 0.f, 0.f};

  struct Batch {
    i32x4 q[U][TG];
    float gs[U][TG];
    int gm[U][TG];
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
        bt.gm[u][tg] = (int)__builtin_amdgcn_raw_buffer_load_b32(rm, go, 0, 2);
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
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          i32x4 t = {0, 0, 0, 0};
#pragma unroll
          for (int d = 0; d < 8; ++d)
            t = __builtin_amdgcn_mfma_i32_4x4x4i8(bt.x[u][mb][d >> 2][d & 3], wq[d], t, 0, 0, 0);
#pragma unroll
          for (int v = 0; v < 4; ++v)
            f[tg][mb][v] += bt.gs[u][tg] * (float)(t[v] + __mul24(zp16[mb][v], bt.gm[u][tg]));
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
// M > 16. The per-group fold (one 24-bit multiply-add for the zero point, one
// convert, one fused multiply-add with the group scale per output and group)
// runs on the vector ALU and bounds the kernel; everything else is arranged
// around keeping it fed. A 64 x 64 output tile per workgroup; each wave owns a
// 32 x 32 block (2 x 2 MFMA tiles, fp32 accumulators in registers) and, with
// KH = 2, every other group of each 128-k stage (the halves are summed once
// at the end). One v_mfma_i32_16x16x32_i8 is exactly one group.
//
// Operands go global -> LDS by buffer loads that write LDS, per 128-k stage:
// xq 64 rows x 128 B (8 instructions), nibbles 64 rows x 64 B (4), group
// scales and group sums 64 rows x 16 B (4 dword instructions each) and four
// zero-filling loads into a scratch slot so every wave issues the same count
// (24 / waves). A
// 4-stage ring keeps three stages in flight behind exact vmcnt waits and a
// fence-free barrier, as in the int8 GEMM. xq rows store their 16-byte
// chunks XOR-swizzled by row mod 8, nibble rows by row mod 4.
namespace {
constexpr int TB = 64;                          // tile rows and columns
constexpr int Q_STAGES = 3;
constexpr int QA_BYTES = TB * 128;              // xq: 128 k
constexpr int QB_BYTES = TB * 64;               // nibbles: 128 k
constexpr int QG_BYTES = TB * 16;               // 4 group scales (or sums) per row
constexpr int Q_STAGE = QA_BYTES + QB_BYTES + 2 * QG_BYTES;  // 14 KB
constexpr int Q_DUMMY = Q_STAGES * Q_STAGE;     // scratch slot for padding loads
constexpr int Q_LDS = Q_DUMMY + 1024;
constexpr int Q_TILE_LD = TB + 4;               // words per staged output row
static_assert(TB * Q_TILE_LD * 4 + 4 * 4 * 64 * 16 <= Q_DUMMY, "epilogue (tile + half-sum exchange) fits in the ring");
}  // namespace

// Kind of a wave's q-th load per stage (see the kernel): xq, nibbles,
// padding or a group-scale / group-sum dword load.
enum { KXQ, KNIB, KPAD, KGS };
template <int KH>
__host__ __device__ constexpr int q4_load_kind(int q) {
  return KH == 1 ? (q < 2 ? KXQ : q == 2 ? KNIB : q == 3 ? KPAD : KGS)
                 : (q == 0 ? KXQ : q == 1 ? KNIB : KGS);
}

template <int KH>
__global__ __launch_bounds__(256 * KH, 2 / KH) void k_dq8ca_q4_tiled(Q4Args p, int tiles_m, int tiles_n) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  constexpr int NW = 4 * KH, NL = 24 / NW;  // waves, loads per wave per stage
  const int nt = tiles_m * tiles_n;
  const int lin = blockIdx.x;
  int tile = lin;
  if ((nt & 7) == 0) tile = (lin & 7) * (nt >> 3) + (lin >> 3);
  const int tn = tile / tiles_m, tm = tile % tiles_m;
  const int64_t n0 = (int64_t)tn * TB, m0 = (int64_t)tm * TB;
  const int64_t M = p.M, N = p.N, K = p.K, G = K / 32, KB = K / 2;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kh = wave >> 2, wm = (wave >> 1) & 1, wn = wave & 1;
  const int r = lane & 15, g4 = lane >> 4;
  const int64_t mval = M - m0 < TB ? M - m0 : TB;
  const int64_t nval = N - n0 < TB ? N - n0 : TB;

  // ---- per stage 24 loads, NL per wave. Load q of a wave is of one kind for
  // every wave (so its size is a compile-time constant); waves differ only in
  // uniform addresses. Kinds: xq (8 rows x 128 B), nibbles (16 rows x 64 B),
  // group scales / group sums (16 rows x 4 dwords, one dword per lane so each is
  // range-checked on its own: a row's groups need not fill the last stage),
  // and zero-filling padding into a scratch slot.
  // (buffer descriptors are formed at issue time: an array of them is not a
  // host-side type)
  const void *rbase[NL];
  uint32_t rbytes[NL];
  uint32_t off[NL], lds_off[NL], kstep[NL];
  int kin_lim[NL];  // per lane: first stage whose bytes for this lane lie past K
#pragma unroll
  for (int q = 0; q < NL; ++q) {
    const int kind = q4_load_kind<KH>(q);
    if (kind == KXQ) {
      const int slot = KH == 1 ? 4 * q + wave : wave;  // 0..7
      const int row = 8 * slot + (lane >> 3), c = (lane & 7) ^ (row & 7);
      rbase[q] = p.xq + m0 * K;
      rbytes[q] = (uint32_t)(mval * K);
      off[q] = (uint32_t)row * (uint32_t)K + 16u * c;
      lds_off[q] = (uint32_t)(slot * 1024);
      kstep[q] = 128;
      kin_lim[q] = (int)((K - 16 * c + 127) / 128);
    } else if (kind == KNIB || kind == KPAD) {
      // KH = 2: waves 4..7 pad
      const bool pad = kind == KPAD || wave >= 4;
      const int slot = wave & 3;
      const int row = 16 * slot + (lane >> 2), c = (lane & 3) ^ (row & 3);
      rbase[q] = p.q4 + n0 * KB;
      rbytes[q] = pad ? 0u : (uint32_t)(nval * KB);
      off[q] = pad ? (uint32_t)OOB : (uint32_t)row * (uint32_t)KB + 16u * c;
      lds_off[q] = pad ? (uint32_t)Q_DUMMY : (uint32_t)(QA_BYTES + slot * 1024);
      kstep[q] = pad ? 0u : 64u;
      kin_lim[q] = pad ? 0 : (int)((KB - 16 * c + 63) / 64);
    } else {
      // KH = 1: load 4 = scales, 5 = sums; KH = 2: waves 0..3 scales, 4..7 sums
      const bool sums = KH == 1 ? q == 5 : wave >= 4;
      const int part = wave & 3;
      const int row = 16 * part + (lane >> 2), e = lane & 3;
      rbase[q] = sums ? (const void *)(p.gsum + n0 * G) : (const void *)(p.gs + n0 * G);
      rbytes[q] = (uint32_t)(nval * G * 4);
      off[q] = (uint32_t)row * (uint32_t)(G * 4) + 4u * e;
      lds_off[q] = (uint32_t)(QA_BYTES + QB_BYTES + (sums ? QG_BYTES : 0) + part * 256);
      kstep[q] = 16;
      kin_lim[q] = (int)((G - e + 3) / 4);
    }
  }
  const uint32_t lds_base = (uint32_t)(uintptr_t)smem;
  auto issue = [&](int kt) {
#pragma unroll
    for (int q = 0; q < NL; ++q) {
      const bool pad = lds_off[q] == (uint32_t)Q_DUMMY;
      const uint32_t dst = lds_base + lds_off[q] + (pad ? 0u : (uint32_t)((kt % Q_STAGES) * Q_STAGE));
      const int o = kt < kin_lim[q] ? (int)(off[q] + kstep[q] * (uint32_t)kt) : OOB;
      lds_void *d = (lds_void *)(uintptr_t)__builtin_amdgcn_readfirstlane(dst);
      const __amdgpu_buffer_rsrc_t rs = rsrc(rbase[q], rbytes[q]);
      if (q4_load_kind<KH>(q) == KGS)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, d, 4, o, 0, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, d, 16, o, 0, 0, 0);
    }
  };

  int zp16[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t m = m0 + wm * 32 + i * 16 + 4 * g4 + v;
      zp16[i][v] = m < M ? -16 * p.xz[m] : 0;
    }
  f32x4 f[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) f[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int kt) {
    const char *st = smem + (kt % Q_STAGES) * Q_STAGE;
#pragma unroll
    for (int x = 0; x < 4 / KH; ++x) {
      const int gg = kh + KH * x;  // group within the stage
      if (4 * kt + gg < G) {       // uniform: the last stage may hold fewer groups
        long fa[2], fb[2];
        float gsv[2];
        int gmv[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int R = wm * 32 + i * 16 + r;
          const int c = 2 * gg + (g4 >> 1);
          fa[i] = *reinterpret_cast<const long *>(st + R * 128 + 16 * (c ^ (R & 7)) + 8 * (g4 & 1));
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int R = wn * 32 + j * 16 + r;
          const uint32_t w = *reinterpret_cast<const uint32_t *>(st + QA_BYTES + R * 64 +
                                                                 16 * (gg ^ (R & 3)) + 4 * g4);
          fb[j] = unpack_q4x8(w);
          gsv[j] = *reinterpret_cast<const float *>(st + QA_BYTES + QB_BYTES + R * 16 + 4 * gg);
          gmv[j] = *reinterpret_cast<const int *>(st + QA_BYTES + QB_BYTES + QG_BYTES + R * 16 + 4 * gg);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const i32x4 t = __builtin_amdgcn_mfma_i32_16x16x32_i8(fa[i], fb[j], i32x4{0, 0, 0, 0}, 0, 0, 0);
#pragma unroll
            for (int v = 0; v < 4; ++v)  // |zp16| <= 2048, |gsum| <= 256: 24-bit product
              f[i][j][v] += gsv[j] * (float)(t[v] + __mul24(zp16[i][v], gmv[j]));
          }
      }
    }
  };

  const int nk = (int)((K + 127) / 128);
#pragma unroll
  for (int s = 0; s < Q_STAGES - 1; ++s) issue(s);
  int kt = 0;
  for (; kt < nk - (Q_STAGES - 1); ++kt) {
    __builtin_amdgcn_s_waitcnt(0x0F70 | (NL * (Q_STAGES - 2)));
    __builtin_amdgcn_s_barrier();
    issue(kt + Q_STAGES - 1);
    compute(kt);
    __builtin_amdgcn_s_waitcnt(0xC07F);
  }
#pragma unroll
  for (int t = 0; t < Q_STAGES - 1; ++t) {
    if (kt < nk) {
      if (t == 0) __builtin_amdgcn_s_waitcnt(0x0F70 | (NL * (Q_STAGES - 2)));
      else if (t == 1) __builtin_amdgcn_s_waitcnt(0x0F70 | (NL * (Q_STAGES - 3)));
      else __builtin_amdgcn_s_waitcnt(0x0F70);
      __builtin_amdgcn_s_barrier();
      compute(kt);
      __builtin_amdgcn_s_waitcnt(0xC07F);
    }
    ++kt;
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();

  // ---- sum the group halves (KH = 2), then stage the tile in LDS
  f32x4 *xch = reinterpret_cast<f32x4 *>(smem + TB * Q_TILE_LD * 4);
  if constexpr (KH == 2) {
    if (kh == 1) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) xch[((wave - 4) * 4 + i * 2 + j) * 64 + lane] = f[i][j];
    }
    __syncthreads();
  }
  float *tl = reinterpret_cast<float *>(smem);
  if (kh == 0) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        f32x4 v4 = f[i][j];
        if constexpr (KH == 2) v4 += xch[(wave * 4 + i * 2 + j) * 64 + lane];
        const int col = wn * 32 + j * 16 + r;
        const int64_t n = n0 + col;
        const float bv = (n < N && p.bias) ? p.bias[n] : 0.0f;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int row = wm * 32 + i * 16 + 4 * g4 + v;
          const int64_t m = m0 + row;
          const float xs = m < M ? p.xs[m] : 0.0f;
          tl[row * Q_TILE_LD + col] = xs * (v4[v] * 0.0625f) + bv;
        }
      }
  }
  __syncthreads();
  // 16 lanes x 16 B per row
  const bool vec = (N & 3) == 0;
  for (int u = tid; u < TB * 16; u += 256 * KH) {
    const int row = u >> 4, c = u & 15;
    const int64_t m = m0 + row, n = n0 + 4 * c;
    if (m >= M || n >= N) continue;
    const f32x4 val = *reinterpret_cast<const f32x4 *>(tl + row * Q_TILE_LD + 4 * c);
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

}  // namespace

hipError_t launch_dq8ca_q4(const Q4Args &a, hipStream_t st) {
  if (a.M <= 16) {
    // same launch-shape rule as the weight-only GEMV: 8-channel tiles for
    // M <= 2, 16 otherwise; waves per workgroup until ~768 wave-tiles
    const int MB = a.M <= 4 ? 1 : (a.M <= 8 ? 2 : 4);
    const int TG = a.M <= 2 ? 2 : 4;
    const int64_t nst = (a.K / 2 + 255) / 256;
    const int64_t tiles = (a.N + 4 * TG - 1) / (4 * TG);
    int W = 1;
    while (W < 8 && tiles * W < 768 && W * 4 <= nst) W <<= 1;
    const dim3 grid((unsigned)tiles, 1);
    if (TG == 2) launch_stream_tg<2>(MB, W, grid, a, st);
    else launch_stream_tg<4>(MB, W, grid, a, st);
  } else {
    const int tiles_m = (int)((a.M + TB - 1) / TB);
    const int tiles_n = (int)((a.N + TB - 1) / TB);
    const int64_t tiles = (int64_t)tiles_m * tiles_n;
    // split each stage's groups over two waves when there are too few tiles
    // to give every SIMD several waves
    if (tiles < 1024) {
      static bool attr2 = false;
      if (!attr2) {
        (void)hipFuncSetAttribute((const void *)k_dq8ca_q4_tiled<2>,
                                  hipFuncAttributeMaxDynamicSharedMemorySize, Q_LDS);
        (void)hipGetLastError();
        attr2 = true;
      }
      hipLaunchKernelGGL(k_dq8ca_q4_tiled<2>, dim3((unsigned)tiles), dim3(512), Q_LDS, st, a,
                         tiles_m, tiles_n);
    } else {
      static bool attr1 = false;
      if (!attr1) {
        (void)hipFuncSetAttribute((const void *)k_dq8ca_q4_tiled<1>,
                                  hipFuncAttributeMaxDynamicSharedMemorySize, Q_LDS);
        (void)hipGetLastError();
        attr1 = true;
      }
      hipLaunchKernelGGL(k_dq8ca_q4_tiled<1>, dim3((unsigned)tiles), dim3(256), Q_LDS, st, a,
                         tiles_m, tiles_n);
    }
  }
  return hipGetLastError();
}

}  // namespace aql
