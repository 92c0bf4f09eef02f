// Weight-only W8A16 linear for prefill-sized M (tiny-llm quant, Step 4.6):
// y[m, n] = scale[n] * sum_k x[m, k] * q[n, k] (+ bias[n]), bf16 in and out.
//
// The scale factors out of the sum and int8 -> bf16 is exact, so the sum runs
// on the bf16 matrix cores (v_mfma_f32_16x16x32_bf16, fp32 accumulation) with
// the weights widened in registers, and the scale is applied once per output.
//
// Tiles: on large grids 128 rows of x x 256 output channels per workgroup of 8
// waves side by side along N (k_w8a16_gemm_wide, below); otherwise BM (64 or
// 128) rows x 128 channels (k_w8a16_gemm): a group of waves covers the tile
// for one 64-k stage, (BM / 64) x 2 quadrants of 64 x 64 (4 x 4 MFMA tiles
// each) times 2 halves of the stage, and for the 64-row tile two such groups
// take alternate stages, which puts two waves on every SIMD (one wave's
// widening then overlaps the other's MFMAs). The partial fp32 accumulators
// are added once at the end.
// Operands go global -> LDS by buffer loads that write LDS directly (hardware
// zero-fill past M, N and K): x as bf16 rows of 128 B, the weights as int8 rows
// of 64 B (half the bytes of bf16; they are widened after the fragment read).
// A ring of stages (4 or 8; 2 for the wide tile on the largest grids) keeps
// the next stages in flight behind exact vmcnt waits and a fence-free barrier
// (a straight-line loop, so the compiler's wait counts stay exact); when K is
// a multiple of 64 the k advance of a load is a scalar offset. x rows store
// their 16-byte chunks XOR-swizzled by (row / 2) mod 8 and weight rows by
// (row / 4) mod 4, which makes every fragment read conflict-free.
// The output tile is staged in LDS as bf16 and written as whole rows.
#include <type_traits>

#include "common.h"
#include "w8a16_gemm.h"

namespace aql {
namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int BN = 128, BK = 64;
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

// s_waitcnt immediate that waits for vmcnt <= n (0..63: bits 3:0 and 15:14)
// and leaves the other counters alone.
constexpr int vmcnt_imm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

template <int I, int N, class F>
__device__ __forceinline__ void static_for(F &&f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

__device__ __forceinline__ int swz_x(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ int swz_w(int row) { return (row >> 2) & 3; }

// BM = 64 WM rows. A group of waves covers the tile for one 64-k stage: every
// wave of it computes 16 TI rows x 64 channels over one 32-k half of the stage,
// so a group has NG = (BM / 16 TI) x 2 x 2 waves. KP groups take consecutive
// stages (stage KP t + kp in step t), which puts KP waves on every SIMD to
// overlap one wave's weight widening with another's MFMAs; SG stages of LDS
// form the ring (SG / KP steps). The partial sums of the 2 KP waves that share
// an output block are added through LDS at the end.
template <int WM, int TI, int SG, int KP>
struct GemmLds {
  static constexpr int BM = 64 * WM;
  static constexpr int WMW = BM / (16 * TI);    // waves along M
  static constexpr int NG = 4 * WMW;            // waves per group
  static constexpr int NW = KP * NG;            // waves per workgroup
  static constexpr int PS = SG / KP;            // steps in the ring
  static constexpr int NXL = (BM / 8) / NG;     // x loads per wave per step
  static constexpr int NWL = 8 / NG;            // weight loads per wave per step
  static constexpr int XS = BM * 128;           // x stage: BM rows x 64 bf16
  static constexpr int WS = BN * 64;            // weight stage: 128 rows x 64 int8
  static constexpr int STAGE = XS + WS;
  static constexpr int RING = SG * STAGE;
  static constexpr int XCH = (NW - 2 * WMW) * TI * 4 * 64 * 16;  // partial sums to add
  static constexpr int TLD = BN + 8;            // bf16 per staged output row
  static constexpr int TILE = BM * TLD * 2;
  static constexpr int BYTES = RING > XCH + TILE ? RING : XCH + TILE;
  static_assert(NXL * NG == BM / 8 && NWL * NG == 8, "load slots split evenly");
  static_assert(SG % KP == 0 && PS >= 3, "ring of whole steps, one read ahead");
};

// RAG: K is not a multiple of 64, so the last stage is partial and every load
// checks its chunk against the row end; otherwise the k advance of a load is a
// uniform (scalar) offset and costs no vector instruction.
template <int WM, int TI, int SG, int KP, bool RAG>
__global__ __launch_bounds__((64 * GemmLds<WM, TI, SG, KP>::NW)) void k_w8a16_gemm(
    const uint16_t *__restrict__ x, const int8_t *__restrict__ q, const float *__restrict__ scale,
    const uint16_t *__restrict__ bias, uint16_t *__restrict__ y, int64_t M, int64_t N, int64_t K,
    int tiles_m, int tiles_n) {
  using L = GemmLds<WM, TI, SG, KP>;
  constexpr int BM = L::BM, NG = L::NG, NW = L::NW, PS = L::PS, NXL = L::NXL;
  constexpr int NL = L::NXL + L::NWL;
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int nt = tiles_m * tiles_n;
  const int lin = blockIdx.x;
  int tile = lin;
  if ((nt & 7) == 0) tile = (lin & 7) * (nt >> 3) + (lin >> 3);
  const int tn = tile / tiles_m, tm = tile % tiles_m;
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kp = wave / NG, wig = wave % NG;  // group, wave in group
  const int kh = wig / (2 * L::WMW), wm = (wig >> 1) % L::WMW, wn = wig & 1;
  const int r = lane & 15, g = lane >> 4;
  const int64_t mval = M - m0 < BM ? M - m0 : BM;
  const int64_t nval = N - n0 < BN ? N - n0 : BN;
  const __amdgpu_buffer_rsrc_t rx = rsrc(x + m0 * K, (uint32_t)(mval * K * 2));
  const __amdgpu_buffer_rsrc_t rq = rsrc(q + n0 * K, (uint32_t)(nval * K));

  // Each group loads the stages it computes. Loads per stage: BM/8 x-slots
  // (8 rows x 128 B) and 8 weight slots (16 rows x 64 B), NL per wave of the
  // group; load qq of every wave is of one kind: qq < NXL x-slot qq NG + wig,
  // else weight slot (qq - NXL) NG + wig.
  uint32_t off[NL], ldso[NL], kstep[NL];
  int kin_lim[NL];
#pragma unroll
  for (int qq = 0; qq < NL; ++qq) {
    if (qq < NXL) {
      const int slot = qq * NG + wig;
      const int row = 8 * slot + (lane >> 3), c = (lane & 7) ^ swz_x(row);
      off[qq] = (uint32_t)row * (uint32_t)(2 * K) + 16u * c;
      ldso[qq] = (uint32_t)(slot * 1024);
      kstep[qq] = 128;
      kin_lim[qq] = (int)((2 * K - 16 * c + 127) / 128);
    } else {
      const int slot = (qq - NXL) * NG + wig;
      const int row = 16 * slot + (lane >> 2), c = (lane & 3) ^ swz_w(row);
      off[qq] = (uint32_t)row * (uint32_t)K + 16u * c;
      ldso[qq] = (uint32_t)(L::XS + slot * 1024);
      kstep[qq] = 64;
      kin_lim[qq] = (int)((K - 16 * c + 63) / 64);
    }
  }
  const int nk = (int)((K + BK - 1) / BK);  // stages
  const uint32_t lds_base = (uint32_t)(uintptr_t)smem + (uint32_t)(kp * L::STAGE);
  // this group's stage of step t into ring slot `slot`; a stage past K loads
  // zeros (RAG) or stage 0 again, and its sums are skipped
  auto issue = [&](int t, int slot) {
    const int kt = KP * t + kp;
#pragma unroll
    for (int qq = 0; qq < NL; ++qq) {
      const uint32_t dst = lds_base + (uint32_t)(slot * KP * L::STAGE) + ldso[qq];
      int vo, so;
      if constexpr (RAG) {
        vo = kt < kin_lim[qq] ? (int)(off[qq] + kstep[qq] * (uint32_t)kt) : OOB;
        so = 0;
      } else {
        vo = (int)off[qq];
        so = kt < nk ? kt * (qq < NXL ? 128 : 64) : 0;
      }
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          qq < NXL ? rx : rq, (lds_void *)(uintptr_t)__builtin_amdgcn_readfirstlane(dst), 16, vo,
          so, 0, 0);
    }
  };

  // fragment offsets within a stage
  int fxo[TI], fwo[4];
#pragma unroll
  for (int i = 0; i < TI; ++i) {
    const int R = wm * 16 * TI + i * 16 + r;
    fxo[i] = kp * L::STAGE + R * 128 + 16 * ((4 * kh + g) ^ swz_x(R));
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int S = wn * 64 + j * 16 + r;
    fwo[j] = kp * L::STAGE + L::XS + S * 64 + 16 * ((2 * kh + (g >> 1)) ^ swz_w(S)) + 8 * (g & 1);
  }

  f32x4 acc[TI][4];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Software pipeline, one step deep: step t reads stage t + 1's fragments
  // from LDS and widens its weights between the MFMAs of stage t (whose
  // operands were made ready in step t - 1), so the VALU work of the widening
  // issues while the matrix core runs.
  struct Frag {
    bf16x8 a[TI];
    bf16x8 b[4];
  };
  i32x2 wr[4];
  auto read = [&](int slot, Frag &f) {
    const char *st = smem + slot * KP * L::STAGE;
#pragma unroll
    for (int i = 0; i < TI; ++i) f.a[i] = *reinterpret_cast<const bf16x8 *>(st + fxo[i]);
#pragma unroll
    for (int j = 0; j < 4; ++j) wr[j] = *reinterpret_cast<const i32x2 *>(st + fwo[j]);
  };
  auto widen = [&](Frag &f) {
#pragma unroll
    for (int j = 0; j < 4; ++j) f.b[j] = widen8((uint32_t)wr[j][0], (uint32_t)wr[j][1]);
  };
  auto mma = [&](const Frag &f) {
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
  };
  // interleave: the fragment reads first, then one MFMA per 3 VALU ops
  auto interleave = [&]() {
    __builtin_amdgcn_sched_group_barrier(0x100, TI + 4, 0);  // DS reads
#pragma unroll
    for (int u = 0; u < 4 * TI; ++u) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // VALU
    }
  };

  // steps of KP stages (a stage past K loads zeros and adds nothing)
  const int ns = (int)((K + KP * BK - 1) / (KP * BK));
#pragma unroll
  for (int t = 0; t < PS - 1; ++t) issue(t, t);
  Frag cur, nxt;
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(NL * (PS - 2)));
  __builtin_amdgcn_s_barrier();  // step 0 complete everywhere
  read(0, cur);
  widen(cur);
  int ts = 0;
  // Step t: stage t + 1 must have landed (the loads of steps up to t + PS - 2
  // are out, so at most NL (PS - 3) of this wave's may stay outstanding), and
  // the slot refilled is that of step t - 1, whose fragments every wave has
  // consumed before this barrier. u = t mod PS.
  auto step = [&](int t, int u) {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(NL * (PS - 3)));
    __builtin_amdgcn_s_barrier();
    issue(t + PS - 1, (u + PS - 1) % PS);
    read((u + 1) % PS, nxt);
    mma(cur);
    widen(nxt);
    interleave();
    cur = nxt;
  };
  // whole turns of the ring first: each step's LDS offsets become constants
  const int nmain = ns - (PS - 1);
  for (; ts + PS - 1 < nmain; ts += PS)
    static_for<0, PS>([&](auto u) { step(ts + decltype(u)::value, decltype(u)::value); });
  for (; ts < nmain; ++ts) step(ts, ts % PS);
  // the last PS - 1 steps: nothing more is issued; the last loads were those
  // of step ns - 1, so stage ts + 1 has landed with at most NL (ns - 2 - ts)
  // of this wave's loads outstanding
  static_for<0, PS - 1>([&](auto u) {
    constexpr int left = PS - 3 - decltype(u)::value;
    if (ts < ns) {
      if (ts + 1 < ns) {  // (only the last step can hold a stage past K)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(NL * (left > 0 ? left : 0)));
        __builtin_amdgcn_s_barrier();
        read((ts + 1) % PS, nxt);
        mma(cur);
        widen(nxt);
        interleave();
      } else if (KP * ts + kp < nk) {
        mma(cur);
      }
      cur = nxt;
    }
    ++ts;
  });
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();

  // ---- add the partial sums, then scale + bias + bf16 into the LDS output
  // tile. acc[i][j] lane holds D[4g + v][r] of MFMA tile (i, j): row m, column
  // n. Partner p = 2 kp + kh (1 .. 2 KP - 1) of output block b = 2 wm + wn
  // writes slot (p - 1) 2 WMW + b; partner 0 adds them in the order of p.
  f32x4 *xch = reinterpret_cast<f32x4 *>(smem);
  const int part = 2 * kp + kh, blk = 2 * wm + wn;
  if (part != 0) {
    const int slot = (part - 1) * 2 * L::WMW + blk;
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) xch[(slot * 4 * TI + i * 4 + j) * 64 + lane] = acc[i][j];
  }
  __syncthreads();
  uint16_t *tl = reinterpret_cast<uint16_t *>(smem + L::XCH);
  if (part == 0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = wn * 64 + j * 16 + r;
      const int64_t n = n0 + col;
      const float s = n < N ? scale[n] : 0.0f;
      const float b = (n < N && bias) ? bf16_to_f32(bias[n]) : 0.0f;
#pragma unroll
      for (int i = 0; i < TI; ++i) {
        f32x4 v4 = acc[i][j];
#pragma unroll
        for (int pp = 1; pp < 2 * KP; ++pp)
          v4 += xch[(((pp - 1) * 2 * L::WMW + blk) * 4 * TI + i * 4 + j) * 64 + lane];
#pragma unroll
        for (int v = 0; v < 4; ++v)
          tl[(wm * 16 * TI + i * 16 + 4 * g + v) * L::TLD + col] = f32_to_bf16_rne(s * v4[v] + b);
      }
    }
  }
  __syncthreads();
  // 16 lanes x 16 B per 256-byte row
  const bool vec = (N & 7) == 0;
  for (int u = tid; u < BM * 16; u += 64 * NW) {
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
  static constexpr int TLDF = BNW + 4;          // fp32 per staged partial-sum row (split K)
  static constexpr int TILEF = BM * TLDF * 4;
  static constexpr int BYTES_SPLIT = RING > TILEF ? RING : TILEF;
};

// SG = 4: a 4-stage ring, one workgroup a CU. SG = 2: a 2-stage ring in
// 64 KB, so two workgroups share a CU and each covers the other's waits at
// the stage barrier (from 512 tiles on, where every CU gets two).
//
// SPLIT: the grid is tiles x S units, unit (tile, sp) taking the ks stages of
// 64 k from sp * ks (a multiple of SG); it writes its fp32 partial sums, before
// any scale, to part[sp][M][N], which k_w8a16_splitk_reduce adds. This serves
// the grids of few tiles and long rows (M = 512, K = 14336, N = 4096: 64 tiles
// of 4 x 3584 k instead of 256 tiles of 64 x 128 over the whole row), where
// every CU otherwise streams the whole of K for a small tile: the operand
// bytes per CU halve.
template <int SG, bool SPLIT>
__global__ __launch_bounds__(512, SG == 2 ? 4 : 2) void k_w8a16_gemm_wide(const uint16_t *__restrict__ x,
                                                         const int8_t *__restrict__ q,
                                                         const float *__restrict__ scale,
                                                         const uint16_t *__restrict__ bias,
                                                         uint16_t *__restrict__ y, int64_t M,
                                                         int64_t N, int64_t K, int tiles_m,
                                                         int tiles_n, float *__restrict__ part,
                                                         int ks) {
  using L = WideLds<SG>;
  constexpr int BM = L::BM, BNW = L::BNW, NL = 4;  // loads per wave per stage
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int nt = tiles_m * tiles_n;
  const int nu = (int)gridDim.x;  // nt tiles x (nu / nt) splits of K
  const int lin = blockIdx.x;
  int unit = lin;
  if ((nu & 7) == 0) unit = (lin & 7) * (nu >> 3) + (lin >> 3);
  const int tile = unit % nt, sp = unit / nt;
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

  const int nk_all = (int)((K + BK - 1) / BK);
  const int k0 = SPLIT ? sp * ks : 0;  // stages [k0, nk) of this unit
  const int nk = SPLIT ? (k0 + ks < nk_all ? k0 + ks : nk_all) : nk_all;
#pragma unroll
  for (int s = 0; s < SG - 1; ++s) issue(k0 + s);
  int kt = k0;
  auto step = [&](int k) {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(NL * (SG - 2)));
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
      if (t == 0) __builtin_amdgcn_s_waitcnt(vmcnt_imm(NL * (SG - 2)));
      else if (t == 1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(SG > 3 ? NL * (SG - 3) : 0));
      else __builtin_amdgcn_s_waitcnt(0x0F70);
      __builtin_amdgcn_s_barrier();
      compute(kt);
      __builtin_amdgcn_s_waitcnt(0xC07F);
    }
    ++kt;
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();

  if constexpr (SPLIT) {
    // the partial sums through LDS, then whole rows of 1 KB: 64 lanes x 16 B
    float *tf = reinterpret_cast<float *>(smem);
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) tf[(i * 16 + 4 * g + v) * L::TLDF + wn * 32 + j * 16 + r] = acc[i][j][v];
    __syncthreads();
    const bool vec4 = (N & 3) == 0;
    float *pb = part + (int64_t)sp * M * N;
    for (int u = tid; u < BM * 64; u += 512) {
      const int row = u >> 6, c = u & 63;
      const int64_t m = m0 + row, n = n0 + 4 * c;
      if (m >= M || n >= N) continue;
      const f32x4 val = *reinterpret_cast<const f32x4 *>(tf + row * L::TLDF + 4 * c);
      float *dst = pb + m * N + n;
      if (vec4) {
        *reinterpret_cast<f32x4 *>(dst) = val;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (n + e < N) dst[e] = val[e];
      }
    }
    return;
  }

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

// y[m, n] = bf16(scale[n] (part[0][m][n] + ... + part[S-1][m][n]) + bias[n]),
// the sum in split order; a thread takes 4 consecutive outputs of a row (one
// 16-byte load per split: 4.4 us for S = 4 at M = 512, N = 4096, against 9.5
// with 8 outputs a thread).
__global__ __launch_bounds__(256) void k_w8a16_splitk_reduce(const float *__restrict__ part, int S,
                                                            int64_t M, int64_t N,
                                                            const float *__restrict__ scale,
                                                            const uint16_t *__restrict__ bias,
                                                            uint16_t *__restrict__ y) {
  const int64_t ng = (N + 3) / 4;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= M * ng) return;
  const int64_t m = i / ng, n = (i % ng) * 4;
  const int cnt = N - n < 4 ? (int)(N - n) : 4;
  const bool vec = (N & 3) == 0;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if (vec && S <= 4) {
    // all the splits' loads in flight before the first add (same order of sums)
    f32x4 v[4];
#pragma unroll
    for (int s = 0; s < 4; ++s)
      v[s] = s < S ? __builtin_nontemporal_load(
                         reinterpret_cast<const f32x4 *>(part + ((int64_t)s * M + m) * N + n))
                   : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s)
      if (s < S) acc += v[s];
  } else {
    for (int s = 0; s < S; ++s) {
      const float *src = part + ((int64_t)s * M + m) * N + n;
      if (vec) {
        acc += *reinterpret_cast<const f32x4 *>(src);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (e < cnt) acc[e] += src[e];
      }
    }
  }
  uint16_t out[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int64_t nn = n + (e < cnt ? e : 0);
    const float b = bias ? bf16_to_f32(bias[nn]) : 0.0f;
    out[e] = f32_to_bf16_rne(scale[nn] * acc[e] + b);
  }
  uint16_t *dst = y + m * N + n;
  if (vec) {
    *reinterpret_cast<uint2 *>(dst) = *reinterpret_cast<const uint2 *>(out);
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (e < cnt) dst[e] = out[e];
  }
}

}  // namespace

hipError_t launch_w8a16_splitk_reduce(const float *part, int S, int64_t M, int64_t N,
                                      const float *scale, const uint16_t *bias, uint16_t *y,
                                      hipStream_t st) {
  const int64_t groups = M * ((N + 3) / 4);
  hipLaunchKernelGGL(k_w8a16_splitk_reduce, dim3((unsigned)((groups + 255) / 256)), dim3(256), 0,
                     st, part, S, M, N, scale, bias, y);
  return hipGetLastError();
}

namespace {

template <int SG>
hipError_t launch_wide(const uint16_t *x, int64_t M, int64_t K, const int8_t *q, const float *scale,
                       const uint16_t *bias, int64_t N, uint16_t *y, hipStream_t st) {
  using L = WideLds<SG>;
  static bool attr_set = false;
  if (!attr_set) {  // more than 64 KB of dynamic LDS; a launch the limit refuses reports itself
    (void)hipFuncSetAttribute((const void *)k_w8a16_gemm_wide<SG, false>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, L::BYTES);
    (void)hipGetLastError();
    attr_set = true;
  }
  const int tiles_m = (int)((M + L::BM - 1) / L::BM), tiles_n = (int)((N + L::BNW - 1) / L::BNW);
  hipLaunchKernelGGL((k_w8a16_gemm_wide<SG, false>), dim3((unsigned)(tiles_m * tiles_n)), dim3(512),
                     L::BYTES, st, x, q, scale, bias, y, M, N, K, tiles_m, tiles_n, nullptr, 0);
  return hipGetLastError();
}

// The wide tile over S splits of K into part (S M N floats), then the sum.
hipError_t launch_wide_split(const uint16_t *x, int64_t M, int64_t K, const int8_t *q,
                             const float *scale, const uint16_t *bias, int64_t N, uint16_t *y,
                             float *part, int S, hipStream_t st) {
  constexpr int SG = 4;
  using L = WideLds<SG>;
  static bool attr_set = false;
  if (!attr_set) {
    (void)hipFuncSetAttribute((const void *)k_w8a16_gemm_wide<SG, true>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, L::BYTES_SPLIT);
    (void)hipGetLastError();
    attr_set = true;
  }
  const int tiles_m = (int)((M + L::BM - 1) / L::BM), tiles_n = (int)((N + L::BNW - 1) / L::BNW);
  const int nk = (int)((K + BK - 1) / BK);
  int ks = (nk + S - 1) / S;
  ks = (ks + SG - 1) / SG * SG;  // whole turns of the ring
  const int splits = (nk + ks - 1) / ks;
  hipLaunchKernelGGL((k_w8a16_gemm_wide<SG, true>), dim3((unsigned)(tiles_m * tiles_n * splits)),
                     dim3(512), L::BYTES_SPLIT, st, x, q, scale, bias, y, M, N, K, tiles_m,
                     tiles_n, part, ks);
  return launch_w8a16_splitk_reduce(part, splits, M, N, scale, bias, y, st);
}

template <int WM, int TI, int SG, int KP, bool RAG>
hipError_t launch_wm_k(const uint16_t *x, int64_t M, int64_t K, const int8_t *q, const float *scale,
                     const uint16_t *bias, int64_t N, uint16_t *y, hipStream_t st) {
  using L = GemmLds<WM, TI, SG, KP>;
  static bool attr_set = false;
  if (!attr_set) {  // more than 64 KB of dynamic LDS; a launch the limit refuses reports itself
    (void)hipFuncSetAttribute((const void *)k_w8a16_gemm<WM, TI, SG, KP, RAG>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, L::BYTES);
    (void)hipGetLastError();
    attr_set = true;
  }
  const int tiles_m = (int)((M + L::BM - 1) / L::BM), tiles_n = (int)((N + BN - 1) / BN);
  hipLaunchKernelGGL((k_w8a16_gemm<WM, TI, SG, KP, RAG>), dim3((unsigned)(tiles_m * tiles_n)),
                     dim3(64 * L::NW), L::BYTES, st, x, q, scale, bias, y, M, N, K, tiles_m,
                     tiles_n);
  return hipGetLastError();
}

template <int WM, int TI, int SG, int KP>
hipError_t launch_wm(const uint16_t *x, int64_t M, int64_t K, const int8_t *q, const float *scale,
                     const uint16_t *bias, int64_t N, uint16_t *y, hipStream_t st) {
  if (K % BK == 0) return launch_wm_k<WM, TI, SG, KP, false>(x, M, K, q, scale, bias, N, y, st);
  return launch_wm_k<WM, TI, SG, KP, true>(x, M, K, q, scale, bias, N, y, st);
}

}  // namespace

int w8a16_gemm_splits(int64_t M, int64_t N, int64_t K) {
  const int64_t twide = ((M + 127) / 128) * ((N + 255) / 256);
  const int64_t nk = (K + BK - 1) / BK;
  if (twide >= 160 || nk < 128) return 1;
  int S = 1;
  while (S < 16 && twide * 2 * S <= 256 && nk / (2 * S) >= 16) S *= 2;
  return S;
}

size_t w8a16_gemm_part_bytes(int64_t M, int64_t N, int64_t K) {
  const int S = w8a16_gemm_splits(M, N, K);
  return S > 1 ? (size_t)S * (size_t)M * (size_t)N * 4 : 0;
}

// Few wide tiles and long rows (a workspace given): the wide tile over K
// splits, then the sum (M = 512, N = 4096, K = 14336: 76 vs 89 us; M = 128:
// 37 vs 82 us; rotated weights). Else 128 x 256 tiles from 160 of them on
// (fewer than one per CU still beats the smaller tiles' extra round), two
// workgroups a CU from 512 on; else 128 x 128 tiles when those fill the CUs,
// else 64 x 128 tiles with two stage groups and an 8-stage ring (measured at
// M = 512, K = 14336, N = 4096: 74 us against 95 us for one group of 4 waves).
hipError_t launch_w8a16_gemm(const uint16_t *x, int64_t M, int64_t K, const int8_t *q,
                             const float *scale, const uint16_t *bias, int64_t N, uint16_t *y,
                             float *part, size_t part_bytes, hipStream_t st) {
  const int S = w8a16_gemm_splits(M, N, K);
  if (S > 1 && part && part_bytes >= w8a16_gemm_part_bytes(M, N, K))
    return launch_wide_split(x, M, K, q, scale, bias, N, y, part, S, st);
  const int64_t twide = ((M + 127) / 128) * ((N + 255) / 256);
  if (twide >= 512) return launch_wide<2>(x, M, K, q, scale, bias, N, y, st);
  if (twide >= 160) return launch_wide<4>(x, M, K, q, scale, bias, N, y, st);
  const int64_t t128 = ((M + 127) / 128) * ((N + BN - 1) / BN);
  if (t128 >= 256) return launch_wm<2, 4, 4, 1>(x, M, K, q, scale, bias, N, y, st);
  return launch_wm<1, 4, 8, 2>(x, M, K, q, scale, bias, N, y, st);
}

}  // namespace aql
