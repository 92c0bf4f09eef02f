// GPTQ int8 on the device, in binary64.
//
// SmolVLM q8 recipe, gptq_int8 (after Frantar et al.): with the weight
// quantizer's per-channel scales (amax / 127.5 of the original weight), the
// Hessian's dead columns (zero diagonal) get a unit diagonal and a zeroed weight
// column, the diagonal is damped by damp * mean(diag H), and hinv is the upper
// Cholesky factor of H^-1 (formed as chol(chol_inverse(chol(H)))). Columns are
// then rounded in order, block by block; each column's rounding error, divided
// by hinv[i][i], is pushed onto the block's later columns through hinv's row i,
// and a finished block's errors onto all later columns through hinv's rows.
//
// The page leaves the order of its library reductions open. Here every sum
// (a Cholesky element, an element of the triangular inverse, of X^T X, of a
// block's trailing update, and the mean of the diagonal) is a plain ascending
// sum from 0 with each product and addition rounded on its own, subtracted or
// used once complete. The kernels get parallelism from independent elements
// only: a sum is never split or reassociated. The factorizations are blocked
// right-looking ones (32-column panels, one wave each; trailing updates
// gathered over 128 columns) that keep each element's partial sum in an
// accumulator matrix between launches, so the order per element stays
// ascending. The O(K^3) and O(N K^2) parts run in one tiled fp64 kernel
// (k_seqdot: up to 128 x 128 tiles, up to 8 x 8 sums a thread, operands staged
// through LDS). Zero products entering a sum (the structural zeros of the
// triangular factors, padding past a range) leave it unchanged: an accumulator
// that starts at +0 never becomes -0, and x + (+-0) = x for x != 0.
//
// fp64 division and square root are IEEE-correctly rounded; nothing is
// contracted into a fused multiply-add.
#include "gptq.h"

#include <math.h>

#include "aql.h"
#include "quant.h"

#pragma clang fp contract(off)

namespace aql {
namespace {

typedef double f64x2 __attribute__((ext_vector_type(2)));

constexpr int PB = 32;        // panel width of the factorizations
constexpr int SB = 128;       // columns whose trailing update is applied at once
constexpr int TKC = 16;       // k_seqdot: k per LDS stage

inline size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

// p[e] where ok, else `other`. The load itself is unconditional (from p[0] when
// !ok), so unrolled loops issue their loads back to back instead of waiting
// after each branch-guarded one.
__device__ __forceinline__ double ld_or(const double *p, int64_t e, bool ok, double other) {
  const double v = p[ok ? e : 0];
  return ok ? v : other;
}

struct GptqWs {
  double *A;    // damped Hessian, later X^T X (lower triangle)
  double *acc;  // per-element partial sums of a factorization
  double *L;    // Cholesky factor (lower), first of H, then of H^-1
  double *X;    // L^-1 stored transposed (X[j][k] = (L^-1)[k][j]), later hinv (upper)
  double *W;    // working copy of the weight rows
  double *E;    // a block's scaled rounding errors [N, block]
  uint8_t *dead;
};

GptqWs carve(void *ws, int64_t N, int64_t K, int64_t block) {
  char *p = static_cast<char *>(ws);
  const size_t kk = align256(sizeof(double) * K * K);
  GptqWs r;
  r.A = reinterpret_cast<double *>(p);
  r.acc = reinterpret_cast<double *>(p + kk);
  r.L = reinterpret_cast<double *>(p + 2 * kk);
  r.X = reinterpret_cast<double *>(p + 3 * kk);
  p += 4 * kk;
  r.W = reinterpret_cast<double *>(p);
  p += align256(sizeof(double) * N * K);
  r.E = reinterpret_cast<double *>(p);
  p += align256(sizeof(double) * N * block);
  r.dead = reinterpret_cast<uint8_t *>(p);
  return r;
}

// ------------------------------------------------------------ small kernels

__global__ __launch_bounds__(256) void k_fill_f64(double *p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    p[i] = 0.0;
}

// A = lower triangle of H; a zero diagonal entry marks a dead column and becomes 1.
__global__ __launch_bounds__(256) void k_gptq_prep(const double *__restrict__ H, int64_t K,
                                                   double *__restrict__ A,
                                                   uint8_t *__restrict__ dead) {
  for (int64_t r = blockIdx.x; r < K; r += gridDim.x) {
    for (int64_t c = threadIdx.x; c <= r; c += 256) {
      double v = H[r * K + c];
      if (c == r) {
        const bool d = v == 0.0;
        dead[r] = d;
        if (d) v = 1.0;
      }
      A[r * K + c] = v;
    }
  }
}

// diag(A) += damp * (sum_k A[k][k] / K), the sum ascending; clears info.
__global__ __launch_bounds__(256) void k_gptq_damp(double *A, int64_t K, double damp,
                                                   int32_t *info) {
  __shared__ double d[2048];
  __shared__ double c_sh;
  double sum = 0.0;
  for (int64_t base = 0; base < K; base += 2048) {
    const int n = (int)(K - base < 2048 ? K - base : 2048);
    for (int i = threadIdx.x; i < n; i += 256) d[i] = A[(base + i) * (K + 1)];
    __syncthreads();
    if (threadIdx.x == 0)
      for (int i = 0; i < n; ++i) sum = sum + d[i];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    c_sh = damp * (sum / (double)K);
    *info = 0;
  }
  __syncthreads();
  const double c = c_sh;
  for (int64_t k = threadIdx.x; k < K; k += 256) A[k * (K + 1)] = A[k * (K + 1)] + c;
}

// W = w with the dead columns zeroed, in binary64.
__global__ __launch_bounds__(256) void k_gptq_wcopy(const float *__restrict__ w, int64_t N,
                                                    int64_t K, const uint8_t *__restrict__ dead,
                                                    double *__restrict__ W) {
  for (int64_t n = blockIdx.x; n < N; n += gridDim.x)
    for (int64_t k = threadIdx.x; k < K; k += 256)
      W[n * K + k] = dead[k] ? 0.0 : (double)w[n * K + k];
}

// hinv[i][j] = L[j][i] for j >= i, 0 below the diagonal (64 x 64 tiles through LDS).
__global__ __launch_bounds__(256) void k_gptq_upper_of(const double *__restrict__ L, int64_t K,
                                                       double *__restrict__ hinv) {
  __shared__ double t[64][65];
  const int64_t bi = (int64_t)blockIdx.x * 64, bj = (int64_t)blockIdx.y * 64;
  const int c = threadIdx.x & 63, r4 = threadIdx.x >> 6;
  // tile of L rows bj.., columns bi..
  for (int r = r4; r < 64; r += 4) {
    const int64_t lr = bj + r, lc = bi + c;
    t[r][c] = (lr < K && lc < K && lc <= lr) ? L[lr * K + lc] : 0.0;
  }
  __syncthreads();
  for (int r = r4; r < 64; r += 4) {
    const int64_t i = bi + r, j = bj + c;
    if (i < K && j < K) hinv[i * K + j] = t[c][r];
  }
}

// -------------------------------------------------------- panel kernels

__device__ __forceinline__ double readlane_f64(double v, int l) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// One 32-column panel [k0, k0 + bn) of the lower Cholesky factor L of A, in
// one wave. acc[i][j] holds sum_{k < k0} L[i][k] L[j][k] (ascending k) from the
// earlier panels' updates. Every workgroup factors the diagonal block (lane t
// holds row t & 31); workgroup 0 stores it, workgroup g >= 1 also solves rows
// k0 + 32 + 64 (g - 1) .. + 63 of the panel (lane t, row t) in the same steps:
// step k needs only column k of the block, so the two solves' divisions
// overlap. Both are right-looking: at step k the new column k of L adds its
// term k to every later element's running sum, so each sum still runs over k
// in ascending order. The block's column k goes through LDS, column-major
// (Lc[k][j] = L[j][k]): the wave writes it and reads it back (LDS serves one
// wave's accesses in order). Past the matrix the diagonal block is padded
// with an identity, which keeps the padded pivots at 1.
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_chol_panel(
    const double *__restrict__ A, const double *__restrict__ acc, double *__restrict__ L,
    int64_t K, int64_t k0, int32_t *info, int32_t code0) {
  __shared__ double Da[PB][PB + 1];                          // diagonal block of A (row-major)
  __shared__ double Dc[PB][PB + 1];                          // ... of acc
  __shared__ __attribute__((aligned(16))) double Lc[PB][PB];  // ... of L, column-major
  __shared__ double R[64][PB + 1];                           // this workgroup's rows of A
  __shared__ double S[64][PB + 1];                           // ... of acc
  const int t = threadIdx.x, tr = t & (PB - 1);
  const int bn = (int)(K - k0 < PB ? K - k0 : PB);
  constexpr int DM = PB * PB / 64;  // diagonal-block elements a thread stages
  const bool rows = blockIdx.x > 0;
  const int64_t r0 = k0 + PB + (int64_t)(blockIdx.x - 1) * 64;
  {
    // all loads first, then the selects (the unrolled code keeps source order);
    // workgroup 0 has no rows and reads element 0 in their place
    double va[DM], vc[DM], ra[PB], rc[PB];
#pragma unroll
    for (int m = 0; m < DM; ++m) {
      const int r = m * (64 / PB) + t / PB;
      const int64_t e = r < bn && tr <= r ? (k0 + r) * K + k0 + tr : 0;
      va[m] = A[e];
      vc[m] = acc[e];
    }
#pragma unroll
    for (int m = 0; m < PB; ++m) {
      const int r = m * (64 / PB) + t / PB;
      const int64_t e = rows && r0 + r < K ? (r0 + r) * K + k0 + tr : 0;
      ra[m] = A[e];
      rc[m] = acc[e];
    }
#pragma unroll
    for (int m = 0; m < DM; ++m) {
      const int r = m * (64 / PB) + t / PB;
      const bool ok = r < bn && tr <= r;
      Da[r][tr] = ok ? va[m] : (r == tr ? 1.0 : 0.0);
      Dc[r][tr] = ok ? vc[m] : 0.0;
    }
#pragma unroll
    for (int m = 0; m < PB; ++m) {
      const int r = m * (64 / PB) + t / PB;
      const bool ok = rows && r0 + r < K;
      R[r][tr] = ok ? ra[m] : 0.0;
      S[r][tr] = ok ? rc[m] : 0.0;
    }
  }
  __syncthreads();

  // sd[j]: running sum of diagonal-block element (tr, j); sr[j]: of element
  // (r0 + t, j). Each step's updates are pinned to that step: left free, the
  // compiler defers them to where the sums are next read and holds every
  // column in registers meanwhile.
  double sd[PB], sr[PB];
#pragma unroll
  for (int j = 0; j < PB; ++j) {
    sd[j] = Dc[tr][j];
    sr[j] = S[t][j];
  }
  int bad = 0;
#pragma unroll
  for (int k = 0; k < PB; ++k) {
    const double d = readlane_f64(Da[tr][k], k) - readlane_f64(sd[k], k);
    const bool fail = (k < bn) & !(d > 0.0);
    bad = ((bad == 0) & fail) ? code0 + k + 1 : bad;
    const double lkk = sqrt(d);
    const double below = (Da[tr][k] - sd[k]) / lkk;
    const double lrow = (R[t][k] - sr[k]) / lkk;
    const double l = tr == k ? lkk : below;
    Lc[k][tr] = l;  // lanes t and t + 32 store the same value
    R[t][k] = lrow;  // the new value replaces the element of A it came from
    double col[PB];
#pragma unroll
    for (int p = (k + 1) / 2; p < PB / 2; ++p) {
      const f64x2 v = *reinterpret_cast<const f64x2 *>(&Lc[k][2 * p]);
      col[2 * p] = v.x;
      col[2 * p + 1] = v.y;
    }
#pragma unroll
    for (int j = k + 1; j < PB; ++j) {
      sd[j] = sd[j] + l * col[j];
      sr[j] = sr[j] + lrow * col[j];
      asm volatile("" : "+v"(sd[j]), "+v"(sr[j]));  // the updates happen in this step
    }
  }
  if (info && bad && t == 0) atomicCAS(info, 0, bad);
  if (!rows) {
    if (t < bn) {
#pragma unroll
      for (int c = 0; c < PB; ++c)
        if (c < bn) L[(k0 + t) * K + k0 + c] = c <= t ? Lc[c][t] : 0.0;
    }
    return;
  }
  __syncthreads();
  for (int r = t / PB; r < 64; r += 64 / PB)
    if (r0 + r < K && tr < bn) L[(r0 + r) * K + k0 + tr] = R[r][tr];
}

// Rows [k0, k0 + bn) of Xm = L^-1, one lane a column j < k0 + bn:
// Xm[i][j] = 1 / L[i][i] (i == j), -(sum_{k=j}^{i-1} L[i][k] Xm[k][j]) / L[i][i]
// (i > j), 0 (i < j). acc[i][j] holds the sum over k < k0 (the terms with k < j
// are zero). Right-looking: Xm[k][j] adds its term to rows i > k at step k.
// L's diagonal block sits in LDS column-major; column i + 1 is read while step
// i computes. Stored transposed: X[j][i] = Xm[i][j].
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_trinv_panel(
    const double *__restrict__ L, const double *__restrict__ acc, double *__restrict__ X,
    int64_t K, int64_t k0) {
  __shared__ __attribute__((aligned(16))) double Lc[PB][PB];  // Lc[i][r] = L[k0 + r][k0 + i]
  __shared__ double V[PB][65];                                // [i][t]: Xm[k0 + i][j]
  const int t = threadIdx.x, tr = t & (PB - 1);
  const int bn = (int)(K - k0 < PB ? K - k0 : PB);
  const int64_t k1 = k0 + bn;
  const int64_t jb = (int64_t)blockIdx.x * 64, j = jb + t;
  // row tr of the diagonal block (identity past the matrix) and this column's
  // partial sums: all loads first (the unrolled code keeps source order)
  double ld[PB], sv[PB];
#pragma unroll
  for (int c = 0; c < PB; ++c) ld[c] = L[tr < bn && c <= tr ? (k0 + tr) * K + k0 + c : 0];
#pragma unroll
  for (int r = 0; r < PB; ++r) sv[r] = acc[r < bn && j < k1 ? (k0 + r) * K + j : 0];
#pragma unroll
  for (int c = 0; c < PB; ++c) ld[c] = tr < bn && c <= tr ? ld[c] : (c == tr ? 1.0 : 0.0);
#pragma unroll
  for (int r = 0; r < PB; ++r) sv[r] = r < bn && j < k1 ? sv[r] : 0.0;
  if (t < PB) {
#pragma unroll
    for (int c = 0; c < PB; ++c) Lc[c][tr] = ld[c];
  }
  __syncthreads();
  double col[2][PB];
#pragma unroll
  for (int p = 0; p < PB / 2; ++p) {
    const f64x2 v = *reinterpret_cast<const f64x2 *>(&Lc[0][2 * p]);
    col[0][2 * p] = v.x;
    col[0][2 * p + 1] = v.y;
  }
#pragma unroll
  for (int i = 0; i < PB; ++i) {
    if (i + 1 < PB) {
#pragma unroll
      for (int p = (i + 1) / 2; p < PB / 2; ++p) {
        const f64x2 v = *reinterpret_cast<const f64x2 *>(&Lc[i + 1][2 * p]);
        col[(i + 1) & 1][2 * p] = v.x;
        col[(i + 1) & 1][2 * p + 1] = v.y;
      }
    }
    const int64_t gi = k0 + i;
    const double v = (gi == j ? 1.0 : -sv[i]) / col[i & 1][i];
    const double x = gi < j ? 0.0 : v;
    V[i][t] = x;
#pragma unroll
    for (int r = i + 1; r < PB; ++r) sv[r] = sv[r] + col[i & 1][r] * x;
    __builtin_amdgcn_sched_barrier(0);  // keep the column reads one step ahead, no further
  }
  __syncthreads();
  for (int r = t / PB; r < 64; r += 64 / PB)
    if (jb + r < k1 && tr < bn) X[(jb + r) * K + k0 + tr] = V[tr][r];
}

// ------------------------------------------------------- ordered fp64 tiles

enum { SEQ_STORE = 0, SEQ_CONT = 1, SEQ_SUB = 2 };

// For rows i in [i0, i1) and columns j in [j0, j1) (LOWER: j <= i only):
//   s = sum over k in [kb, ke), ascending, of P[i][k] * Q[j][k]
// accumulated one rounded product and one rounded addition at a time, starting
// from 0 (SEQ_STORE: out = s; SEQ_SUB: out = out - s) or from out itself
// (SEQ_CONT: the sum carries on from the value stored). KFROM_ROW starts a
// tile's sum at max(kb, its first row), for products whose terms vanish for
// k < i. P[i][k] is at P[i * ldp + k], Q[j][k] at Q[j * ldq + k], out[i][j] at
// out[i * ldo + j]. 256 threads as 16 x 16, each TI x TJ sums: a 16 TI x 16 TJ
// tile (128 x 128 for large grids, smaller ones so that narrow or late updates
// still spread over the chip).
template <int MODE, bool LOWER, bool KFROM_ROW, int TI, int TJ>
__global__ __launch_bounds__(256, 2) void k_seqdot(const double *__restrict__ P, int64_t ldp,
                                                   const double *__restrict__ Q, int64_t ldq,
                                                   double *__restrict__ out, int64_t ldo,
                                                   int64_t i0, int64_t i1, int64_t j0,
                                                   int64_t j1, int64_t kb, int64_t ke) {
  constexpr int TM = 16 * TI, TN = 16 * TJ;   // tile rows (P side), columns (Q side)
  constexpr int EP = TM / 16, EQ = TN / 16;   // k values a thread stages per row
  __shared__ __attribute__((aligned(16))) double Ps[2][TKC][TM + 2];
  __shared__ __attribute__((aligned(16))) double Qs[2][TKC][TN + 2];
  // KFROM_ROW tiles get the row tile from blockIdx.y, so that the tiles with
  // the longest sums (the first rows) are dispatched first.
  const int64_t bx = KFROM_ROW ? blockIdx.y : blockIdx.x, by = KFROM_ROW ? blockIdx.x : blockIdx.y;
  const int64_t ti = i0 + bx * TM, tj = j0 + by * TN;
  if (LOWER && tj > ti + TM - 1) return;
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  const int64_t ks = KFROM_ROW ? (ti > kb ? ti : kb) : kb;

  // staging: thread loads EP consecutive k of P tile row pr, EQ of Q tile row qr
  const int pr = tid / (16 / EP), ph = (tid % (16 / EP)) * EP;
  const int qr = tid / (16 / EQ), qh = (tid % (16 / EQ)) * EQ;
  const bool pok = ti + pr < i1, qok = tj + qr < j1;
  const double *pp = P + (pok ? ti + pr : 0) * ldp;
  const double *qp = Q + (qok ? tj + qr : 0) * ldq;
  // gload only issues the loads (from clamped addresses); the zero fill past
  // the ranges is applied when the values go to LDS, after the current stage's
  // arithmetic, so the loads stay in flight meanwhile.
  double pv[EP], qv[EQ];
  auto gload = [&](int64_t k) {
#pragma unroll
    for (int e = 0; e < EP; ++e) pv[e] = pp[k + ph + e < ke ? k + ph + e : kb];
#pragma unroll
    for (int e = 0; e < EQ; ++e) qv[e] = qp[k + qh + e < ke ? k + qh + e : kb];
  };
  auto sstore = [&](int buf, int64_t k) {
#pragma unroll
    for (int e = 0; e < EP; ++e) Ps[buf][ph + e][pr] = pok && k + ph + e < ke ? pv[e] : 0.0;
#pragma unroll
    for (int e = 0; e < EQ; ++e) Qs[buf][qh + e][qr] = qok && k + qh + e < ke ? qv[e] : 0.0;
  };

  // element (r, c) of this thread is out[(ti + TI ty + r) * ldo + tj + TJ tx + c]
  auto valid = [&](int r, int c) {
    const int64_t i = ti + ty * TI + r, j = tj + tx * TJ + c;
    return i < i1 && j < j1 && (!LOWER || j <= i);
  };
  // in bounds for every (r, c): rows and columns past the range are clamped
  auto oidx = [&](int r, int c) {
    const int64_t i = ti + ty * TI + r, j = tj + tx * TJ + c;
    return (i < i1 ? i : i1 - 1) * ldo + (j < j1 ? j : j1 - 1);
  };
  double acc[TI][TJ];
  if (MODE == SEQ_CONT) {
    // all loads first, then the selects (unrolled code keeps source order)
#pragma unroll
    for (int r = 0; r < TI; ++r)
#pragma unroll
      for (int c = 0; c < TJ; ++c) acc[r][c] = out[oidx(r, c)];
#pragma unroll
    for (int r = 0; r < TI; ++r)
#pragma unroll
      for (int c = 0; c < TJ; ++c) acc[r][c] = valid(r, c) ? acc[r][c] : 0.0;
  } else {
#pragma unroll
    for (int r = 0; r < TI; ++r)
#pragma unroll
      for (int c = 0; c < TJ; ++c) acc[r][c] = 0.0;
  }

  if (ks < ke) {
    int buf = 0;
    gload(ks);
    sstore(0, ks);
    __syncthreads();
    for (int64_t k = ks; k < ke; k += TKC) {
      const bool more = k + TKC < ke;
      if (more) gload(k + TKC);
#pragma unroll 2
      for (int kk = 0; kk < TKC; ++kk) {
        double a[TI], b[TJ];
#pragma unroll
        for (int h = 0; h < TI / 2; ++h) {
          const f64x2 x = *reinterpret_cast<const f64x2 *>(&Ps[buf][kk][ty * TI + 2 * h]);
          a[2 * h] = x.x;
          a[2 * h + 1] = x.y;
        }
#pragma unroll
        for (int h = 0; h < TJ / 2; ++h) {
          const f64x2 y = *reinterpret_cast<const f64x2 *>(&Qs[buf][kk][tx * TJ + 2 * h]);
          b[2 * h] = y.x;
          b[2 * h + 1] = y.y;
        }
#pragma unroll
        for (int r = 0; r < TI; ++r)
#pragma unroll
          for (int c = 0; c < TJ; ++c) acc[r][c] = acc[r][c] + a[r] * b[c];
      }
      if (more) sstore(buf ^ 1, k + TKC);
      __syncthreads();
      buf ^= 1;
    }
  }

  if (MODE == SEQ_SUB) {
    // up to four rows at a time: their loads, then the subtractions and stores
    constexpr int RB = TI < 4 ? TI : 4;
#pragma unroll
    for (int h = 0; h < TI; h += RB) {
      double o[RB][TJ];
#pragma unroll
      for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int c = 0; c < TJ; ++c) o[r][c] = out[oidx(h + r, c)];
#pragma unroll
      for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int c = 0; c < TJ; ++c)
          if (valid(h + r, c)) out[oidx(h + r, c)] = o[r][c] - acc[h + r][c];
    }
  } else {
#pragma unroll
    for (int r = 0; r < TI; ++r)
#pragma unroll
      for (int c = 0; c < TJ; ++c)
        if (valid(r, c)) out[oidx(r, c)] = acc[r][c];
  }
}

template <int MODE, bool LOWER, bool KFROM_ROW, int TI, int TJ>
void seqdot_launch(const double *P, int64_t ldp, const double *Q, int64_t ldq, double *out,
                   int64_t ldo, int64_t i0, int64_t i1, int64_t j0, int64_t j1, int64_t kb,
                   int64_t ke, hipStream_t st) {
  const unsigned gr = (unsigned)((i1 - i0 + 16 * TI - 1) / (16 * TI));
  const unsigned gc = (unsigned)((j1 - j0 + 16 * TJ - 1) / (16 * TJ));
  const dim3 grid(KFROM_ROW ? gc : gr, KFROM_ROW ? gr : gc);
  k_seqdot<MODE, LOWER, KFROM_ROW, TI, TJ>
      <<<grid, 256, 0, st>>>(P, ldp, Q, ldq, out, ldo, i0, i1, j0, j1, kb, ke);
}

// Tiles of the (i, j) range with t x t tiles (about half of them for LOWER).
inline int64_t tile_count(int64_t rows, int64_t cols, int64_t t, bool lower) {
  const int64_t n = ((rows + t - 1) / t) * ((cols + t - 1) / t);
  return lower ? (n + (rows + t - 1) / t) / 2 : n;
}

// 128 x 128 tiles while there are enough of them to fill the chip twice over
// (two workgroups per CU), 64 x 64 while those fill it, else 64 x 32.
template <int MODE, bool LOWER, bool KFROM_ROW>
void seqdot(const double *P, int64_t ldp, const double *Q, int64_t ldq, double *out, int64_t ldo,
            int64_t i0, int64_t i1, int64_t j0, int64_t j1, int64_t kb, int64_t ke,
            hipStream_t st) {
  if (i1 <= i0 || j1 <= j0) return;
  const int64_t R = i1 - i0, C = j1 - j0;
  if (tile_count(R, C, 128, LOWER) >= 512)
    seqdot_launch<MODE, LOWER, KFROM_ROW, 8, 8>(P, ldp, Q, ldq, out, ldo, i0, i1, j0, j1, kb, ke,
                                                st);
  else if (tile_count(R, C, 64, LOWER) >= 256)
    seqdot_launch<MODE, LOWER, KFROM_ROW, 4, 4>(P, ldp, Q, ldq, out, ldo, i0, i1, j0, j1, kb, ke,
                                                st);
  else
    seqdot_launch<MODE, LOWER, KFROM_ROW, 4, 2>(P, ldp, Q, ldq, out, ldo, i0, i1, j0, j1, kb, ke,
                                                st);
}

// ---------------------------------------------------------- column blocks


// Columns [i1, i1 + bl) of every row, in order: qc = clamp(round(w / s), -128, 127),
// e = (w - qc s) / hinv[i][i], then w[j] -= e hinv[i][j] for the block's later
// columns. One wave a row, lane l holding columns i1 + l + 64 c. hinv rows are
// read two steps ahead. The errors go to E [N, bl] for the trailing update.
template <int CPL>
__global__ __launch_bounds__(256) void k_gptq_block(const double *__restrict__ W, int64_t N,
                                                    int64_t K, const double *__restrict__ hinv,
                                                    const float *__restrict__ scale, int64_t i1,
                                                    int bl, double *__restrict__ E,
                                                    int8_t *__restrict__ q,
                                                    int32_t *__restrict__ wsum, int first) {
  const int lane = threadIdx.x & 63;
  const int64_t n = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= N) return;
  const double *hb = hinv + i1 * K + i1;
  double wv[CPL], ev[CPL];
  int qv[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int jj = lane + 64 * c;
    wv[c] = ld_or(W, n * K + i1 + jj, jj < bl, 0.0);
    ev[c] = 0.0;
    qv[c] = 0;
  }
  auto hrow = [&](int l, double *h) {
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int jj = lane + 64 * c;
      const bool ok = l < bl && jj < bl;
      h[c] = ld_or(hb, (int64_t)l * K + jj, ok, 0.0);
    }
  };
  double h0[CPL], h1[CPL], h2[CPL];
  hrow(0, h0);
  hrow(1, h1);
  const double s = (double)scale[n];
  for (int l = 0; l < bl; ++l) {
    hrow(l + 2, h2);
    const int cl = l >> 6, ln = l & 63;
    double col = 0.0, hii = 1.0;
#pragma unroll
    for (int c = 0; c < CPL; ++c)
      if (c == cl) {
        col = readlane_f64(wv[c], ln);
        hii = readlane_f64(h0[c], ln);
      }
    double qc = rint(col / s);
    qc = fmin(fmax(qc, -128.0), 127.0);
    const double e = (col - qc * s) / hii;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      wv[c] = wv[c] - e * h0[c];
      if (c == cl && lane == ln) {
        ev[c] = e;
        qv[c] = (int)qc;
      }
      h0[c] = h1[c];
      h1[c] = h2[c];
    }
  }
  int tot = 0;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int jj = lane + 64 * c;
    if (jj < bl) {
      E[n * bl + jj] = ev[c];
      q[n * K + i1 + jj] = (int8_t)qv[c];
    }
    tot += qv[c];
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) tot += __shfl_xor(tot, o);
  if (wsum && lane == 0) wsum[n] = first ? tot : wsum[n] + tot;
}

template <int CPL>
void gptq_block(const double *W, int64_t N, int64_t K, const double *hinv, const float *scale,
                int64_t i1, int bl, double *E, int8_t *q, int32_t *wsum, int first,
                hipStream_t st) {
  k_gptq_block<CPL><<<(unsigned)((N + 3) / 4), 256, 0, st>>>(W, N, K, hinv, scale, i1, bl, E, q,
                                                             wsum, first);
}

// ------------------------------------------------------------- factorizations

// Lower Cholesky factor L of A (lower triangle read); acc is scratch [K, K].
// Panels of PB columns; within a group of SB columns each panel's update
// reaches the group's later columns at once, the rest of the matrix receives
// the whole group's update in one launch (terms still added in ascending k).
void cholesky(const double *A, double *acc, double *L, int64_t K, int32_t *info, int32_t code0,
              hipStream_t st) {
  const int64_t kk = K * K;
  k_fill_f64<<<(unsigned)((kk + 255) / 256 < 8192 ? (kk + 255) / 256 : 8192), 256, 0, st>>>(acc,
                                                                                           kk);
  for (int64_t s0 = 0; s0 < K; s0 += SB) {
    const int64_t s1 = s0 + SB < K ? s0 + SB : K;
    for (int64_t k0 = s0; k0 < s1; k0 += PB) {
      const int64_t k1 = k0 + PB < K ? k0 + PB : K;
      k_chol_panel<<<(unsigned)(1 + (K - k1 + 63) / 64), 64, 0, st>>>(A, acc, L, K, k0, info,
                                                                        code0 + (int32_t)k0);
      if (k1 < s1)
        seqdot<SEQ_CONT, true, false>(L + k0, K, L + k0, K, acc, K, k1, K, k1, s1, 0, k1 - k0,
                                      st);
    }
    if (s1 < K)
      seqdot<SEQ_CONT, true, false>(L + s0, K, L + s0, K, acc, K, s1, K, s1, K, 0, s1 - s0, st);
  }
}

// X = (L^-1) stored transposed; acc is scratch [K, K]. X must be zero on entry.
void tri_inverse(const double *L, double *acc, double *X, int64_t K, hipStream_t st) {
  const int64_t kk = K * K;
  k_fill_f64<<<(unsigned)((kk + 255) / 256 < 8192 ? (kk + 255) / 256 : 8192), 256, 0, st>>>(acc,
                                                                                           kk);
  for (int64_t s0 = 0; s0 < K; s0 += SB) {
    const int64_t s1 = s0 + SB < K ? s0 + SB : K;
    for (int64_t k0 = s0; k0 < s1; k0 += PB) {
      const int64_t k1 = k0 + PB < K ? k0 + PB : K;
      k_trinv_panel<<<(unsigned)((k1 + 63) / 64), 64, 0, st>>>(L, acc, X, K, k0);
      if (k1 < s1)
        seqdot<SEQ_CONT, false, false>(L + k0, K, X + k0, K, acc, K, k1, s1, 0, k1, 0, k1 - k0,
                                       st);
    }
    if (s1 < K)
      seqdot<SEQ_CONT, false, false>(L + s0, K, X + s0, K, acc, K, s1, K, 0, s1, 0, s1 - s0, st);
  }
}

}  // namespace

size_t gptq_workspace_bytes(int64_t N, int64_t K, int64_t block) {
  return 4 * align256(sizeof(double) * K * K) + align256(sizeof(double) * N * K) +
         align256(sizeof(double) * N * block) + align256((size_t)K);
}

hipError_t launch_gptq_int8(const float *w, int64_t N, int64_t K, const double *H, double damp,
                            int block, int8_t *q, float *scale, int32_t *wsum, double *hinv_out,
                            int32_t *info, void *ws, hipStream_t st) {
  const GptqWs b = carve(ws, N, K, block);
  const int64_t kk = K * K;
  const unsigned fill_grid = (unsigned)((kk + 255) / 256 < 8192 ? (kk + 255) / 256 : 8192);
  hipError_t e = launch_quantize_weight_int8(w, false, N, K, AQL_WQ_SYM127_5, q, scale, nullptr,
                                             st);
  if (e != hipSuccess) return e;
  const unsigned rows_grid = (unsigned)(K < 4096 ? K : 4096);
  k_gptq_prep<<<rows_grid, 256, 0, st>>>(H, K, b.A, b.dead);
  k_gptq_damp<<<1, 256, 0, st>>>(b.A, K, damp, info);
  // L = chol(Hd); X = L^-1 (transposed); A = X^T X = Hd^-1 (lower); L = chol(Hd^-1)
  cholesky(b.A, b.acc, b.L, K, info, 0, st);
  k_fill_f64<<<fill_grid, 256, 0, st>>>(b.X, kk);
  tri_inverse(b.L, b.acc, b.X, K, st);
  // 64 x 64 tiles: the sums of the first tile row run over all of K, the last
  // over one tile, so many small tiles (longest first) balance the chip
  seqdot_launch<SEQ_STORE, true, true, 4, 4>(b.X, K, b.X, K, b.A, K, 0, K, 0, K, 0, K, st);
  cholesky(b.A, b.acc, b.L, K, info, (int32_t)K, st);
  // hinv = L^T (upper), into X
  k_gptq_upper_of<<<dim3((unsigned)((K + 63) / 64), (unsigned)((K + 63) / 64)), 256, 0, st>>>(
      b.L, K, b.X);
  const double *hinv = b.X;
  k_gptq_wcopy<<<(unsigned)(N < 8192 ? N : 8192), 256, 0, st>>>(w, N, K, b.dead, b.W);
  for (int64_t i1 = 0; i1 < K; i1 += block) {
    const int64_t i2 = i1 + block < K ? i1 + block : K;
    const int bl = (int)(i2 - i1);
    const int first = i1 == 0;
    if (bl <= 64)
      gptq_block<1>(b.W, N, K, hinv, scale, i1, bl, b.E, q, wsum, first, st);
    else if (bl <= 128)
      gptq_block<2>(b.W, N, K, hinv, scale, i1, bl, b.E, q, wsum, first, st);
    else
      gptq_block<4>(b.W, N, K, hinv, scale, i1, bl, b.E, q, wsum, first, st);
    // W[n][j] -= sum_t E[n][t] hinv[i1 + t][j] for j >= i2; hinv[t][j] = L[j][t]
    if (i2 < K) seqdot<SEQ_SUB, false, false>(b.E, bl, b.L + i1, K, b.W, K, 0, N, i2, K, 0, bl, st);
  }
  if (hinv_out) {
    e = hipMemcpyAsync(hinv_out, hinv, sizeof(double) * kk, hipMemcpyDeviceToDevice, st);
    if (e != hipSuccess) return e;
  }
  return hipGetLastError();
}

}  // namespace aql
