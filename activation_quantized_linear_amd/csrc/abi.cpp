// C ABI of libaql.so: argument validation, M-dispatch and launches.
// Every check runs before the first HIP call, so an invalid call launches
// nothing and touches no device state; an empty problem (M == 0 or N == 0)
// returns AQL_OK without a HIP call, and its (zero-element) buffers may be NULL.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>
#include <vector>

#include "aql.h"
#include "calib.h"
#include "dq8ca_q4.h"
#include "gemm_i8.h"
#include "gptq.h"
#include "quant.h"
#include "w8a16.h"
#include "measure.h"
#include "w8a16_gemm.h"

// Rows of x from which aql_linear_w8a16 uses the tiled GEMM.
constexpr int64_t kW8A16GemmMinM = 64;

namespace {

thread_local std::string g_err;

int fail(int code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return AQL_OK;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool finite_pos(float s) { return std::isfinite(s) && s > 0.0f; }

bool z_ok(int32_t z) { return z >= -128 && z <= 127; }

size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

// Per-device "is gfx950" cache: 0 unknown, 1 yes, 2 no.
std::atomic<int> g_dev_ok[64];

int check_device(const char *fn) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess)
    return fail(AQL_ERR_DEVICE, "%s: no HIP device (%s)", fn, hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(AQL_ERR_DEVICE, "%s: device index %d out of range", fn, dev);
  int st = g_dev_ok[dev].load(std::memory_order_relaxed);
  if (st == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess)
      return fail(AQL_ERR_DEVICE, "%s: hipGetDeviceProperties failed (%s)", fn,
                  hipGetErrorString(e));
    st = (std::string(prop.gcnArchName).rfind("gfx950", 0) == 0) ? 1 : 2;
    g_dev_ok[dev].store(st, std::memory_order_relaxed);
    if (st == 2)
      return fail(AQL_ERR_DEVICE, "%s: device %d is %s, this library is built for gfx950", fn,
                  dev, prop.gcnArchName);
  }
  if (st == 2) return fail(AQL_ERR_DEVICE, "%s: device %d is not a gfx950", fn, dev);
  return AQL_OK;
}

int launched(hipError_t e, const char *fn) {
  if (e != hipSuccess) return fail(AQL_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return ok();
}

#define REQUIRE(cond, code, ...) \
  do {                           \
    if (!(cond)) return fail(code, __VA_ARGS__); \
  } while (0)

size_t ws_q8ta(int64_t M, int64_t K) { return 2 * align256((size_t)M * (size_t)K); }

// activation operand (int8 codes, or bf16 differences for the tiled 4-bit
// kernel: 2 bytes per element), then row scales and zero points
size_t ws_dq8ca(int64_t M, int64_t K) {
  return align256(2 * (size_t)M * (size_t)K) + 2 * align256((size_t)M * 4);
}

// Largest K of the W8A16 kernels: a 16-row tile of x (bf16) stays below the
// out-of-range offset its buffer loads use.
constexpr int64_t kMaxKW8A16 = 1 << 24;

// Host table of a grouped W8A16 launch: this header, then one entry per
// non-empty problem.
struct GroupHeader {
  uint32_t magic;
  uint32_t version;
  int32_t count;         // entries that follow (non-empty problems)
  int32_t total_blocks;  // grid size
  int32_t waves;         // waves per workgroup
  int32_t mblocks;       // 4-row blocks of x per tile (0: single-row tile)
  int32_t tgroups;       // 4-channel groups per tile
  int32_t cgroups;       // wave tiles per workgroup along N (single-row tile)
  int32_t xlds;          // LDS bytes holding x (single-row tile; 0: none)
  int32_t kind;          // 0: the tile kernels above; 1: single-row pieces kernel
  int32_t reserved[6];
};
static_assert(sizeof(GroupHeader) == 64, "table header");
constexpr uint32_t kGroupMagic = 0x47514c41u;  // "ALQG"

int check_w8a16(const char *fn, const uint16_t *x, int64_t M, int64_t K, const int8_t *q,
                const float *scale, const uint16_t *bias, int64_t N, const uint16_t *y) {
  REQUIRE(M >= 0 && N >= 0 && K >= 16 && K % 16 == 0 && K <= kMaxKW8A16, AQL_ERR_SHAPE,
          "%s: need M, N >= 0 and K a multiple of 16 in [16, %lld] (M=%lld N=%lld K=%lld)", fn,
          (long long)kMaxKW8A16, (long long)M, (long long)N, (long long)K);
  REQUIRE(M <= 0xffff * 16LL && N <= 0x7fffffffLL * 16, AQL_ERR_SHAPE, "%s: M or N too large",
          fn);
  REQUIRE(aligned16(x) && aligned16(q) && aligned16(scale) && aligned16(bias) && aligned16(y),
          AQL_ERR_ALIGN, "%s: pointers must be 16-byte aligned", fn);
  if (M == 0 || N == 0) return AQL_OK;
  REQUIRE(x && q && scale && y, AQL_ERR_NULL, "%s: x, q, scale and y must not be NULL", fn);
  return AQL_OK;
}

// Validation shared by both static W8A8 entry points (all before any HIP call).
int check_q8ta(const char *fn, const float *x, int64_t M, int64_t K, float s1, int32_t z1,
               int two_pass, float s2, int32_t z2, const int8_t *q, const int32_t *wsum,
               const float *wscale, const float *bias, int64_t N, const float *y) {
  REQUIRE(finite_pos(s1) && z_ok(z1), AQL_ERR_PARAM,
          "%s: s1 must be finite and > 0, z1 in [-128, 127]", fn);
  REQUIRE(!two_pass || (finite_pos(s2) && z_ok(z2)), AQL_ERR_PARAM,
          "%s: s2 must be finite and > 0, z2 in [-128, 127]", fn);
  REQUIRE(M >= 0 && N >= 0 && K >= 16 && K % 16 == 0 && K <= AQL_MAX_K_INT8, AQL_ERR_SHAPE,
          "%s: need M, N >= 0 and K a multiple of 16 in [16, %d] (M=%lld N=%lld K=%lld)", fn,
          AQL_MAX_K_INT8, (long long)M, (long long)N, (long long)K);
  REQUIRE(M < (1LL << 31) / 128 && N < (1LL << 31) / 128, AQL_ERR_SHAPE, "%s: M or N too large",
          fn);
  REQUIRE(aligned16(x) && aligned16(q) && aligned16(wsum) && aligned16(wscale) &&
              aligned16(bias) && aligned16(y),
          AQL_ERR_ALIGN, "%s: pointers must be 16-byte aligned", fn);
  if (M == 0 || N == 0) return AQL_OK;
  REQUIRE(x && q && wsum && wscale && y, AQL_ERR_NULL,
          "%s: x, q, wsum, wscale and y must not be NULL", fn);
  return AQL_OK;
}

// The static W8A8 linear on a validated call: the activation quantizer writes
// xq1 (and xq2) into ws, then the int8 GEMM with the fused epilogue. Every
// byte of ws that the GEMM reads is written by the quantizer first, so ws
// needs no clearing.
int run_q8ta(const char *fn, const float *x, int64_t M, int64_t K, float s1, int32_t z1,
             int two_pass, float s2, int32_t z2, const int8_t *q, const int32_t *wsum,
             const float *wscale, const float *bias, int64_t N, float *y, void *ws,
             hipStream_t st) {
  int8_t *xq1 = static_cast<int8_t *>(ws);
  int8_t *xq2 = xq1 + align256((size_t)M * (size_t)K);
  hipError_t e = aql::launch_quantize_act_per_tensor(x, M * K, s1, z1, two_pass != 0, s2, z2, xq1,
                                                     xq2, st);
  if (e != hipSuccess) return launched(e, fn);
  aql::GemmArgs a{};
  a.a1 = xq1;
  a.a2 = xq2;
  a.b = q;
  a.M = M;
  a.N = N;
  a.K = K;
  a.y = y;
  a.wsum = wsum;
  a.wscale = wscale;
  a.bias = bias;
  a.s1 = s1;
  a.s2 = s2;
  a.z1 = z1;
  a.z2 = z2;
  return launched(aql::launch_gemm_i8(a, aql::EPI_Q8TA, two_pass != 0, st), fn);
}

// Scratch of the allocation-free entry point: a fixed device array that every
// GPU the library runs on holds until the process ends. Host code never uses
// the array's name as an address (on the host it is only a stand-in for the
// symbol); each device's address comes from hipGetSymbolAddress, taken once
// per device with that device current, and is what the kernels are given.
__device__ __align__(256) unsigned char scratch[AQL_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
void *g_scratch_ptr[64];  // per device index (check_device bounds it to 64)

int scratch_of_current_device(const char *fn, void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= 64)
    return fail(AQL_ERR_DEVICE, "%s: no usable HIP device", fn);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(AQL_ERR_HIP, "%s: hipGetSymbolAddress of the scratch array failed on device "
                  "%d (%s)", fn, dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return AQL_OK;
}

}  // namespace

extern "C" {

int aql_version(void) { return 100; }

const char *aql_last_error(void) { return g_err.c_str(); }

size_t aql_workspace_bytes(int op, int64_t M, int64_t N, int64_t K) {
  if (M < 0 || N < 0 || K < 0) return 0;
  if (op == AQL_OP_Q8TA_Q8CSW) return ws_q8ta(M, K);
  if (op == AQL_OP_DQ8CA) return ws_dq8ca(M, K);
  if (op == AQL_OP_GPTQ_INT8) {
    if (M < 1 || M > aql::kGptqMaxBlock || K > AQL_MAX_K_INT8) return 0;
    return aql::gptq_workspace_bytes(N, K, M);
  }
  if (op == AQL_OP_W8A16) {
    if (N == 0 || K > kMaxKW8A16) return 0;
    if (M < kW8A16GemmMinM) return aql::w8a16_skinny_part_bytes(M, N, K);
    if (K > (1LL << 22)) return 0;
    return aql::w8a16_gemm_part_bytes(M, N, K);
  }
  return 0;
}

int aql_quantize_weight_int8(const void *w, int w_dtype, int64_t N, int64_t K, int mode,
                             int8_t *q, float *scale, int32_t *wsum, void *stream) {
  const char *fn = "aql_quantize_weight_int8";
  REQUIRE(w_dtype == AQL_F32 || w_dtype == AQL_BF16, AQL_ERR_PARAM, "%s: unknown w_dtype %d", fn,
          w_dtype);
  REQUIRE(mode == AQL_WQ_SYM127 || mode == AQL_WQ_SYM127_5, AQL_ERR_PARAM, "%s: unknown mode %d",
          fn, mode);
  REQUIRE(N >= 0 && K >= 1 && K % 4 == 0, AQL_ERR_SHAPE,
          "%s: need N >= 0, K >= 1 and K %% 4 == 0 (N=%lld K=%lld)", fn, (long long)N,
          (long long)K);
  REQUIRE(aligned16(w) && aligned16(q) && aligned16(scale) && aligned16(wsum), AQL_ERR_ALIGN,
          "%s: pointers must be 16-byte aligned", fn);
  if (N == 0) return ok();
  REQUIRE(w && q && scale, AQL_ERR_NULL, "%s: w, q and scale must not be NULL", fn);
  if (int e = check_device(fn)) return e;
  return launched(aql::launch_quantize_weight_int8(w, w_dtype == AQL_BF16, N, K, mode, q, scale,
                                                   wsum, (hipStream_t)stream),
                  fn);
}

int aql_quantize_weight_q4gsw(const float *w, int64_t N, int64_t K, int group, uint8_t *q4,
                              float *gscale, int32_t *gsum, void *stream) {
  const char *fn = "aql_quantize_weight_q4gsw";
  REQUIRE(group == 32, AQL_ERR_PARAM, "%s: group must be 32 (got %d)", fn, group);
  REQUIRE(N >= 0 && K >= 32 && K % 32 == 0, AQL_ERR_SHAPE,
          "%s: need N >= 0 and K a positive multiple of 32 (N=%lld K=%lld)", fn, (long long)N,
          (long long)K);
  REQUIRE(aligned16(w) && aligned16(q4) && aligned16(gscale) && aligned16(gsum), AQL_ERR_ALIGN,
          "%s: pointers must be 16-byte aligned", fn);
  if (N == 0) return ok();
  REQUIRE(w && q4 && gscale, AQL_ERR_NULL, "%s: w, q4 and gscale must not be NULL", fn);
  if (int e = check_device(fn)) return e;
  return launched(aql::launch_quantize_weight_q4gsw(w, N, K, q4, gscale, gsum,
                                                    (hipStream_t)stream),
                  fn);
}

int aql_choose_qparams_rows(const float *x, int64_t M, int64_t K, float *scale, int32_t *zp,
                            int8_t *xq, void *stream) {
  const char *fn = "aql_choose_qparams_rows";
  REQUIRE(M >= 0 && K >= 1 && K % 4 == 0, AQL_ERR_SHAPE,
          "%s: need M >= 0, K >= 1 and K %% 4 == 0 (M=%lld K=%lld)", fn, (long long)M,
          (long long)K);
  REQUIRE(aligned16(x) && aligned16(scale) && aligned16(zp) && aligned16(xq), AQL_ERR_ALIGN,
          "%s: pointers must be 16-byte aligned", fn);
  if (M == 0) return ok();
  REQUIRE(x && scale && zp, AQL_ERR_NULL, "%s: x, scale and zp must not be NULL", fn);
  if (int e = check_device(fn)) return e;
  return launched(
      aql::launch_choose_qparams_rows(x, M, K, scale, zp, xq, aql::QP_CODES, (hipStream_t)stream),
      fn);
}

int aql_quantize_act_per_tensor(const float *x, int64_t M, int64_t K, float s1, int32_t z1,
                                int two_pass, float s2, int32_t z2, int8_t *xq1, int8_t *xq2,
                                void *stream) {
  const char *fn = "aql_quantize_act_per_tensor";
  REQUIRE(finite_pos(s1) && z_ok(z1), AQL_ERR_PARAM,
          "%s: s1 must be finite and > 0, z1 in [-128, 127]", fn);
  REQUIRE(!two_pass || (finite_pos(s2) && z_ok(z2)), AQL_ERR_PARAM,
          "%s: s2 must be finite and > 0, z2 in [-128, 127]", fn);
  REQUIRE(M >= 0 && K >= 1 && K % 4 == 0, AQL_ERR_SHAPE,
          "%s: need M >= 0, K >= 1 and K %% 4 == 0 (M=%lld K=%lld)", fn, (long long)M,
          (long long)K);
  REQUIRE(aligned16(x) && aligned16(xq1) && aligned16(xq2), AQL_ERR_ALIGN,
          "%s: pointers must be 16-byte aligned", fn);
  if (M == 0) return ok();
  REQUIRE(x && xq1 && (!two_pass || xq2), AQL_ERR_NULL,
          "%s: x, xq1 (and xq2 with two_pass) must not be NULL", fn);
  if (int e = check_device(fn)) return e;
  return launched(aql::launch_quantize_act_per_tensor(x, M * K, s1, z1, two_pass != 0, s2, z2,
                                                      xq1, xq2, (hipStream_t)stream),
                  fn);
}

int aql_linear_w8a16(const uint16_t *x, int64_t M, int64_t K, const int8_t *q,
                     const float *scale, const uint16_t *bias, int64_t N, uint16_t *y,
                     void *ws, size_t ws_bytes, void *stream) {
  const char *fn = "aql_linear_w8a16";
  if (int e = check_w8a16(fn, x, M, K, q, scale, bias, N, y)) return e;
  REQUIRE(aligned16(ws), AQL_ERR_ALIGN, "%s: ws must be 16-byte aligned", fn);
  if (M == 0 || N == 0) return ok();
  if (int e = check_device(fn)) return e;
  // M-dispatch (flashrt schemes, W8A16Decode: the decode band goes to the
  // weight-streaming kernel): from 64 rows on, the tiled bf16-MFMA GEMM reads
  // each weight once per 64 or 128 rows instead of once per 16.
  if (M >= kW8A16GemmMinM && K <= (1LL << 22))
    return launched(aql::launch_w8a16_gemm(x, M, K, q, scale, bias, N, y, static_cast<float *>(ws),
                                           ws ? ws_bytes : 0, (hipStream_t)stream),
                    fn);
  return launched(aql::launch_w8a16(x, M, K, q, scale, bias, N, y, static_cast<float *>(ws),
                                    ws ? ws_bytes : 0, (hipStream_t)stream),
                  fn);
}

size_t aql_w8a16_group_table_bytes(int count) {
  if (count < 1) return 0;
  return sizeof(GroupHeader) + (size_t)count * sizeof(aql::W8A16GroupEntry);
}

int aql_w8a16_group_plan(const aql_w8a16_problem *problems, int count, void *table,
                         size_t table_bytes) {
  const char *fn = "aql_w8a16_group_plan";
  REQUIRE(count >= 1, AQL_ERR_SHAPE, "%s: count must be >= 1 (got %d)", fn, count);
  REQUIRE(problems, AQL_ERR_NULL, "%s: problems must not be NULL", fn);
  REQUIRE(table && table_bytes >= aql_w8a16_group_table_bytes(count), AQL_ERR_WORKSPACE,
          "%s: table needs %zu bytes", fn, aql_w8a16_group_table_bytes(count));
  GroupHeader *h = static_cast<GroupHeader *>(table);
  aql::W8A16GroupEntry *e = reinterpret_cast<aql::W8A16GroupEntry *>(h + 1);
  // One launch shape for the whole group, from the smallest K and the largest M.
  // Groups of single-row problems with kW8A16PiecesMinK <= K <= kW8A16PiecesMaxK
  // take the pieces kernel (whole 1 KB row pieces, no bytes read past a row).
  int64_t kmin = 0, kmax = 0, mmax = 0, nsum = 0;
  for (int i = 0; i < count; ++i) {
    const aql_w8a16_problem &p = problems[i];
    char name[64];
    snprintf(name, sizeof name, "%s: problem %d", fn, i);
    if (int rc = check_w8a16(name, p.x, p.M, p.K, p.q, p.scale, p.bias, p.N, p.y)) return rc;
    if (p.M == 0 || p.N == 0) continue;
    kmin = (kmin == 0 || p.K < kmin) ? p.K : kmin;
    kmax = p.K > kmax ? p.K : kmax;
    mmax = p.M > mmax ? p.M : mmax;
    nsum += p.N * ((p.M + 15) / 16);
  }
  const bool pieces = mmax == 1 && kmin >= aql::kW8A16PiecesMinK && kmax <= aql::kW8A16PiecesMaxK;
  aql::W8A16Shape sh = aql::w8a16_shape(mmax ? mmax : 1, nsum ? nsum : 1, kmin ? kmin : 16);
  if (sh.waves > 8) sh.waves = 8;
  // x shared through LDS only if every problem's x fits
  if (sh.mblocks == 0) sh.xlds = aql::w8a16_xlds_bytes(kmax ? kmax : 16);
  if (pieces) {
    sh = aql::W8A16Shape{};
    sh.waves = 4;
    sh.tgroups = 2;
    sh.mblocks = 0;
  }
  int64_t blocks = 0;
  int n = 0;
  for (int i = 0; i < count; ++i) {
    const aql_w8a16_problem &p = problems[i];
    if (p.M == 0 || p.N == 0) continue;
    const int64_t rows =
        pieces ? aql::w8a16_pieces_tile_channels(p.K) : 4 * sh.tgroups * sh.cgroups;
    const int64_t nblk = (p.N + rows - 1) / rows, mblk = (p.M + 15) / 16;
    REQUIRE(blocks + nblk * mblk <= 0x7fffffffLL, AQL_ERR_SHAPE, "%s: too many tiles in total",
            fn);
    aql::W8A16GroupEntry &d = e[n++];
    d = aql::W8A16GroupEntry{};
    d.x = p.x;
    d.q = p.q;
    d.scale = p.scale;
    d.bias = p.bias;
    d.y = p.y;
    d.M = p.M;
    d.N = p.N;
    d.K = p.K;
    d.blk_begin = (int32_t)blocks;
    d.nblk = (int32_t)nblk;
    blocks += nblk * mblk;
  }
  *h = GroupHeader{};
  h->magic = kGroupMagic;
  h->version = 2;
  h->count = n;
  h->total_blocks = (int32_t)blocks;
  h->waves = sh.waves;
  h->mblocks = sh.mblocks;
  h->tgroups = sh.tgroups;
  h->cgroups = sh.cgroups;
  h->xlds = sh.xlds;
  h->kind = pieces ? 1 : 0;
  return ok();
}

int aql_linear_w8a16_grouped(const void *table, const void *dev_table, void *stream) {
  const char *fn = "aql_linear_w8a16_grouped";
  REQUIRE(table, AQL_ERR_NULL, "%s: table must not be NULL", fn);
  const GroupHeader *h = static_cast<const GroupHeader *>(table);
  const bool m1 = h->mblocks == 0;
  const bool pieces = h->kind == 1;
  REQUIRE(h->magic == kGroupMagic && h->version == 2 && h->count >= 0 && h->total_blocks >= 0 &&
              (h->kind == 0 || (pieces && h->waves == 4 && h->mblocks == 0 && h->tgroups == 2 &&
                                h->cgroups == 1 && h->xlds == 0)) &&
              (h->waves == 1 || h->waves == 2 || h->waves == 4 || h->waves == 8) &&
              (h->mblocks == 0 || h->mblocks == 1 || h->mblocks == 2 || h->mblocks == 4 ||
               h->mblocks == aql::kW8A16Skinny) &&
              (h->mblocks == aql::kW8A16Skinny ? (h->tgroups == 4 || h->tgroups == 8)
                                               : (h->tgroups == 1 || h->tgroups == 2 ||
                                                  h->tgroups == 4)) &&
              (m1 ? (h->tgroups == 2 && (h->cgroups == 1 || h->cgroups == 2 || h->cgroups == 4) &&
                     h->waves * h->cgroups <= 16 && h->xlds >= 0 &&
                     h->xlds <= aql::kW8A16MaxXlds && h->xlds % 1024 == 0)
                  : (h->cgroups == 1 && h->xlds == 0)),
          AQL_ERR_PARAM, "%s: table was not written by aql_w8a16_group_plan", fn);
  if (h->count == 0 || h->total_blocks == 0) return ok();
  REQUIRE(dev_table, AQL_ERR_NULL, "%s: dev_table must not be NULL", fn);
  REQUIRE(aligned16(dev_table), AQL_ERR_ALIGN, "%s: dev_table must be 16-byte aligned", fn);
  if (int e = check_device(fn)) return e;
  const aql::W8A16GroupEntry *dev_entries = reinterpret_cast<const aql::W8A16GroupEntry *>(
      static_cast<const char *>(dev_table) + sizeof(GroupHeader));
  aql::W8A16Shape sh;
  sh.waves = h->waves;
  sh.mblocks = h->mblocks;
  sh.tgroups = h->tgroups;
  sh.cgroups = h->cgroups;
  sh.xlds = h->xlds;
  if (pieces)
    return launched(aql::launch_w8a16_m1p_grouped(
                        dev_entries,
                        reinterpret_cast<const aql::W8A16GroupEntry *>(
                            static_cast<const char *>(table) + sizeof(GroupHeader)),
                        h->count, h->total_blocks, (hipStream_t)stream),
                    fn);
  return launched(aql::launch_w8a16_grouped(dev_entries, h->count, h->total_blocks, sh,
                                            (hipStream_t)stream),
                  fn);
}

int aql_linear_q8ta_q8csw(const float *x, int64_t M, int64_t K, float s1, int32_t z1,
                          int two_pass, float s2, int32_t z2, const int8_t *q,
                          const int32_t *wsum, const float *wscale, const float *bias, int64_t N,
                          float *y, void *ws, size_t ws_bytes, void *stream) {
  const char *fn = "aql_linear_q8ta_q8csw";
  if (int e = check_q8ta(fn, x, M, K, s1, z1, two_pass, s2, z2, q, wsum, wscale, bias, N, y))
    return e;
  REQUIRE(aligned16(ws), AQL_ERR_ALIGN, "%s: pointers must be 16-byte aligned", fn);
  if (M == 0 || N == 0) return ok();
  const size_t need = ws_q8ta(M, K);
  REQUIRE(ws && ws_bytes >= need, AQL_ERR_WORKSPACE, "%s: workspace needs %zu bytes (got %zu)",
          fn, need, ws ? ws_bytes : (size_t)0);
  if (int e = check_device(fn)) return e;
  return run_q8ta(fn, x, M, K, s1, z1, two_pass, s2, z2, q, wsum, wscale, bias, N, y, ws,
                  (hipStream_t)stream);
}

int aql_linear_q8ta_q8csw_noalloc(const float *x, int64_t M, int64_t K, float s1, int32_t z1,
                                  int two_pass, float s2, int32_t z2, const int8_t *q,
                                  const int32_t *wsum, const float *wscale, const float *bias,
                                  int64_t N, float *y, void *stream) {
  const char *fn = "aql_linear_q8ta_q8csw_noalloc";
  if (int e = check_q8ta(fn, x, M, K, s1, z1, two_pass, s2, z2, q, wsum, wscale, bias, N, y))
    return e;
  if (M == 0 || N == 0) return ok();
  const size_t need = ws_q8ta(M, K);
  REQUIRE(need <= (size_t)AQL_NOALLOC_SCRATCH_BYTES, AQL_ERR_WORKSPACE,
          "%s: M x K = %lld x %lld needs %zu bytes of scratch, more than the library's fixed "
          "%d (use aql_linear_q8ta_q8csw with a workspace)",
          fn, (long long)M, (long long)K, need, AQL_NOALLOC_SCRATCH_BYTES);
  if (int e = check_device(fn)) return e;
  void *ws = nullptr;
  if (int e = scratch_of_current_device(fn, &ws)) return e;
  return run_q8ta(fn, x, M, K, s1, z1, two_pass, s2, z2, q, wsum, wscale, bias, N, y, ws,
                  (hipStream_t)stream);
}

int aql_linear_dq8ca(const float *x, int64_t M, int64_t K, int wfmt, const void *wq,
                     const float *wscale, const int32_t *wsum, int group, const float *bias,
                     int64_t N, float *y, float *x_scale_out, int32_t *x_zp_out, void *ws,
                     size_t ws_bytes, void *stream) {
  const char *fn = "aql_linear_dq8ca";
  REQUIRE((wfmt == AQL_W_Q8CSW && group == 0) || (wfmt == AQL_W_Q4GSW && group == 32),
          AQL_ERR_PARAM, "%s: wfmt/group must be Q8CSW/0 or Q4GSW/32 (got %d/%d)", fn, wfmt,
          group);
  const int64_t kmul = wfmt == AQL_W_Q4GSW ? 32 : 16;
  REQUIRE(M >= 0 && N >= 0 && K >= kmul && K % kmul == 0 && K <= AQL_MAX_K_INT8, AQL_ERR_SHAPE,
          "%s: need M, N >= 0 and K a multiple of %lld in [%lld, %d] (M=%lld N=%lld K=%lld)", fn,
          (long long)kmul, (long long)kmul, AQL_MAX_K_INT8, (long long)M, (long long)N,
          (long long)K);
  REQUIRE(M < (1LL << 31) / 128 && N < (1LL << 31) / 128, AQL_ERR_SHAPE, "%s: M or N too large",
          fn);
  REQUIRE(aligned16(x) && aligned16(wq) && aligned16(wscale) && aligned16(wsum) &&
              aligned16(bias) && aligned16(y) && aligned16(x_scale_out) &&
              aligned16(x_zp_out) && aligned16(ws),
          AQL_ERR_ALIGN, "%s: pointers must be 16-byte aligned", fn);
  if (M == 0 || N == 0) return ok();
  REQUIRE(x && wq && wscale && wsum && y, AQL_ERR_NULL,
          "%s: x, wq, wscale, wsum and y must not be NULL", fn);
  const size_t need = ws_dq8ca(M, K);
  REQUIRE(ws && ws_bytes >= need, AQL_ERR_WORKSPACE, "%s: workspace needs %zu bytes (got %zu)",
          fn, need, ws ? ws_bytes : (size_t)0);
  if (int e = check_device(fn)) return e;
  hipStream_t st = (hipStream_t)stream;
  const bool q4 = wfmt == AQL_W_Q4GSW;
  char *base = static_cast<char *>(ws);
  const size_t xbytes = align256(2 * (size_t)M * (size_t)K);
  int8_t *xq = reinterpret_cast<int8_t *>(base);
  float *xs = x_scale_out ? x_scale_out : reinterpret_cast<float *>(base + xbytes);
  int32_t *xz = x_zp_out ? x_zp_out
                         : reinterpret_cast<int32_t *>(base + xbytes + align256((size_t)M * 4));
  const aql::QpOut mode = !q4 ? aql::QP_CODES
                              : (M <= aql::kQ4StreamMaxM ? aql::QP_CODES_PERM8 : aql::QP_DIFF_BF16);
  hipError_t e = aql::launch_choose_qparams_rows(x, M, K, xs, xz, xq, mode, st);
  if (e != hipSuccess) return launched(e, fn);
  if (q4) {
    aql::Q4Args a{};
    a.xq = xq;
    a.xd = reinterpret_cast<const uint16_t *>(xq);
    a.xs = xs;
    a.xz = xz;
    a.q4 = static_cast<const uint8_t *>(wq);
    a.gs = wscale;
    a.gsum = wsum;
    a.bias = bias;
    a.y = y;
    a.M = M;
    a.N = N;
    a.K = K;
    return launched(aql::launch_dq8ca_q4(a, st), fn);
  }
  aql::GemmArgs a{};
  a.a1 = xq;
  a.b = static_cast<const int8_t *>(wq);
  a.M = M;
  a.N = N;
  a.K = K;
  a.y = y;
  a.wsum = wsum;
  a.wscale = wscale;
  a.bias = bias;
  a.xs = xs;
  a.xz = xz;
  return launched(aql::launch_gemm_i8(a, aql::EPI_DQ8, false, st), fn);
}

int aql_gemm_i8_i32(const int8_t *a, const int8_t *b, int32_t *c, int64_t M, int64_t N,
                    int64_t K, void *stream) {
  const char *fn = "aql_gemm_i8_i32";
  REQUIRE(M >= 0 && N >= 0 && K >= 16 && K % 16 == 0 && K <= AQL_MAX_K_INT8, AQL_ERR_SHAPE,
          "%s: need M, N >= 0 and K a multiple of 16 in [16, %d] (M=%lld N=%lld K=%lld)", fn,
          AQL_MAX_K_INT8, (long long)M, (long long)N, (long long)K);
  REQUIRE(M < (1LL << 31) / 128 && N < (1LL << 31) / 128, AQL_ERR_SHAPE, "%s: M or N too large",
          fn);
  REQUIRE(aligned16(a) && aligned16(b) && aligned16(c), AQL_ERR_ALIGN,
          "%s: pointers must be 16-byte aligned", fn);
  if (M == 0 || N == 0) return ok();
  REQUIRE(a && b && c, AQL_ERR_NULL, "%s: a, b and c must not be NULL", fn);
  if (int e = check_device(fn)) return e;
  aql::GemmArgs g{};
  g.a1 = a;
  g.b = b;
  g.c = c;
  g.M = M;
  g.N = N;
  g.K = K;
  return launched(aql::launch_gemm_i8(g, aql::EPI_RAW, false, (hipStream_t)stream), fn);
}

int aql_minmax_reset(float *state, void *stream) {
  const char *fn = "aql_minmax_reset";
  REQUIRE(state, AQL_ERR_NULL, "%s: state must not be NULL", fn);
  REQUIRE(aligned16(state), AQL_ERR_ALIGN, "%s: state must be 16-byte aligned", fn);
  if (int e = check_device(fn)) return e;
  return launched(aql::launch_minmax_reset(state, (hipStream_t)stream), fn);
}

int aql_minmax_observe(const float *x, int64_t rows, int64_t cols, int64_t seq, int residual,
                       float s1, int32_t z1, float *state, void *stream) {
  const char *fn = "aql_minmax_observe";
  REQUIRE(rows >= 0 && cols >= 0 && cols % 4 == 0 && seq >= 0, AQL_ERR_SHAPE,
          "%s: need rows, seq >= 0 and cols >= 0 a multiple of 4 (rows=%lld cols=%lld seq=%lld)",
          fn, (long long)rows, (long long)cols, (long long)seq);
  REQUIRE(!residual || (finite_pos(s1) && z_ok(z1)), AQL_ERR_PARAM,
          "%s: the residual needs s1 finite > 0 and z1 in [-128, 127]", fn);
  REQUIRE(state, AQL_ERR_NULL, "%s: state must not be NULL", fn);
  REQUIRE(aligned16(state) && aligned16(x), AQL_ERR_ALIGN, "%s: pointers must be 16-byte aligned",
          fn);
  if (rows == 0 || cols == 0) return ok();
  REQUIRE(x, AQL_ERR_NULL, "%s: x must not be NULL", fn);
  if (int e = check_device(fn)) return e;
  return launched(aql::launch_minmax_observe(x, rows, cols, seq, residual != 0, s1, z1, state,
                                             (hipStream_t)stream),
                  fn);
}

int aql_minmax_qparams(const float *state, float *scale, int32_t *zp, void *stream) {
  const char *fn = "aql_minmax_qparams";
  REQUIRE(state && scale && zp, AQL_ERR_NULL, "%s: state, scale and zp must not be NULL", fn);
  REQUIRE(aligned16(state) && aligned16(scale) && aligned16(zp), AQL_ERR_ALIGN,
          "%s: pointers must be 16-byte aligned", fn);
  if (int e = check_device(fn)) return e;
  return launched(aql::launch_minmax_qparams(state, scale, zp, (hipStream_t)stream), fn);
}

int aql_keep_outliers(const float *amax, const int32_t *seam, int64_t npoints, int32_t nseams,
                      double factor, int32_t *keep) {
  const char *fn = "aql_keep_outliers";
  REQUIRE(npoints >= 0 && nseams >= 0, AQL_ERR_SHAPE, "%s: counts must be >= 0", fn);
  REQUIRE((npoints == 0 || (amax && seam)) && (nseams == 0 || keep), AQL_ERR_NULL,
          "%s: arrays must not be NULL", fn);
  for (int64_t p = 0; p < npoints; ++p)
    REQUIRE(seam[p] >= 0 && seam[p] < nseams, AQL_ERR_PARAM,
            "%s: point %lld names seam %d of %d", fn, (long long)p, (int)seam[p], (int)nseams);
  for (int32_t i = 0; i < nseams; ++i) keep[i] = 0;
  if (factor == 0.0) return ok();
  std::vector<double> vals;
  for (int64_t p = 0; p < npoints; ++p)
    if (!std::isnan(amax[p]) && amax[p] > 0.0f) vals.push_back((double)amax[p]);
  if (vals.empty()) return ok();
  std::sort(vals.begin(), vals.end());
  const size_t n = vals.size();
  const double median = n % 2 ? vals[n / 2] : (vals[n / 2 - 1] + vals[n / 2]) / 2.0;
  std::vector<double> worst((size_t)nseams, -INFINITY);
  std::vector<char> seen((size_t)nseams, 0);
  for (int64_t p = 0; p < npoints; ++p) {
    if (std::isnan(amax[p])) continue;
    const double v = (double)amax[p];
    if (!seen[seam[p]] || v > worst[seam[p]]) worst[seam[p]] = v;
    seen[seam[p]] = 1;
  }
  for (int32_t i = 0; i < nseams; ++i) keep[i] = seen[i] && worst[i] > factor * median;
  return ok();
}

int aql_gptq_int8(const float *w, int64_t N, int64_t K, const double *H, double damp,
                  int64_t block, int8_t *q, float *scale, int32_t *wsum, double *hinv_out,
                  int32_t *info, void *ws, size_t ws_bytes, void *stream) {
  const char *fn = "aql_gptq_int8";
  REQUIRE(N >= 0 && K >= 4 && K % 4 == 0 && K <= AQL_MAX_K_INT8, AQL_ERR_SHAPE,
          "%s: need N >= 0, 4 <= K <= %d and K %% 4 == 0 (N=%lld K=%lld)", fn, AQL_MAX_K_INT8,
          (long long)N, (long long)K);
  REQUIRE(block >= 1 && block <= aql::kGptqMaxBlock, AQL_ERR_SHAPE,
          "%s: block must be in 1..%d (got %lld)", fn, aql::kGptqMaxBlock, (long long)block);
  REQUIRE(std::isfinite(damp) && damp >= 0.0, AQL_ERR_PARAM,
          "%s: damp must be finite and >= 0", fn);
  REQUIRE(aligned16(w) && aligned16(H) && aligned16(q) && aligned16(scale) && aligned16(wsum) &&
              aligned16(hinv_out) && aligned16(info) && aligned16(ws),
          AQL_ERR_ALIGN, "%s: pointers must be 16-byte aligned", fn);
  if (N == 0) return ok();
  REQUIRE(w && H && q && scale && info, AQL_ERR_NULL,
          "%s: w, H, q, scale and info must not be NULL", fn);
  const size_t need = aql::gptq_workspace_bytes(N, K, block);
  REQUIRE(ws && ws_bytes >= need, AQL_ERR_WORKSPACE, "%s: workspace of %zu bytes needed", fn,
          need);
  if (int e = check_device(fn)) return e;
  return launched(aql::launch_gptq_int8(w, N, K, H, damp, (int)block, q, scale, wsum, hinv_out,
                                        info, ws, (hipStream_t)stream),
                  fn);
}

int aql_measure_read(const void *buf, int64_t bytes, uint32_t *sink, void *stream) {
  const char *fn = "aql_measure_read";
  REQUIRE(buf && sink, AQL_ERR_NULL, "%s: buf and sink must not be NULL", fn);
  REQUIRE(aligned16(buf) && aligned16(sink), AQL_ERR_ALIGN, "%s: pointers must be 16-byte aligned",
          fn);
  REQUIRE(bytes >= 1024 && bytes % 1024 == 0 && bytes <= (1LL << 31) - 1024, AQL_ERR_SHAPE,
          "%s: bytes must be a multiple of 1024 in [1024, 2^31 - 1024] (got %lld)", fn,
          (long long)bytes);
  if (int e = check_device(fn)) return e;
  return launched(aql::launch_measure_read(buf, bytes, sink, (hipStream_t)stream), fn);
}

int aql_measure_mfma_i8(int64_t iters, int32_t *sink, void *stream) {
  const char *fn = "aql_measure_mfma_i8";
  REQUIRE(sink, AQL_ERR_NULL, "%s: sink must not be NULL", fn);
  REQUIRE(aligned16(sink), AQL_ERR_ALIGN, "%s: sink must be 16-byte aligned", fn);
  REQUIRE(iters >= 1 && iters <= (1LL << 30), AQL_ERR_SHAPE, "%s: iters must be in [1, 2^30]", fn);
  if (int e = check_device(fn)) return e;
  return launched(aql::launch_measure_mfma_i8(iters, sink, (hipStream_t)stream), fn);
}

}  // extern "C"
