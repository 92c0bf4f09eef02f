// Weight-only W8A16 GEMV / skinny-GEMM launchers and launch shapes (internal
// to libaql.so). Each returns hipSuccess or the launch error; arguments are
// validated by the C ABI layer.
#pragma once

#include "common.h"

namespace aql {

hipError_t launch_w8a16(const uint16_t *x, int64_t M, int64_t K, const int8_t *q,
                        const float *scale, const uint16_t *bias, int64_t N, uint16_t *y,
                        hipStream_t st);

// Launch shape of the W8A16 kernel: waves per channel group (they split K),
// groups of 4 output channels per wave tile (1, 2 or 4) and blocks of 4 rows of
// x per tile (1, 2 or 4; 0 selects the single-row tile, M = 1; kW8A16Skinny
// selects the 16-row skinny tile on 16x16x32 MFMAs, with 4 or 8 channel
// groups). The single-row
// tile also takes cgroups, wave tiles along N per workgroup (1, 2 or 4), and
// xlds, the LDS bytes the workgroup copies x into (0: each wave loads its x
// from memory; else 2 K rounded up to 1 KiB for the largest K it serves).
struct W8A16Shape {
  int waves, tgroups, mblocks;
  int cgroups = 1;
  int xlds = 0;
};
W8A16Shape w8a16_shape(int64_t M, int64_t N, int64_t K);
constexpr int kW8A16Skinny = 16;     // mblocks value of the skinny tile
constexpr int kW8A16SkinnyMinM = 4;  // rows from which the skinny tile serves (up to the GEMM band)
// LDS budget for x in the single-row tile (K <= 16384), and the xlds value for
// a given K (0 past the budget).
constexpr int kW8A16MaxXlds = 32768;
int w8a16_xlds_bytes(int64_t K);
hipError_t launch_w8a16_shape(const W8A16Shape &sh, const uint16_t *x, int64_t M, int64_t K,
                              const int8_t *q, const float *scale, const uint16_t *bias,
                              int64_t N, uint16_t *y, hipStream_t st);

// One problem of a grouped W8A16 launch, as stored in the device table.
struct W8A16GroupEntry {
  const uint16_t *x;
  const int8_t *q;
  const float *scale;
  const uint16_t *bias;
  uint16_t *y;
  int64_t M, N, K;
  int32_t blk_begin;  // first grid block of this problem
  int32_t nblk;       // tiles along N
  int32_t pad[2];
};
static_assert(sizeof(W8A16GroupEntry) == 80, "table layout");

hipError_t launch_w8a16_grouped(const W8A16GroupEntry *dev_tab, int count, int total_blocks,
                                const W8A16Shape &sh, hipStream_t st);

}  // namespace aql
