// Weight-only W8A16 GEMV / skinny-GEMM launchers and launch shapes (internal
// to libaql.so). Each returns hipSuccess or the launch error; arguments are
// validated by the C ABI layer.
#pragma once

#include "common.h"

namespace aql {

// part (may be null): device memory for split-K partial sums; with at least
// w8a16_skinny_part_bytes(M, N, K) bytes the shapes that split do so.
hipError_t launch_w8a16(const uint16_t *x, int64_t M, int64_t K, const int8_t *q,
                        const float *scale, const uint16_t *bias, int64_t N, uint16_t *y,
                        float *part, size_t part_bytes, hipStream_t st);

// K splits of the shared-x skinny tile below kW8A16ShareMinN channels (1: the
// shape does not split): 12 <= M < 64, K >= 8192, 4 splits up to 128 tiles of
// 64 channels x 16 rows, 2 up to 256, so the grid fills the CUs. The fp32
// partial sums then need w8a16_skinny_part_bytes(M, N, K) bytes.
int w8a16_skinny_splits(int64_t M, int64_t N, int64_t K);
size_t w8a16_skinny_part_bytes(int64_t M, int64_t N, int64_t K);

// Single-row GEMV over contiguous 1 KB row pieces, used by launch_w8a16 for
// M = 1 and kW8A16ContigMinK <= K <= kW8A16ContigMaxK (measured faster than the
// 4-row tile there: 10.8 vs 11.3 us at K = 4096, N = 14336; 12.1 vs 12.9 at
// K = N = 8192; longer rows stream better in the tile's form).
constexpr int64_t kW8A16ContigMinK = 2048;
constexpr int64_t kW8A16ContigMaxK = 8192;
hipError_t launch_w8a16_m1c(const uint16_t *x, int64_t K, const int8_t *q, const float *scale,
                            const uint16_t *bias, int64_t N, uint16_t *y, hipStream_t st);

// 2 <= M <= kW8A16FewMaxM rows over contiguous row pieces (bf16 dot2 on the
// widened weights), used by launch_w8a16 for kW8A16FewMinK <= K <= kW8A16FewMaxK.
constexpr int64_t kW8A16FewMaxM = 4;
constexpr int64_t kW8A16FewMinK = 2048;
constexpr int64_t kW8A16FewMaxK = 16384;
hipError_t launch_w8a16_mfew(const uint16_t *x, int64_t M, int64_t K, const int8_t *q,
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
// From this many channels launch_w8a16 runs the skinny tile's shared-x form
// (64 channels a workgroup, x copied into LDS once per step for 4 waves).
constexpr int64_t kW8A16ShareMinN = 8192;
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

// Small groups travel by value in the kernel arguments.
constexpr int kW8A16InlineMax = 4;
struct W8A16InlineGroup {
  W8A16GroupEntry e[kW8A16InlineMax];
};

hipError_t launch_w8a16_grouped(const W8A16GroupEntry *dev_tab, int count, int total_blocks,
                                const W8A16Shape &sh, hipStream_t st);

// Grouped single-row GEMVs over contiguous 1 KB row pieces, for groups whose
// problems all have M = 1 and kW8A16PiecesMinK <= K <= kW8A16PiecesMaxK. A
// problem's tiles (workgroups of 4 waves) cover 32 channels when K <= 1024 and
// 8 channels otherwise (w8a16_pieces_tile_channels).
constexpr int64_t kW8A16PiecesMinK = 768;
constexpr int64_t kW8A16PiecesMaxK = 4096;
constexpr int64_t w8a16_pieces_tile_channels(int64_t K) { return K > 1024 ? 8 : 32; }
// host_tab (may be NULL): the same entries in host memory; a group of at most
// kW8A16InlineMax entries then goes by value in the kernel arguments
hipError_t launch_w8a16_m1p_grouped(const W8A16GroupEntry *dev_tab, const W8A16GroupEntry *host_tab,
                                    int count, int total_blocks, hipStream_t st);

}  // namespace aql
