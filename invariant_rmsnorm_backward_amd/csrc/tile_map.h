// Workgroup order over the output tiles of the matrix-core kernels (y, dX and
// the dW group chains).  The order decides only which workgroup computes a
// tile, never a bit of the result.
//
// The grid of tmc x tnc tiles is cut into 4 x 8 super-blocks (those on the
// right and bottom edges may hang over the grid).  XCD x -- the chip hands
// workgroup id to XCD id % 8 -- takes super-blocks x, x + 8, ..., so the 32
// workgroups one XCD runs at a time share 4 row blocks and 8 column blocks
// of the operands in its L2.  The launch then holds whole super-blocks, their
// number rounded up to a multiple of 8, and a workgroup whose tile lies
// outside the grid exits at once.  Where that would add more than 1/16 to
// the grid (small grids), one workgroup per tile in column-major order.
//
// constexpr functions compile for the host (the launch size, a CPU check of
// the map) and for the device alike.
#pragma once

#include <cstdint>

namespace rbi {
namespace lin {

constexpr int kSuperRows = 4;   // tile rows per super-block
constexpr int kSuperCols = 8;   // tile columns per super-block

// Workgroups that whole super-blocks take, rounded up to a multiple of 8.
constexpr int64_t sb_slots(int64_t tmc, int64_t tnc) {
  const int64_t sb = ((tmc + kSuperRows - 1) / kSuperRows) * ((tnc + kSuperCols - 1) / kSuperCols);
  return (sb + 7) / 8 * 8 * kSuperRows * kSuperCols;
}
constexpr bool sb_order(int64_t tmc, int64_t tnc) {
  return sb_slots(tmc, tnc) * 16 <= tmc * tnc * 17;
}
// Workgroups a tmc x tnc grid launches.
constexpr int64_t tile_slots(int64_t tmc, int64_t tnc) {
  return sb_order(tmc, tnc) ? sb_slots(tmc, tnc) : tmc * tnc;
}
// Tile (tm, tn) of workgroup id (0 <= id < tile_slots); false: no tile, the
// workgroup exits.
constexpr bool xcd_tile(int id, int tmc, int tnc, int& tm, int& tn) {
  if (!sb_order(tmc, tnc)) {
    tm = id % tmc;
    tn = id / tmc;
    return true;
  }
  const int sbm = (tmc + kSuperRows - 1) / kSuperRows;
  const int xcd = id & 7, slot = id >> 3;
  const int sb = (slot >> 5) * 8 + xcd, w = slot & 31;
  tm = (sb % sbm) * kSuperRows + w % kSuperRows;
  tn = (sb / sbm) * kSuperCols + w / kSuperRows;
  return tm < tmc && tn < tnc;
}

}  // namespace lin
}  // namespace rbi
