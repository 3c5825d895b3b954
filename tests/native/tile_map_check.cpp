// Host check of the matrix-core kernels' workgroup-to-tile map, built with
// AddressSanitizer + UndefinedBehaviorSanitizer by tests/test_sanitizers.py:
// over every grid up to 80 x 80 tiles and the shapes of the 4096-wide layers
// and an LM head, the workgroups of a launch take every tile exactly once,
// none gets a tile outside the grid, the super-block order is kept for every
// grid that 4 x 8 super-blocks tile in a multiple of 8, and the extra
// workgroups stay within 1/16 of the grid.
#include <cstdio>
#include <vector>

#include "tile_map.h"

using namespace rbi::lin;

static int fails = 0;
#define CHECK(c) do { if (!(c)) { std::printf("FAIL %s:%d %s\n", __FILE__, __LINE__, #c); ++fails; } } while (0)

static void check_grid(int tmc, int tnc) {
  const int64_t slots = tile_slots(tmc, tnc);
  CHECK(slots >= (int64_t)tmc * tnc);
  CHECK(slots * 16 <= (int64_t)tmc * tnc * 17);
  std::vector<int> hits((size_t)tmc * tnc, 0);
  for (int64_t id = 0; id < slots; ++id) {
    int tm = -1, tn = -1;
    if (!xcd_tile((int)id, tmc, tnc, tm, tn)) continue;
    CHECK(tm >= 0 && tm < tmc && tn >= 0 && tn < tnc);
    if (tm >= 0 && tm < tmc && tn >= 0 && tn < tnc) ++hits[(size_t)tn * tmc + tm];
  }
  for (int h : hits) CHECK(h == 1);
  // exactly tiled grids keep the super-block order with no extra workgroup
  if (tmc % kSuperRows == 0 && tnc % kSuperCols == 0 &&
      ((tmc / kSuperRows) * (tnc / kSuperCols)) % 8 == 0) {
    CHECK(sb_order(tmc, tnc));
    CHECK(slots == (int64_t)tmc * tnc);
  }
  // in super-block order, the 32 workgroups an XCD runs at a time (ids
  // x, x + 8, ..., x + 248 of each 256) touch at most 4 row and 8 column blocks
  if (sb_order(tmc, tnc)) {
    for (int64_t base = 0; base < slots; base += 256)
      for (int x = 0; x < 8; ++x) {
        int rmin = 1 << 30, rmax = -1, cmin = 1 << 30, cmax = -1;
        for (int j = 0; j < 32; ++j) {
          int tm = 0, tn = 0;
          if (!xcd_tile((int)(base + x + 8 * j), tmc, tnc, tm, tn)) continue;
          rmin = tm < rmin ? tm : rmin; rmax = tm > rmax ? tm : rmax;
          cmin = tn < cmin ? tn : cmin; cmax = tn > cmax ? tn : cmax;
        }
        if (rmax >= 0) CHECK(rmax - rmin < kSuperRows && cmax - cmin < kSuperCols);
      }
  }
}

int main() {
  for (int tmc = 1; tmc <= 80; ++tmc)
    for (int tnc = 1; tnc <= 80; ++tnc) check_grid(tmc, tnc);
  // 32,768 rows x 4096 and 32,000 outputs in 256-wide tiles; the dW grids
  check_grid(128, 16);
  check_grid(128, 125);
  check_grid(125, 16);
  check_grid(16, 16);
  CHECK(sb_order(128, 125) && tile_slots(128, 125) == 16384);
  CHECK(sb_order(125, 16) && tile_slots(125, 16) == 2048);
  if (fails) {
    std::printf("tile map: %d failures\n", fails);
    return 1;
  }
  std::printf("tile map: ok\n");
  return 0;
}
