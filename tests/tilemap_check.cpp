// Host-only check of the matrix-core product's workgroup orders
// (int8_block_scaled_amd/csrc/q8_tilemap.h): every order the launcher may
// use is a bijection from workgroup ids onto the tile grid, the automatic
// choice is always admissible, and inadmissible orders are rejected; the
// automatic tile choice always fits its 32-bit buffer ranges.
// Prints one line per failure and exits non-zero if there is any.
#include <cstdio>
#include <vector>

#include "q8_tilemap.h"

static int failures = 0;

static void fail(const char* what, int tm, int tn, int order) {
  if (++failures <= 20) std::printf("FAIL %s: tiles %dx%d order %d\n", what, tm, tn, order);
}

// tile_of(., order) covers every tile exactly once.
static bool bijective(int tiles_m, int tiles_n, int order) {
  const int grid = tiles_m * tiles_n;
  std::vector<unsigned char> seen(static_cast<size_t>(grid), 0);
  for (int b = 0; b < grid; ++b) {
    const q8::TileCoord c = q8::tile_of(b, grid, tiles_m, order);
    if (c.tm < 0 || c.tm >= tiles_m || c.tn < 0 || c.tn >= tiles_n) return false;
    unsigned char& s = seen[static_cast<size_t>(c.tn) * tiles_m + c.tm];
    if (s) return false;
    s = 1;
  }
  return true;
}

int main() {
  long checked = 0, rejected = 0;
  std::vector<std::pair<int, int>> grids;
  for (int tm = 1; tm <= 40; ++tm)
    for (int tn = 1; tn <= 40; ++tn) grids.push_back({tm, tn});
  // grids of the benchmark workloads (128x128 and 64x128 tiles)
  const int extra[][2] = {{16, 96}, {64, 136}, {64, 40}, {4, 48}, {4, 32}, {4, 192}, {8, 96},
                          {32, 96}, {128, 136}, {8, 32}, {8, 48}, {8, 192}};
  for (auto& g : extra) grids.push_back({g[0], g[1]});
  for (auto& g : grids) {
    const int tm = g.first, tn = g.second;
    for (int order = -2; order <= 17; ++order) {
      if (!q8::order_admissible(order, tm, tn)) {
        ++rejected;
        continue;
      }
      ++checked;
      if (!bijective(tm, tn, order)) fail("admissible order is not a bijection", tm, tn, order);
    }
    for (long long K : {32LL, 4096LL, 17408LL, 1LL << 24})
      for (long long bm : {64LL, 128LL}) {
        const int order = q8::choose_order(tm, tn, bm, K);
        if (!q8::order_admissible(order, tm, tn)) fail("chosen order not admissible", tm, tn, order);
      }
  }
  // The automatic tile choice: always a configuration whose 32-bit buffer
  // ranges hold K, for K up to 2^24; and the expected tile on the benchmark
  // workloads.
  long tiles_checked = 0;
  for (long long M : {65LL, 96LL, 128LL, 509LL, 512LL, 1024LL, 2048LL, 4096LL, 8192LL, 32768LL})
    for (long long N : {64LL, 384LL, 4096LL, 5120LL, 6144LL, 12288LL, 17408LL, 24576LL, 98304LL})
      for (long long K : {32LL, 4096LL, 17408LL, (1LL << 22), 11184800LL, 11184832LL, (1LL << 24)}) {
        const int t = q8::choose_tile(M, N, K);
        ++tiles_checked;
        if (t < 0 || t >= q8::kNumTileDims) {
          fail("tile index out of the table", static_cast<int>(M), static_cast<int>(N), t);
          continue;
        }
        if (!q8::buffer_ranges_fit(q8::kTileDims[t].bm, q8::kTileDims[t].bn, K))
          fail("chosen tile's buffer ranges cannot hold K", static_cast<int>(M),
               static_cast<int>(K >> 10), t);
      }
  const struct { long long M, N, K; int tile; } want[] = {
      {2048, 12288, 4096, 9},  {8192, 17408, 5120, 9}, {8192, 5120, 17408, 4},
      {2048, 17408, 5120, 9},  {2048, 8192, 8192, 4},  {4096, 8192, 8192, 4},
      {512, 6144, 4096, 8},    {509, 6144, 4096, 8},   {512, 4096, 4096, 6},
      {512, 24576, 4096, 9},   {512, 4096, 12288, 6},  {128, 4096, 4096, 5},
      // the 128x384 tile cannot hold K >= 2^32 / 384: the 128x128 tile instead
      {2048, 12288, 1LL << 24, 4}};
  for (auto& w : want) {
    const int t = q8::choose_tile(w.M, w.N, w.K);
    if (t != w.tile) fail("unexpected tile for a workload", static_cast<int>(w.M),
                          static_cast<int>(w.N), t);
  }
  // cases that break the map if let through (tile index past the grid, or a
  // division by zero), which the launcher must therefore reject
  if (q8::order_admissible(2, 3, 8)) fail("order 2 on a 3x8 grid admitted", 3, 8, 2);
  if (bijective(3, 8, 2)) fail("order 2 on a 3x8 grid unexpectedly bijective", 3, 8, 2);
  if (q8::order_admissible(16, 16, 96)) fail("order 16 admitted", 16, 96, 16);
  if (q8::order_admissible(3, 16, 96)) fail("order 3 admitted", 16, 96, 3);
  if (q8::order_admissible(1, 3, 5)) fail("order 1 on 15 tiles admitted", 3, 5, 1);
  // the prefill grid takes the 2 x 4 rectangles
  if (q8::choose_order(16, 96, 128, 4096) != 2) fail("prefill grid order", 16, 96, 2);
  // a grid whose rows fit no rectangle's L2 share takes the plain order
  // (large down: 64 x 40 tiles of 128 rows at K = 17408), and a grid whose
  // rows all fit takes the contiguous one (M512 on 128-row tiles)
  if (q8::choose_order(64, 40, 128, 17408) != 0) fail("large grid order", 64, 40, 0);
  if (q8::choose_order(4, 64, 128, 4096) != 1) fail("small grid order", 4, 64, 1);
  // 32-bit buffer ranges: a 128x256 tile cannot hold K = 2^24, a 128x128 can
  if (q8::buffer_ranges_fit(128, 256, 1LL << 24)) fail("128x256 at K=2^24 fits", 128, 256, 0);
  if (!q8::buffer_ranges_fit(128, 128, 1LL << 24)) fail("128x128 at K=2^24 does not fit", 128, 128, 0);
  std::printf("orders checked %ld, rejected %ld, failures %d\n", checked, rejected, failures);
  return failures ? 1 : 0;
}
