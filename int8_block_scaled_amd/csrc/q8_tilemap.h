// q8_tilemap.h -- workgroup order of the matrix-core product: which output
// tile a workgroup computes, and which orders a tile grid admits.
//
// Hardware workgroup id i runs on XCD i % 8, and each XCD has its own L2.
// The orders:
//   0      plain: tile (tm, tn) = (i % tiles_m, i / tiles_m), M fastest;
//   1      contiguous: XCD x takes the logical tiles x*G/8 .. (x+1)*G/8 - 1
//          (G = tiles_m * tiles_n), M fastest within them, so consecutive
//          tiles of one XCD share weight columns in its L2;
//   sm in {2, 4, 8}: the grid is cut into sm x (8/sm) rectangles of
//          (tiles_m/sm) x (tiles_n/(8/sm)) tiles, one per XCD, M fastest
//          within a rectangle, so an XCD needs only 1/sm of the activation
//          rows.
// Order 1 needs G % 8 == 0; order sm needs tiles_m % sm == 0 and
// tiles_n % (8/sm) == 0.  Under those conditions each order is a bijection
// from [0, G) onto the tile grid; order_admissible() is the check, and the
// launcher never passes an order that fails it.
//
// Plain C++ so that a host-only unit test can include it; the kernels use
// the same inline function.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define Q8_HOST_DEVICE __host__ __device__
#else
#define Q8_HOST_DEVICE
#endif

namespace q8 {

struct TileCoord {
  int tm, tn;
};

Q8_HOST_DEVICE inline TileCoord tile_of(int bid, int grid, int tiles_m, int order) {
  TileCoord c;
  if (order >= 2) {
    const int sm = order, sn = 8 / order;
    const int tmx = tiles_m / sm, tnx = grid / tiles_m / sn;
    const int x = bid & 7, local = bid >> 3;
    c.tm = (x % sm) * tmx + local % tmx;
    c.tn = (x / sm) * tnx + local / tmx;
  } else {
    int b = bid;
    if (order == 1) {
      const int per = grid >> 3;
      b = (b & 7) * per + (b >> 3);
    }
    c.tm = b % tiles_m;
    c.tn = b / tiles_m;
  }
  return c;
}

inline bool order_admissible(int order, int64_t tiles_m, int64_t tiles_n) {
  if (tiles_m < 1 || tiles_n < 1) return false;
  switch (order) {
    case 0: return true;
    case 1: return (tiles_m * tiles_n) % 8 == 0;
    case 2: case 4: case 8: return tiles_m % order == 0 && tiles_n % (8 / order) == 0;
    default: return false;
  }
}

// The order the launcher picks: contiguous per XCD when the grid splits
// evenly over the 8 XCDs and the activation rows of a tile column (tiles_m
// * BM rows of K bytes) fit an XCD's 4 MB L2; rectangles when the rows of
// one rectangle do; otherwise plain.  In that last case the contiguous
// order would give each XCD a strip of one tile column, whose concurrent
// tiles all read different activation rows, while the plain order spreads
// an XCD's concurrent tiles over a few rows and columns of tiles.
inline int choose_order(int64_t tiles_m, int64_t tiles_n, int64_t bm, int64_t K) {
  if ((tiles_m * tiles_n) % 8 != 0) return 0;
  constexpr int64_t kL2Bytes = int64_t(4) << 20;
  if (tiles_m * bm * K <= kL2Bytes) return 1;
  for (int sm = 2; sm <= 8; sm *= 2)
    if (order_admissible(sm, tiles_m, tiles_n) && tiles_m / sm * bm * K <= kL2Bytes) return sm;
  return 0;
}

// A BM x BN tile addresses its BM rows of q_a (BM*K bytes) and its BN/64
// packed weight groups (BN*K bytes) through 32-bit buffer ranges.
inline bool buffer_ranges_fit(int64_t bm, int64_t bn, int64_t K) {
  constexpr int64_t kRange = int64_t(1) << 32;
  return bm * K < kRange && bn * K < kRange;
}

// Output tile of each compiled matrix-core configuration, by index (the
// kernels' table is checked against it at compile time).
struct TileDims {
  int bm, bn;
};
constexpr TileDims kTileDims[] = {
    {128, 128},   // 0: 8 waves of 32x64
    {64, 128},    // 1: 4 waves of 32x64
    {128, 128},   // 2: as 0 on 16x16 MFMAs
    {128, 256},   // 3: 16 waves of 32x64
    {128, 128},   // 4: as 0, MFMAs first
    {64, 64},     // 5: 4 K groups of 2 waves
    {64, 128},    // 6: 2 K groups of 4 waves, stages of 8, MFMAs first
    {64, 128},    // 7: 2 K groups of 4 waves, stages of 4
    {64, 192},    // 8: 2 K groups of 6 waves
    {128, 384},   // 9: 12 waves of 32x128
};
constexpr int kNumTileDims = static_cast<int>(sizeof(kTileDims) / sizeof(kTileDims[0]));

// The configuration the launcher takes for an M x N x K product (M > 64):
//  - 128x384 tiles when they make at least one round of the 256 CUs (one
//    workgroup per CU) and the work they waste -- the unused columns of a
//    ragged last column tile, the unused rows of a ragged last row tile and
//    the idle CUs of a partial last round -- leaves them within 10 % of the
//    128x128 tiles' useful fraction (which waste the same way, at two
//    workgroups per CU); per launch round the 128x384 tile does about 10 %
//    more work per unit time than the 128x128 tile (measured on gfx950:
//    M8192 N17408 K5120 1745 vs 1880 us, 11.5 rounds; M8192 N5120 K17408
//    1830 vs 1802 us, 3.5 rounds and a third of a column tile idle);
//  - 128x128 tiles when there are at least two per CU;
//  - 64x192 tiles when N is whole 192-column tiles and they make 3/4 to 1
//    tile per CU;
//  - 64x128 tiles in stages of 4 (two workgroups per CU) when they are more
//    than one per CU, in stages of 8 (one per CU) from 3/4 to 1 per CU;
//  - else 64x64 tiles in four K groups.
// A candidate whose 32-bit buffer ranges cannot hold K is passed over (the
// 128x128 and smaller tiles hold every K up to 2^24).
// Useful fraction of a launch of bm x bn tiles, `slots` resident at a time:
// the product's outputs over the outputs of the tiles' whole rounds.
inline double launch_fill(int64_t M, int64_t N, int bm, int bn, int64_t slots) {
  const int64_t tm = (M + bm - 1) / bm, tn = (N + bn - 1) / bn;
  const int64_t rounds = (tm * tn + slots - 1) / slots;
  return static_cast<double>(M) * static_cast<double>(N) /
         (static_cast<double>(rounds * slots) * bm * bn);
}

inline int choose_tile(int64_t M, int64_t N, int64_t K) {
  auto fits = [K](int t) { return buffer_ranges_fit(kTileDims[t].bm, kTileDims[t].bn, K); };
  const int64_t t128 = ((M + 127) / 128) * ((N + 127) / 128);
  const int64_t t64 = ((M + 63) / 64) * ((N + 127) / 128);
  const int64_t t192 = ((M + 63) / 64) * (N / 192);
  const int64_t t384 = ((M + 127) / 128) * ((N + 383) / 384);
  if (t384 >= 256 && fits(9) &&
      1.1 * launch_fill(M, N, 128, 384, 256) >= launch_fill(M, N, 128, 128, 512))
    return 9;
  if (t128 >= 512) return 4;
  if (N % 192 == 0 && t192 >= 192 && t192 <= 256 && fits(8)) return 8;
  if (t64 > 256) return 7;
  if (t64 >= 192) return 6;
  return 5;
}

}  // namespace q8
