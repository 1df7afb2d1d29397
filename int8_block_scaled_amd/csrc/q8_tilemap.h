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
// evenly over the 8 XCDs, and rectangles when one XCD's share of activation
// rows (tiles_m * BM rows of K bytes) would not fit its 4 MB L2.
inline int choose_order(int64_t tiles_m, int64_t tiles_n, int64_t bm, int64_t K) {
  if ((tiles_m * tiles_n) % 8 != 0) return 0;
  constexpr int64_t kL2Bytes = int64_t(4) << 20;
  if (tiles_m * bm * K > kL2Bytes)
    for (int sm = 2; sm <= 8; sm *= 2)
      if (order_admissible(sm, tiles_m, tiles_n) && tiles_m / sm * bm * K <= kL2Bytes) return sm;
  return 1;
}

// A BM x BN tile addresses its BM rows of q_a (BM*K bytes) and its BN/64
// packed weight groups (BN*K bytes) through 32-bit buffer ranges.
inline bool buffer_ranges_fit(int64_t bm, int64_t bn, int64_t K) {
  constexpr int64_t kRange = int64_t(1) << 32;
  return bm * K < kRange && bn * K < kRange;
}

}  // namespace q8
