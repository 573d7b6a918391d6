// tile_order.h — which output tiles a persistent workgroup of the GEMMs computes.
//
// The dispatcher places workgroup b on XCD b % X (X = the device's XCD count; one XCD when
// the partition exposes only one). Each XCD takes one contiguous range of the tile list,
// so the tiles that share operand rows run on the same L2: XCD x owns tiles
// [x T / X, (x + 1) T / X), and its workgroups b = x, x + X, x + 2X, ... take every
// n-th tile of that range, n being the number of workgroups on XCD x. With fewer workgroups
// than XCDs the split would leave ranges without a workgroup, so such grids stride the
// whole list instead.
//
// Plain C++ (no HIP types) so that the host tests can check the coverage directly.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define FP8Q_HD __host__ __device__
#else
#define FP8Q_HD
#endif

namespace fp8q {

struct TileSpan {
  int64_t beg, end, stride;  // tiles beg, beg + stride, ... < end
};

FP8Q_HD inline TileSpan tile_span(int64_t tiles, int64_t block, int64_t grid, int64_t xcds) {
  TileSpan s;
  if (xcds <= 1 || grid < xcds) {
    s.beg = block;
    s.end = tiles;
    s.stride = grid;
    return s;
  }
  const int64_t x = block % xcds;
  s.beg = (x * tiles) / xcds + block / xcds;
  s.end = ((x + 1) * tiles) / xcds;
  s.stride = (grid - x + xcds - 1) / xcds;  // workgroups on XCD x
  return s;
}

}  // namespace fp8q
