"""The persistent GEMM grids' tile split (fp8_group_quant_amd/csrc/tile_order.h), compiled for
the host: every tile of the list is computed by exactly one workgroup, for grids that are or
are not multiples of the XCD count, smaller than it, and for one-XCD partitions."""
import os
import subprocess
import tempfile

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

DRIVER = r"""
#include <cstdio>
#include <vector>
#include "tile_order.h"
int main() {
  const long tiles_list[] = {0, 1, 5, 8, 63, 64, 255, 256, 257, 896, 1023, 1024, 7833, 100000};
  const long grids[] = {1, 3, 7, 8, 9, 64, 200, 248, 255, 256, 257, 304};
  const long xcds_list[] = {1, 2, 4, 8};
  long bad = 0, cases = 0;
  for (long T : tiles_list)
    for (long grid : grids)
      for (long X : xcds_list) {
        std::vector<int> hits(T, 0);
        for (long b = 0; b < grid; b++) {
          const fp8q::TileSpan s = fp8q::tile_span(T, b, grid, X);
          if (s.stride < 1) { bad++; break; }
          for (long t = s.beg; t < s.end; t += s.stride) {
            if (t < 0 || t >= T) { bad++; break; }
            hits[t]++;
          }
        }
        for (long t = 0; t < T; t++) bad += hits[t] != 1;
        cases++;
      }
  std::printf("%ld %ld\n", cases, bad);
  return bad != 0;
}
"""


def test_every_tile_exactly_once():
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "drv.cpp")
        exe = os.path.join(d, "drv")
        with open(src, "w") as f:
            f.write(DRIVER)
        subprocess.run(["g++", "-O1", "-std=c++17", "-I", os.path.join(ROOT, "fp8_group_quant_amd", "csrc"),
                        src, "-o", exe], check=True)
        r = subprocess.run([exe], capture_output=True, text=True)
        cases, bad = map(int, r.stdout.split())
        assert cases == 14 * 12 * 4 and bad == 0, r.stdout
