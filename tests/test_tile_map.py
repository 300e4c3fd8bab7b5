"""Host-side check of the workgroup -> tile maps of the GEMM kernels
(csrc/common.hpp): every tile of a launch is taken by exactly one workgroup,
the chunked map keeps the promised locality, and the grouped tile orders of
the 256-wide kernels visit every tile of a full grid or lower triangle once
for every group height a tuning hint may set.  The header is compiled
into a small host program with hipcc (no GPU needed)."""
import os
import shutil
import subprocess

import pytest

CSRC = os.path.join(os.path.dirname(os.path.dirname(__file__)), "matrix_aware_optimizer_muon_amd",
                    "csrc")

PROGRAM = r"""
#include <cmath>
#include <cstdio>
#include <vector>
#include "common.hpp"
using namespace muon;
int main() {
  const unsigned totals[] = {1, 7, 8, 9, 63, 64, 65, 168, 255, 256, 257, 1023, 1024, 1036, 2940,
                             5880, 10976, 29008, 58016};
  const unsigned chunks[] = {0, 1, 3, 25, 64, 128, 130, 4096};
  for (unsigned total : totals)
    for (unsigned C : chunks) {
      std::vector<int> seen(total, 0);
      for (unsigned b = 0; b < total; ++b) {
        const unsigned t = C ? xcd_remap_chunked(b, total, C) : xcd_remap(b, total);
        if (t >= total) { printf("out of range total=%u C=%u b=%u t=%u\n", total, C, b, t); return 1; }
        ++seen[t];
      }
      for (unsigned t = 0; t < total; ++t)
        if (seen[t] != 1) { printf("tile %u taken %d times (total=%u C=%u)\n", t, seen[t], total, C); return 1; }
      // locality: inside whole windows, the k-th run of XCD x is the
      // consecutive range [k 8C + x C, +C)
      if (C) {
        const unsigned span = 8 * C, full = total / span;
        for (unsigned b = 0; b < full * span; ++b) {
          const unsigned x = b % 8, slot = b / 8;
          const unsigned want = (slot / C) * span + x * C + slot % C;
          if (xcd_remap_chunked(b, total, C) != want) { printf("run order total=%u C=%u\n", total, C); return 1; }
        }
      }
    }
  // tile-order maps of the 256-wide kernels, every group height a hint may
  // set: each (row, column) tile of a full grid / lower triangle once
  for (int G = 1; G <= 64; ++G) {
    for (int tm : {1, 2, 3, 7, 14, 16, 74}) {
      for (int tn : {1, 3, 14, 74}) {
        std::vector<int> seen(tm * tn, 0);
        for (int t = 0; t < tm * tn; ++t) {
          int i, j;
          full_tile_grouped(t, tm, tn, G, &i, &j);
          if (i < 0 || i >= tm || j < 0 || j >= tn) { printf("full out of range G=%d\n", G); return 1; }
          ++seen[i * tn + j];
        }
        for (int v : seen) if (v != 1) { printf("full not a bijection G=%d %dx%d\n", G, tm, tn); return 1; }
      }
    }
    for (int T : {1, 2, 3, 4, 5, 14, 16, 17, 64}) {
      std::vector<int> seen(T * T, 0);
      for (int t = 0; t < T * (T + 1) / 2; ++t) {
        int i, j;
        tri_tile_grouped(t, T, G, &i, &j);
        if (j < 0 || i < j || i >= T) { printf("tri out of range G=%d T=%d t=%d\n", G, T, t); return 1; }
        ++seen[i * T + j];
      }
      for (int i = 0; i < T; ++i)
        for (int j = 0; j <= i; ++j)
          if (seen[i * T + j] != 1) { printf("tri not a bijection G=%d T=%d\n", G, T); return 1; }
    }
  }
  printf("ok\n");
  return 0;
}
"""


@pytest.fixture(scope="module")
def tile_map_binary(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    d = tmp_path_factory.mktemp("tilemap")
    src = d / "tile_map.hip"
    src.write_text(PROGRAM)
    exe = d / "tile_map"
    r = subprocess.run([hipcc, "-O1", "-std=c++17", "--offload-arch=gfx950", "-I", CSRC, str(src),
                        "-o", str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return str(exe)


def test_tile_maps_are_bijections(tile_map_binary):
    r = subprocess.run([tile_map_binary], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
