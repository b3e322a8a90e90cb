"""The block -> unit maps of the expert GEMM launches (xcd_remap and
xcd_remap_dealt in csrc/common.h), compiled for the host with hipcc and run
on the CPU: every unit is taken by exactly one block of the launch's grid,
and the dealt units come first in their XCD's order, at most ceil(n / 8) per
XCD."""
import os
import subprocess

import pytest

from tests import isa_check as ic

pytestmark = pytest.mark.skipif(not os.path.exists(ic.HIPCC), reason="hipcc not installed")

PROGRAM = r"""
#include "common.h"
#include <cstdio>
#include <vector>
// Prints one line per failed case; nothing when every case holds.
int main() {
  const int K = moe::kNumXcd;
  int bad = 0;
  for (int nvalid = 0; nvalid <= 700; ++nvalid) {
    const int lasts[] = {0, 1, 7, 8, 9, 10, 16, 17, nvalid / 2, nvalid};
    for (int nlast : lasts) {
      if (nlast > nvalid) continue;
      for (int extra = 0; extra <= 24; extra += 8) {  // grids built from a larger capacity
        const int cap = nvalid + extra;
        const int plain_grid = (cap + K - 1) / K * K;
        const int dealt_grid = ((cap + K - 1) / K + 1) * K;
        std::vector<int> seen(nvalid, 0), seen2(nvalid, 0);
        std::vector<int> dealt_per_xcd(K, 0);
        for (int b = 0; b < plain_grid; ++b) {
          const int u = moe::xcd_remap(b, nvalid);
          if (u >= nvalid || u < -1) { printf("plain %d %d: %d\n", nvalid, b, u); ++bad; }
          else if (u >= 0) ++seen[u];
        }
        for (int b = 0; b < dealt_grid; ++b) {
          const int u = moe::xcd_remap_dealt(b, nvalid, nlast);
          if (u >= nvalid || u < -1) { printf("dealt %d %d %d: %d\n", nvalid, nlast, b, u); ++bad; continue; }
          if (u < 0) continue;
          ++seen2[u];
          const int xcd = b % K, slot = b / K;
          if (u >= nvalid - nlast) {
            // a dealt unit: before every routed unit of its XCD
            if (slot != dealt_per_xcd[xcd]) { printf("order %d %d %d\n", nvalid, nlast, b); ++bad; }
            ++dealt_per_xcd[xcd];
          }
        }
        for (int u = 0; u < nvalid; ++u)
          if (seen[u] != 1 || seen2[u] != 1) {
            printf("count %d %d %d: %d %d\n", nvalid, nlast, u, seen[u], seen2[u]);
            ++bad;
          }
        for (int x = 0; x < K; ++x)
          if (dealt_per_xcd[x] > (nlast + K - 1) / K) { printf("per xcd %d %d\n", nvalid, nlast); ++bad; }
      }
    }
  }
  return bad ? 1 : 0;
}
"""


def test_block_unit_maps_are_bijections(tmp_path):
    src = tmp_path / "remap.hip"
    src.write_text(PROGRAM)
    exe = tmp_path / "remap"
    subprocess.run([ic.HIPCC, "--offload-arch=gfx950", "-O1", "-std=c++17", "-I", ic.CSRC,
                    str(src), "-o", str(exe)], check=True, capture_output=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout[:2000]
