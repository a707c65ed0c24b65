"""The dK/dV kernel's work order (dkdv_work / dkdv_grid in csrc/common.h),
checked on the host: the device function is compiled for the CPU with hipcc
and enumerated over every block index of the grid.

* every (KV head, key tile) unit is run exactly once, for head counts that
  take each of the map's three branches and for odd and even tile counts;
* on the causal headline shape (2 KV heads, 512 key tiles of 128 keys) the
  partner of the first member at cohort slot u of an XCD is the second member
  at slot 2 * COHORT - 1 - u: it is the one that starts on the CU which the
  first member frees, and the two walk their query tiles in opposite
  directions.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sequence_context_parallelism_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC) and shutil.which("hipcc") is None,
                                reason="hipcc not available")

PROGRAM = r"""
#include "common.h"
#include <cstdio>
#include <vector>
using namespace cp;
int main() {
  int bad = 0;
  for (int ng : {1, 2, 3, 4, 5, 6, 8, 16, 24}) {
    for (int nkt : {1, 2, 3, 4, 5, 7, 8, 31, 32, 33, 63, 64, 65, 127, 128, 255, 256, 257, 511, 512, 513, 1000}) {
      const int grid = dkdv_grid(ng, nkt);
      if (grid % 8 != 0) { printf("grid %d not a multiple of 8 (ng=%d nkt=%d)\n", grid, ng, nkt); ++bad; }
      std::vector<int> seen((size_t)ng * nkt, 0);
      for (int b = 0; b < grid; ++b) {
        int g, kt, dir;
        if (!dkdv_work(b, ng, nkt, g, kt, dir)) continue;
        if (g < 0 || g >= ng || kt < 0 || kt >= nkt || (dir != 1 && dir != -1)) {
          printf("out of range: ng=%d nkt=%d b=%d -> %d %d %d\n", ng, nkt, b, g, kt, dir);
          ++bad;
          continue;
        }
        seen[(size_t)g * nkt + kt]++;
      }
      for (size_t u = 0; u < seen.size(); ++u)
        if (seen[u] != 1) {
          printf("ng=%d nkt=%d: unit (%zu, %zu) run %d times\n", ng, nkt, u / nkt, u % nkt, seen[u]);
          ++bad;
          break;
        }
    }
  }
  const int C = DKDV_COHORT;
  if (dkdv_grid(2, 512) != 1024) { printf("grid(2, 512) = %d\n", dkdv_grid(2, 512)); ++bad; }
  for (int xcd = 0; xcd < 8; ++xcd)
    for (int round = 0; round < 2; ++round)
      for (int u = 0; u < C; ++u) {
        int g1, k1, d1, g2, k2, d2;
        const int s1 = round * 2 * C + u, s2 = round * 2 * C + 2 * C - 1 - u;
        const bool ok1 = dkdv_work(s1 * 8 + xcd, 2, 512, g1, k1, d1);
        const bool ok2 = dkdv_work(s2 * 8 + xcd, 2, 512, g2, k2, d2);
        if (!ok1 || !ok2 || g1 != g2 || g1 != xcd % 2 || k2 != 511 - k1 || d1 != -1 || d2 != 1) {
          printf("xcd %d slot %d/%d: (%d %d %d) (%d %d %d)\n", xcd, s1, s2, g1, k1, d1, g2, k2, d2);
          ++bad;
        }
      }
  printf("bad=%d\n", bad);
  return bad != 0;
}
"""


def test_dkdv_work_order(tmp_path):
    src = tmp_path / "work_order.cpp"
    exe = tmp_path / "work_order"
    src.write_text(PROGRAM)
    cmd = [HIPCC, "-x", "hip", "--offload-arch=gfx950", "-O1", f"-I{CSRC}", f"-I{os.path.join(ROOT, 'include')}",
           str(src), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip().endswith("bad=0"), r.stdout
