"""The workgroup placement of the kernels, checked on the host (CPU only).

`xcd_remap` and `causal_lpt` (fa_internal.h) turn a workgroup id into the
(head, query block) tile that workgroup computes.  A small host program
built by hipcc from the library's own header runs both over every grid of
1 to 64 heads and 1 to 80 query blocks per head and checks that

  * each is a bijection of the workgroup ids onto the tile ids (every query
    block of every head is computed exactly once);
  * the workgroups that the dispatcher deals to one XCD (id % 8) get the
    same contiguous range of head-major tile ids from both, so that an XCD's
    L2 serves the same heads under either order;
  * under causal_lpt the ranks (0 = a head's longest rows) never decrease in
    dispatch order within an XCD: the longest-first list schedule of causal
    launches.

A mistake here would skip or repeat query blocks on the GPU; the parity
tests would see it only on the grids they happen to launch.
"""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from tiled_attention_fa_amd import build as hipbuild  # noqa: E402

PROGRAM = r"""
#include <cstdio>
#include <vector>
#include "fa_internal.h"

int main() {
  long checked = 0;
  for (int bh = 1; bh <= 64; ++bh) {
    for (int nq = 1; nq <= 80; ++nq) {
      const int total = bh * nq;
      std::vector<int> seen_remap(total, 0), seen_lpt(total, 0);
      std::vector<int> lo(fa::kXcds, total), hi(fa::kXcds, -1), lo2(fa::kXcds, total), hi2(fa::kXcds, -1);
      std::vector<int> last_rank(fa::kXcds, -1);
      for (int wg = 0; wg < total; ++wg) {
        const int x = wg % fa::kXcds;
        const int a = fa::xcd_remap(wg, total);
        const int b = fa::causal_lpt(wg, total, nq);
        if (a < 0 || a >= total || b < 0 || b >= total) {
          std::printf("out of range: bh %d nq %d wg %d -> %d %d\n", bh, nq, wg, a, b);
          return 1;
        }
        ++seen_remap[a];
        ++seen_lpt[b];
        lo[x] = a < lo[x] ? a : lo[x];
        hi[x] = a > hi[x] ? a : hi[x];
        lo2[x] = b < lo2[x] ? b : lo2[x];
        hi2[x] = b > hi2[x] ? b : hi2[x];
        const int rank = b % nq;
        if (rank < last_rank[x]) {
          std::printf("rank order: bh %d nq %d wg %d rank %d after %d\n", bh, nq, wg, rank, last_rank[x]);
          return 1;
        }
        last_rank[x] = rank;
        ++checked;
      }
      for (int t = 0; t < total; ++t)
        if (seen_remap[t] != 1 || seen_lpt[t] != 1) {
          std::printf("not a bijection: bh %d nq %d tile %d (%d, %d)\n", bh, nq, t, seen_remap[t], seen_lpt[t]);
          return 1;
        }
      for (int x = 0; x < fa::kXcds; ++x) {
        const int cnt = total / fa::kXcds + (x < total % fa::kXcds ? 1 : 0);
        if (cnt == 0) continue;
        if (lo[x] != lo2[x] || hi[x] != hi2[x] || hi[x] - lo[x] + 1 != cnt) {
          std::printf("XCD range: bh %d nq %d xcd %d [%d, %d] vs [%d, %d]\n", bh, nq, x, lo[x], hi[x], lo2[x], hi2[x]);
          return 1;
        }
      }
    }
  }
  std::printf("checked %ld workgroups\n", checked);
  return 0;
}
"""


def test_grid_order_bijective_and_longest_first(tmp_path):
    src = tmp_path / "grid_order.hip"
    src.write_text(PROGRAM)
    exe = tmp_path / "grid_order"
    cmd = [hipbuild.hipcc(), f"--offload-arch={hipbuild.ARCH}", "-O1", "-std=c++17",
           f"-I{hipbuild.CSRC}", f"-I{hipbuild.INCLUDE}", str(src), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    print(r.stdout.strip())
