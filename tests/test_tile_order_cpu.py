"""The count passes' work orders, checked on the CPU: the blocked tile
order (super-tiles of 16 x 16 tiles) must visit every tile I <= J of the
upper triangle exactly once, and the per-XCD split of the items must be a
permutation of them.  The device header is compiled for the host with
hipcc and its functions run on the CPU; no GPU is used."""
import os
import shutil
import subprocess
import tempfile

import pytest

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                    "all_pairs_distance_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

HARNESS = r"""
#include "count_common.h"
#include <cstdio>
#include <vector>
using namespace dbk;
int main() {
  const long long nbs[] = {1, 2, 3, 15, 16, 17, 31, 32, 33, 100, 196, 255, 256,
                           257, 489, 1024, 1031};
  for (long long nb : nbs) {
    const int64_t tiles = nb * (nb + 1) / 2;
    std::vector<char> seen((size_t)(nb * nb), 0);
    for (int64_t t = 0; t < tiles; ++t) {
      int64_t I = -1, J = -1;
      tile_coords_blocked(t, nb, I, J);
      if (I < 0 || J < I || J >= nb) { printf("range nb=%lld t=%lld\n", nb, (long long)t); return 1; }
      if (seen[(size_t)(I * nb + J)]++) { printf("twice nb=%lld t=%lld\n", nb, (long long)t); return 1; }
    }
  }
  const long long counts[] = {1, 7, 8, 9, 15, 16, 17, 1000, 4097, 119805, 524800};
  for (long long items : counts) {
    std::vector<char> seen((size_t)items, 0);
    for (int64_t s = 0; s < items; ++s) {
      const int64_t it = xcd_item(s, items);
      if (it < 0 || it >= items || seen[(size_t)it]++) { printf("xcd items=%lld s=%lld\n", items, (long long)s); return 1; }
      // work-groups on one XCD (s mod 8) take consecutive items
      if (s >= 8 && it != xcd_item(s - 8, items) + 1) { printf("order items=%lld s=%lld\n", items, (long long)s); return 1; }
    }
  }
  printf("ok\n");
  return 0;
}
"""


def test_blocked_tile_order_and_xcd_split_are_bijections():
    if not os.path.exists(HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("hipcc is not available")
    tmp = tempfile.mkdtemp(prefix="tile_order_")
    try:
        src = os.path.join(tmp, "check.hip")
        exe = os.path.join(tmp, "check")
        with open(src, "w") as f:
            f.write(HARNESS)
        p = subprocess.run([HIPCC, "--offload-arch=gfx950", "-O1", "-std=c++17",
                            f"-I{CSRC}", src, "-o", exe],
                           capture_output=True, text=True)
        assert p.returncode == 0, p.stderr[-3000:]
        r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
        assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
