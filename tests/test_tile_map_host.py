"""The library's position -> token map of the 3-D tile order (csrc/sa_layout.h,
used by the pool and attention kernels) against the oracle's tile_order, on
the host: the header is compiled with g++ into a small program that prints
the map (CPU only, no GPU, no library code beyond the header)."""
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle import attention as orc

HDR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "block_sparse_attention_route_amd", "csrc")

PROG = r"""
#define __host__
#define __device__
#include <cstdio>
#include <cstdlib>
#include "sa_layout.h"
int main(int argc, char** argv) {
  int T = atoi(argv[1]), Hg = atoi(argv[2]), Wg = atoi(argv[3]);
  int tt = atoi(argv[4]), th = atoi(argv[5]), tw = atoi(argv[6]);
  sa::TileMap m = sa::make_tile_map(T, Hg, Wg, tt, th, tw);
  for (int p = 0; p < T * Hg * Wg; ++p) printf("%d\n", sa::token_of(m, p));
  return 0;
}
"""


@pytest.fixture(scope="module")
def prog(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    d = tmp_path_factory.mktemp("tilemap")
    src, exe = d / "m.cpp", d / "m"
    src.write_text(PROG)
    subprocess.run(["g++", "-O1", "-std=c++17", f"-I{HDR}", str(src), "-o", str(exe)], check=True)
    return str(exe)


@pytest.mark.parametrize("grid", [(21, 45, 80), (3, 10, 13), (4, 16, 16), (5, 12, 19), (1, 1, 37), (2, 7, 9)])
@pytest.mark.parametrize("tile", [(4, 4, 4), (1, 8, 8), (2, 4, 8), (1, 1, 64), (16, 2, 2), (64, 1, 1)])
def test_token_map_matches_oracle(prog, grid, tile):
    out = subprocess.run([prog, *map(str, grid), *map(str, tile)], check=True, capture_output=True, text=True)
    got = np.array([int(x) for x in out.stdout.split()])
    np.testing.assert_array_equal(got, orc.tile_order(*grid, tile))


def test_raster_when_off(prog):
    out = subprocess.run([prog, "2", "3", "70", "0", "0", "0"], check=True, capture_output=True, text=True)
    assert [int(x) for x in out.stdout.split()] == list(range(420))
