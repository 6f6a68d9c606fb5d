"""The library's schedule functions (csrc/schedule.hpp) compiled for the host
with the undefined-behaviour sanitizer: every tile id the kernels can form --
including the ids past num_tiles that the flattened loop's look-ahead cursors
reach -- maps without undefined behaviour, and the in-range ids agree with the
oracle's enumerated tables."""
import os
import shutil
import subprocess

import pytest

from oracle import schedule as osch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HDR = os.path.join(ROOT, "tile_scheduling_amd", "csrc")

DRIVER = r"""
#include <stdio.h>
#include <stdlib.h>
#include "schedule.hpp"
int main(int argc, char** argv) {
    ts::SchedArgs s;
    s.nm = atoi(argv[1]); s.nn = atoi(argv[2]); s.ks = 1; s.num_tiles = s.nm * s.nn;
    s.order = atoi(argv[3]); s.group_m = atoi(argv[4]); s.grid = atoi(argv[5]);
    s.remap = 0; s.xcds = 8;
    for (int t = 0; t < s.num_tiles + 2 * s.grid + 2; ++t) {
        int tm = -1, tn = -1;
        ts::tile_coords(s, t, tm, tn);
        printf("%d %d %d\n", t, tm, tn);
    }
    return 0;
}
"""


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    d = tmp_path_factory.mktemp("ubsan")
    src = d / "drv.cpp"
    src.write_text(DRIVER)
    exe = d / "drv"
    subprocess.run([gxx, "-std=c++17", "-O1", "-g", "-fsanitize=undefined", "-fno-sanitize-recover=all",
                    "-I", HDR, str(src), "-o", str(exe)], check=True)
    return str(exe)


# (nm, nn, G, P): G dividing nm (a band of zero rows past the end when G*k == nm),
# G leaving a short last band, G above nm, and the headline 64 x 64 grid at G = 8
CASES = [(64, 64, 8, 256), (20, 49, 8, 256), (5, 3, 2, 4), (8, 8, 8, 3), (3, 7, 16, 5), (1, 1, 1, 1)]


@pytest.mark.parametrize("nm,nn,G,P", CASES)
@pytest.mark.parametrize("order", [0, 1])
def test_tile_coords_defined_past_the_last_tile(driver, nm, nn, G, P, order):
    g = min(G, nm)   # the library clamps G to num_m_tiles before any launch
    r = subprocess.run([driver, str(nm), str(nn), str(order), str(g), str(P)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    assert "runtime error" not in r.stderr
    rows = [tuple(int(v) for v in line.split()) for line in r.stdout.split("\n") if line]
    T = nm * nn
    for t, tm, tn in rows:
        if t < T:
            ref = osch.grouped(t, nm, nn, g) if order == 1 else osch.row_major(t, nm, nn)
            assert (tm, tn) == ref, t
        else:
            assert (tm, tn) == (0, 0), t
