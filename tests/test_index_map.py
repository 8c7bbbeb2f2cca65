"""The kernels' scan-direction index map, compiled for the host, against the oracle's.

csrc/gla_index.h holds the map the kernels apply to every load and store
address (scan position -> grid cell, in four directions).  Its functions are
compiled for the host here and compared, in native code, with the oracle's own
map (gla_oracle_scan_index, linked from the oracle's built library) at every
scan position of large and ragged grids, up to the 2^23-token maximum, in all
four directions: single positions (token_cell), the four-position groups and
lagged-gate cells the kernels load with (cells4), and the float-reciprocal
column split (col_major_pos) against exact integer division for every position
below 2^23 at heights whose reciprocals are inexact.  No GPU is needed.
"""
import os
import subprocess

import pytest

import oracle
from recurrent_vision_backbone_chunkwise_amd import build as lib_build

DRIVER = r"""
#include <cstdio>
#include <cstdlib>
#include "gla_index.h"

extern "C" long gla_oracle_scan_index(long t, long grid_h, long grid_w, int direction);

struct Map { int n_tok, gh, gw, dir; float rcp_gh; };

static int fail(const char *what, int gh, int gw, int dir, long t, long got, long want) {
  printf("%s: grid %dx%d direction %d position %ld: %ld, oracle %ld\n", what, gh, gw, dir, t, got, want);
  return 1;
}

int main(int argc, char **argv) {
  long checked = 0;
  // the column split alone, against exact division, for every position below 2^23
  const int heights[] = {3, 5, 7, 1000, 2047, 2049, 4093, 8191, 65521, 1 << 22};
  for (int gh : heights) {
    const float rcp = 1.0f / (float)gh;
    for (int p = 0; p < (1 << 23); ++p) {
      int row, col;
      gtr::col_major_pos(p, gh, rcp, row, col);
      if (col != p / gh || row != p % gh) return fail("col_major_pos", gh, 0, 2, p, col, p / gh);
    }
    checked += 1 << 23;
  }
  for (int a = 1; a + 1 < argc; a += 2) {
    const int gh = atoi(argv[a]), gw = atoi(argv[a + 1]);
    for (int dir = 0; dir < 4; ++dir) {
      const Map m{gh * gw, gh, gw, dir, 1.0f / (float)gh};
      for (int t = 0; t < m.n_tok; ++t) {
        const long want = gla_oracle_scan_index(t, gh, gw, dir);
        const long got = (long)gtr::token_cell(m, t);
        if (got != want) return fail("token_cell", gh, gw, dir, t, got, want);
      }
      // groups of four as the kernels take them (t0 = 64 chunk + 16 wave + 4 row group), through
      // the ragged last chunk, with the cell of the position before (lagged gates)
      const int end = (m.n_tok + 63) / 64 * 64;
      for (int t0 = 0; t0 < end; t0 += 4) {
        uint32_t cell[4], before;
        gtr::cells4<true>(m, t0, cell, before);
        for (int r = 0; r < 4; ++r) {
          const long want = t0 + r < m.n_tok ? gla_oracle_scan_index(t0 + r, gh, gw, dir) : (long)gtr::kNoRow;
          if ((long)cell[r] != want) return fail("cells4", gh, gw, dir, t0 + r, cell[r], want);
        }
        const long wb = t0 > 0 && t0 <= m.n_tok ? gla_oracle_scan_index(t0 - 1, gh, gw, dir) : (long)gtr::kNoRow;
        if ((long)before != wb) return fail("cells4 before", gh, gw, dir, t0, before, wb);
      }
      checked += 2L * m.n_tok;
    }
  }
  printf("ok %ld\n", checked);
  return 0;
}
"""

GRIDS = [(2048, 4096), (4096, 2048), (1, 1 << 23), (1 << 23, 1), (4093, 2049), (2047, 4097),
         (3, 2796202), (1000, 8388), (40, 40), (64, 64), (128, 128), (7, 9), (1, 1), (1, 65), (65, 1)]


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    oracle_lib = oracle.build()
    d = tmp_path_factory.mktemp("index_map")
    src = d / "driver.cpp"
    src.write_text(DRIVER)
    exe = d / "driver"
    hipcc = lib_build._hipcc()
    lib_dir = os.path.dirname(oracle_lib)
    cmd = [hipcc, "-O2", "-std=c++17", f"--offload-arch={lib_build.ARCH}", "-I", lib_build.CSRC, str(src),
           "-L", lib_dir, f"-l:{os.path.basename(oracle_lib)}", f"-Wl,-rpath,{lib_dir}", "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return exe


def test_device_index_map_equals_the_oracle(driver):
    args = [str(x) for g in GRIDS for x in g]
    r = subprocess.run([str(driver), *args], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    assert r.stdout.startswith("ok ")
