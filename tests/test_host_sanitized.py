"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Every source is compiled with hipcc, the sanitizers applied to the host side only
(device code is untouched), and linked into a small driver that goes through the
host paths a machine without a GPU reaches: every argument check, empty calls, the
planner and workspace sizes over a sweep of shapes, the profiler and the release of
workspaces.  Any sanitizer report fails the run.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
from recurrent_vision_backbone_chunkwise_amd import build as lib_build  # noqa: E402

DRIVER = r'''
#include <stdio.h>
#include <string.h>
#include "gtr_gla.h"
#include "gtr_swiglu.h"

static int failures = 0;
static void expect(int got, int want, const char *what) {
  if (got != want) { fprintf(stderr, "%s: got %d, want %d (%s)\n", what, got, want, gtr_gla_last_error()); ++failures; }
}

int main(void) {
  static char buf[1 << 16];
  void *p = (void *)(((unsigned long)buf + 255) & ~255ul);
  char *c = (char *)p;
  /* argument checks, before any HIP call */
  expect(gtr_gla_fwd(p, p, p, p, c + 4096, -1, 1, 4, 4, 64, 64, 0, 1, 0), GTR_ERR_INVALID_ARG, "negative B");
  expect(gtr_gla_fwd(p, p, p, p, c + 4096, 1, 1, 4, 4, 0, 64, 0, 1, 0), GTR_ERR_INVALID_ARG, "d_k 0");
  expect(gtr_gla_fwd(p, p, p, p, c + 4096, 1, 1, 4, 4, 64, 64, 4, 1, 0), GTR_ERR_INVALID_ARG, "direction");
  expect(gtr_gla_fwd(p, p, p, p, c + 4096, 1, 1, 4, 4, 64, 64, 0, 3, 0), GTR_ERR_INVALID_ARG, "dtype");
  expect(gtr_gla_fwd(p, p, p, p, c + 4096, 1, 1, 4, 4, 132, 64, 0, 1, 0), GTR_ERR_UNSUPPORTED, "d_k 132");
  expect(gtr_gla_fwd(p, p, p, p, c + 4096, 1, 1, 4, 4, 6, 64, 0, 1, 0), GTR_ERR_UNSUPPORTED, "d_k 6");
  expect(gtr_gla_fwd(c + 1, p, p, p, c + 8192, 1, 1, 4, 4, 64, 64, 0, 1, 0), GTR_ERR_ALIGNMENT, "alignment");
  expect(gtr_gla_fwd(p, p, p, p, p, 1, 1, 4, 4, 64, 64, 0, 1, 0), GTR_ERR_ALIAS, "alias");
  expect(gtr_gla_fwd(NULL, p, p, p, c + 4096, 1, 1, 4, 4, 64, 64, 0, 1, 0), GTR_ERR_INVALID_ARG, "null q");
  expect(gtr_gla_fwd(p, p, p, p, c + 4096, 1, 1, 1 << 12, 1 << 12, 64, 64, 0, 1, 0), GTR_ERR_INVALID_ARG, "2^24 tokens");
  expect(gtr_gla_fwd(p, p, p, p, c + 4096, 1 << 11, 1 << 10, 4, 4, 64, 64, 0, 1, 0), GTR_ERR_INVALID_ARG, "2^21 sequences");
  expect(gtr_gla_fwd_ex(p, p, p, p, c + 4096, 1, 1, 4, 4, 132, 64, 0, 1, NULL, NULL, 0, GTR_PATH_FUSED, 0),
         GTR_ERR_UNSUPPORTED, "fused d_k 132");
  expect(gtr_gla_fwd_ex(p, p, p, p, c + 4096, 1, 1, 2048, 2048, 128, 64, 0, 1, NULL, NULL, 1, GTR_PATH_FUSED, 0),
         GTR_ERR_INVALID_ARG, "fused segments of two key blocks");
  expect(gtr_gla_fwd_ex(p, p, p, p, c + 4096, 1, 1, 4, 4, 64, 64, 0, 1, NULL, NULL, 0, 7, 0), GTR_ERR_INVALID_ARG, "path");
  expect(gtr_gla_fwd_ex(p, p, p, p, c + 4096, 1, 1, 2048, 4096, 64, 64, 0, 1, NULL, NULL, 1, GTR_PATH_FUSED, 0),
         GTR_ERR_INVALID_ARG, "fused segments");
  /* empty calls: nothing to do, no device needed */
  expect(gtr_gla_fwd(NULL, NULL, NULL, NULL, NULL, 0, 4, 4, 4, 64, 64, 0, 1, 0), GTR_OK, "B = 0");
  expect(gtr_gla_fwd(NULL, NULL, NULL, NULL, NULL, 1, 4, 0, 4, 64, 64, 0, 1, 0), GTR_OK, "no tokens");
  /* a valid call on a machine without a GPU */
  expect(gtr_gla_fwd(p, c + 1024, c + 2048, c + 3072, c + 8192, 1, 1, 2, 2, 64, 64, 0, 1, 0), GTR_ERR_NO_DEVICE, "no device");
  expect(gtr_gla_check(p, c + 1024, c + 2048, c + 3072, c + 8192, 1, 1, 2, 2, 64, 64, 0, 1, NULL, NULL, 0, 0),
         GTR_ERR_NO_DEVICE, "check without device");
  /* backward and Spatial SwiGLU argument checks */
  expect(gtr_gla_bwd(p, p, p, p, p, NULL, NULL, c + 4096, c + 8192, c + 12288, c + 16384, NULL, 1, 1, 4, 4, 64,
                     132, 0, 1, 0), GTR_ERR_UNSUPPORTED, "bwd d_v 132");
  expect(gtr_gla_bwd(p, p, p, p, p, NULL, NULL, c + 4096, c + 8192, c + 12288, c + 16384, NULL, 1, 1, 4, 4, 132,
                     64, 0, 1, 0), GTR_ERR_UNSUPPORTED, "bwd d_k 132");
  expect(gtr_gla_bwd(p, p, p, p, p, NULL, NULL, p, c + 8192, c + 12288, c + 16384, NULL, 1, 1, 4, 4, 64, 64, 0, 1, 0),
         GTR_ERR_ALIAS, "bwd alias");
  expect(gtr_gla_bwd(p, p, p, p, p, NULL, NULL, c + 4096, c + 8192, c + 12288, c + 16384, NULL, 1 << 10, 1 << 10, 2048,
                     4096, 64, 64, 0, 1, 0), GTR_ERR_INVALID_ARG, "bwd too many chunks");
  expect(gtr_swiglu_fwd(p, p, p, NULL, p, c + 4096, 1, 4, 4, 12, 64, 1, 0), GTR_ERR_UNSUPPORTED, "swiglu C 12");
  expect(gtr_swiglu_fwd(NULL, NULL, NULL, NULL, NULL, NULL, 0, 4, 4, 64, 64, 1, 0), GTR_OK, "swiglu empty");
  /* planner and sizes over a sweep of shapes */
  const int dims[] = {4, 32, 60, 64, 96, 128};
  for (int bh = 1; bh <= 4096; bh *= 4)
    for (int side = 1; side <= 512; side = side * 3 + 1)
      for (int di = 0; di < 6; ++di)
        for (int path = 0; path < 3; ++path) {
          int seg = 0, n_seg = 0, fused = 0;
          const int rc = gtr_gla_plan(1, bh, side, side + 3, dims[di], dims[5 - di], 0, path, &seg, &n_seg, &fused);
          if (rc != GTR_OK && rc != GTR_ERR_UNSUPPORTED && rc != GTR_ERR_INVALID_ARG) expect(rc, GTR_OK, "plan");
          if (rc == GTR_OK && (seg < 1 || n_seg < 1)) expect(seg, 1, "plan seg");
          (void)gtr_gla_workspace_bytes_ex(1, bh, side, side + 3, dims[di], dims[5 - di], di % 3, 0, path);
          (void)gtr_gla_workspace_bytes(1, bh, side, side + 3, dims[di], dims[5 - di], di % 3);
          (void)gtr_swiglu_workspace_bytes(bh, side, side, 8 * (di + 1), 64, di % 3);
        }
  /* profiler and workspaces with nothing recorded */
  gtr_gla_profile_begin();
  double ms[16];
  int n[16];
  const int kinds = gtr_gla_profile_end(ms, n, 16);
  for (int i = 0; i < kinds; ++i)
    if (!gtr_gla_kernel_name(i) || n[i] != 0) expect(n[i], 0, "profile");
  gtr_gla_release_workspaces();
  if (strlen(gtr_gla_last_error()) > 4096) ++failures;
  return failures ? 1 : 0;
}
'''


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="needs hipcc")
def test_host_code_under_sanitizers(tmp_path):
    hipcc = lib_build._hipcc()
    flags = [f"--offload-arch={lib_build.ARCH}", "-O1", "-g", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all", "-I", lib_build.INCLUDE, "-I", lib_build.CSRC]

    def compile_one(src):
        obj = str(tmp_path / (os.path.splitext(src)[0] + ".o"))
        r = subprocess.run([hipcc, *flags, "-c", os.path.join(lib_build.CSRC, src), "-o", obj],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        return obj

    with ThreadPoolExecutor(max_workers=min(len(lib_build.SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, lib_build.SOURCES))
    driver = tmp_path / "driver.cpp"
    driver.write_text(DRIVER)
    drv_obj = str(tmp_path / "driver.o")
    r = subprocess.run([hipcc, *flags, "-c", str(driver), "-o", drv_obj], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    exe = tmp_path / "driver"
    link = [f"--offload-arch={lib_build.ARCH}", "-Xarch_host", "-fsanitize=address", "-Xarch_host",
            "-fsanitize=undefined"]
    r = subprocess.run([hipcc, *link, drv_obj, *objs, "-lrocblas", "-o", str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1",
               HIP_VISIBLE_DEVICES=os.environ.get("HIP_VISIBLE_DEVICES", ""))
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
