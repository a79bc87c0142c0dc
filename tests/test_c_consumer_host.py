"""The C ABI from a plain C program (CPU only): include/tbl.h compiles as C11 with every warning
enabled, a program linked against libtbl.so calls the host-only entry points, and what it prints
equals what the same calls return through the Python binding. No GPU call is made: every call
below either needs no device or fails validation before its first HIP call."""

import os
import shutil
import subprocess

import pytest

import thread_block_lds_amd as tbl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GCC = shutil.which("gcc")

PROGRAM = r"""
#include <stdio.h>
#include <stdint.h>
#include "tbl.h"

int main(void) {
  int bm = 0, bn = 0, bk = 0;
  int rc = tbl_gemm_tile_shape(4096, 4096, 4096, &bm, &bn, &bk);
  printf("tile %d %d %d %d\n", rc, bm, bn, bk);
  rc = tbl_gemm_tile_shape(2048, 2048, 2048, &bm, &bn, &bk);
  printf("tile %d %d %d %d\n", rc, bm, bn, bk);
  /* the page's 8192^3 128x128x32 run, row-major, one cache of the chip's L2, 512 resident tiles */
  int64_t hits = 0, accesses = 0;
  rc = tbl_predict_l2(TBL_ROW, 64, 64, 256, 1, 8192, 8192, (int64_t)32 << 20, 1, 0, 512, &hits, &accesses);
  printf("l2 %d %lld %lld\n", rc, (long long)hits, (long long)accesses);
  int64_t misses = 0;
  rc = tbl_predict_l2_lines(TBL_SERPENTINE | TBL_XCD_REMAP, 8192, 8192, 8192, 2, 256, 256, 32, 8, 8, 256, 32,
                            2048, 16, 128, 11, 4, 0, (uint64_t)1 << 27, &hits, &accesses, &misses);
  printf("lines %d %lld %lld %lld\n", rc, (long long)hits, (long long)accesses, (long long)misses);
  /* rejected before any HIP call */
  rc = tbl_gemm(NULL, NULL, NULL, 8, 8, 8, TBL_F16, TBL_ROW, 1, 0, 0, NULL);
  printf("reject %d %s\n", rc, tbl_status_string(rc));
  rc = tbl_transpose_i32((const int32_t*)16, (int32_t*)32, 100, 64, TBL_T_XOR, NULL);
  printf("reject %d\n", rc);
  printf("version %d\n", tbl_version());
  return 0;
}
"""


@pytest.mark.skipif(GCC is None, reason="gcc not installed")
def test_plain_c_program_links_and_calls_the_library(tmp_path):
    lib = tbl.lib()   # builds nothing; fails loudly if libtbl.so is missing
    libdir = os.path.dirname(tbl.LIB_PATH)
    src = tmp_path / "consumer.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "consumer"
    subprocess.run([GCC, "-std=c11", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
                    str(src), "-L", libdir, "-ltbl", f"-Wl,-rpath,{libdir}", "-o", str(exe)],
                   check=True, capture_output=True, text=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True, timeout=120).stdout.split("\n")
    assert out[0] == "tile 0 256 256 32" and out[1] == "tile 0 128 128 32"
    h, a = tbl.predict_l2(tbl.ROW, 64, 64, 256, 1, 8192, 8192, 32 << 20, 1, 0, 512)[:2]
    assert out[2] == f"l2 0 {h} {a}"
    lh, la, lm, st = tbl.predict_l2_lines(tbl.SERPENTINE | tbl.XCD_REMAP, 8192, 8192, 8192, 8, num_programs=256,
                                          resident=32, a_base=0, b_base=1 << 27)
    assert out[3] == f"lines {st} {lh} {la} {lm}"
    assert out[4] == f"reject {tbl.ERR_INVALID_ARG} {tbl.status_string(tbl.ERR_INVALID_ARG)}"
    assert out[5] == f"reject {tbl.ERR_SHAPE}"
    assert out[6] == f"version {tbl.version()}"
    assert lib is not None
