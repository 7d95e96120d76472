"""The C ABI from a C program (CPU only): include/fp4mi.h compiles as C99
with every warning an error, every entry point links against libfp4mi.so
through a function pointer of its declared type, and calls that host-side
validation rejects return the documented status codes (no GPU is touched:
validation runs before any HIP call)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "block_scaled_fp4_amd", "libfp4mi.so")

PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "fp4mi.h"

#define CHECK(expr, want)                                                       \
  do {                                                                          \
    int got_ = (expr);                                                          \
    if (got_ != (want)) {                                                       \
      fprintf(stderr, "%s: got %d (%s), want %d\n", #expr, got_,               \
              fp4_status_string(got_), (want));                                 \
      return 1;                                                                 \
    }                                                                           \
  } while (0)

int main(void) {
  /* every entry point, through a pointer of the declared type */
  int (*q)(const void*, int, int64_t, int64_t, int, int, uint64_t, uint64_t, int, float*,
           uint8_t*, uint8_t*, void*) = fp4_quantize;
  int (*dq)(const uint8_t*, const uint8_t*, const float*, int64_t, int64_t, int, void*, int,
            void*) = fp4_dequantize;
  int (*fe)(const void*, int, int64_t, int64_t, int32_t, uint8_t*, float*, float*, void*) =
      fp4quant_encode;
  int (*fex)(const void*, int, int64_t, int64_t, int32_t, int, uint64_t, uint64_t, uint8_t*,
             float*, float*, void*) = fp4quant_encode_ex;
  int (*fd)(const uint8_t*, const float*, const float*, int64_t, int64_t, int32_t, void*, int,
            void*) = fp4quant_decode;
  int (*ef)(const void*, int, int64_t, int64_t, float*, void*, int, int, uint64_t, uint64_t, int,
            float*, uint8_t*, uint8_t*, void*) = fp4_errfeedback_qdq;
  int (*col)(const uint8_t*, const uint8_t*, const int64_t*, int32_t, int64_t, int64_t, uint8_t*,
             float*, void*) = mxfp4_row_to_fp8_col;
  int (*tok)(const uint8_t*, const uint8_t*, const int64_t*, int32_t, int64_t, int64_t, uint8_t*,
             float*, void*) = mxfp4_row_to_fp8_col_tokblk;
  int (*row)(const uint8_t*, const uint8_t*, int64_t, int64_t, uint8_t*, float*, void*) =
      mxfp4_row_to_fp8_row;
  const char* (*ss)(int) = fp4_status_string;
  int (*ver)(void) = fp4_abi_version;
  float ts = 1.0f;
  int64_t off[2] = {0, 0};

  CHECK(ver(), FP4MI_ABI_VERSION);
  if (strcmp(ss(FP4_OK), "ok") != 0) return 1;
  /* rejected on the host before any launch */
  CHECK(q(NULL, FP4_DTYPE_BF16, -1, 64, FP4_FMT_MXFP4, FP4_ROUND_RTN, 0, 0, FP4_TSCALE_GIVEN,
          &ts, NULL, NULL, NULL), FP4_ESHAPE);
  CHECK(q(NULL, 9, 4, 64, FP4_FMT_MXFP4, FP4_ROUND_RTN, 0, 0, FP4_TSCALE_GIVEN, &ts, NULL, NULL,
          NULL), FP4_EDTYPE);
  CHECK(q(NULL, FP4_DTYPE_BF16, 0, 64, FP4_FMT_MXFP4, FP4_ROUND_RTN, 0, 0, FP4_TSCALE_GIVEN,
          &ts, NULL, NULL, NULL), FP4_OK);                       /* empty: a no-op */
  CHECK(dq(NULL, NULL, NULL, 4, 48, FP4_FMT_MXFP4, NULL, FP4_DTYPE_BF16, NULL), FP4_ESHAPE);
  CHECK(fe(NULL, FP4_DTYPE_BF16, 4, 96, 64, NULL, NULL, NULL, NULL), FP4_ESHAPE);
  CHECK(fex(NULL, FP4_DTYPE_BF16, 4, 64, 64, 7, 0, 0, NULL, NULL, NULL, NULL), FP4_EINVAL);
  CHECK(fd(NULL, NULL, NULL, 4, 64, 48, NULL, FP4_DTYPE_BF16, NULL), FP4_EINVAL);
  CHECK(ef(NULL, FP4_DTYPE_F32, 4, 24, NULL, NULL, FP4_DTYPE_BF16, FP4_ROUND_SR, 0, 0,
           FP4_TSCALE_GIVEN, &ts, NULL, NULL, NULL), FP4_ESHAPE);
  CHECK(col(NULL, NULL, off, 0, 0, 128, NULL, NULL, NULL), FP4_EINVAL);
  CHECK(tok(NULL, NULL, off, 1, 0, 200, NULL, NULL, NULL), FP4_ESHAPE);
  CHECK(row(NULL, NULL, -1, 128, NULL, NULL, NULL), FP4_ESHAPE);
  puts("c abi ok");
  return 0;
}
"""


def test_header_compiles_as_c_and_links(tmp_path):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    if not os.path.exists(LIB):
        pytest.skip("libfp4mi.so is not built")
    src = str(tmp_path / "abi_c.c")
    exe = str(tmp_path / "abi_c")
    with open(src, "w") as f:
        f.write(PROGRAM)
    libdir = os.path.dirname(LIB)
    b = subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
                        "-I", os.path.join(ROOT, "include"), src, "-o", exe,
                        "-L", libdir, "-l:libfp4mi.so", "-Wl,-rpath," + libdir,
                        "-Wl,--allow-shlib-undefined"], capture_output=True, text=True)
    assert b.returncode == 0, b.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "c abi ok" in r.stdout
