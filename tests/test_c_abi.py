"""The header is plain C: a C99 program that includes it compiles with
warnings as errors, links against the library and gets the documented status
codes from host-side validation (no GPU is touched)."""

import os
import shutil
import subprocess

import pytest

import post_weight_quantization_stats_amd as awq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

C_PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "awq_mi355x.h"

#define CHECK(expr, want) do { int got_ = (int)(expr); \
  if (got_ != (want)) { printf("FAIL %s: %d != %d\n", #expr, got_, (int)(want)); return 1; } } while (0)

int main(void) {
  void* fake = (void*)0x10000;
  size_t bytes = 0;
  CHECK(awq_abi_version(), AWQ_ABI_VERSION);
  CHECK(strcmp(awq_status_string(AWQ_ERR_SHAPE), "AWQ_ERR_SHAPE"), 0);
  CHECK(awq_workspace_size(AWQ_OP_ACT_STATS, 65536, 0, 4096, 4, 128, 20, &bytes), AWQ_OK);
  if (bytes == 0) { printf("FAIL zero workspace\n"); return 1; }
  CHECK(awq_workspace_size(AWQ_OP_ACT_STATS, 65536, 0, 4096, 4, 128, 20, NULL), AWQ_ERR_NULL);
  CHECK(awq_act_stats(NULL, 4, 128, fake, fake, bytes, NULL), AWQ_ERR_NULL);
  CHECK(awq_act_stats(fake, 4, 100, fake, fake, bytes, NULL), AWQ_ERR_SHAPE);
  if (strlen(awq_last_error()) == 0) { printf("FAIL empty message\n"); return 1; }
  CHECK(awq_quantize_pack(fake, 4, 128, NULL, 5, 128, fake, fake, fake, NULL), AWQ_ERR_UNSUPPORTED);
  CHECK(awq_quantize_pack16(fake, 4, 128, NULL, 4, 128, AWQ_LAYOUT_INT3_DENSE, fake, fake, fake, NULL),
        AWQ_ERR_UNSUPPORTED);
  CHECK(awq_search_scale(fake, 0, 128, fake, 8, 4, 128, 20, NULL, NULL, NULL, NULL, NULL, NULL, NULL,
                         NULL, 0, NULL) != AWQ_OK, 1);
  printf("ok\n");
  return 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_header_is_c99_and_links(tmp_path):
    src = tmp_path / "abi.c"
    src.write_text(C_PROGRAM)
    exe = tmp_path / "abi"
    lib = awq.library_path()
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
                        "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe),
                        lib, "-Wl,-rpath," + os.path.dirname(lib)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0 and run.stdout.strip() == "ok", run.stdout + run.stderr
