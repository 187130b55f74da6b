"""The host code of the library under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only).

Every source is compiled with the sanitizers on its host half only (the
device code is unchanged and never runs here), linked into a separate copy
of the library, and driven by tests/abi_errors.c: every entry point's
validation errors, the workspace queries at the largest accepted sizes, and
the per-thread error message.  A sanitizer report fails the run (UBSan
without recovery; ASan aborts on the first error).
"""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
from post_weight_quantization_stats_amd import build as B  # noqa: E402

CLANG = "/opt/rocm/llvm/bin/clang"
# Sanitizers on the host half of each translation unit only.
HOST_SANITIZE = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined".split() + \
    "-Xarch_host -fno-sanitize-recover=undefined".split()


def _build_sanitized(out_dir: str) -> str:
    flags = [f for f in B.COMMON_FLAGS if f != "-O3"] + ["-O1", "-g", "-fno-omit-frame-pointer"]
    objs = []
    procs = []
    for src in B.SOURCES:
        obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
        cmd = [B.hipcc(), *flags, *B.SOURCE_FLAGS.get(src, []), *HOST_SANITIZE, "-x", "hip", "-c",
               os.path.join(B.CSRC, src), "-o", obj]
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE,
                                            text=True)))
        objs.append(obj)
    for cmd, p in procs:
        out, err = p.communicate()
        assert p.returncode == 0, f"{' '.join(cmd)}\n{out}\n{err}"
    lib = os.path.join(out_dir, "libawq_mi355x_hostsan.so")
    r = subprocess.run([B.hipcc(), f"--offload-arch={B.ARCH}", "-shared", "-fPIC", "-o", lib, *objs],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return lib


@pytest.mark.skipif(not (os.path.exists(CLANG) and shutil.which("hipcc") or os.path.exists("/opt/rocm/bin/hipcc")),
                    reason="needs hipcc and ROCm's clang")
def test_error_paths_under_address_and_ub_sanitizers(tmp_path):
    lib = _build_sanitized(str(tmp_path))
    exe = str(tmp_path / "abi_errors")
    r = subprocess.run([CLANG, "-std=c99", "-g", "-fsanitize=address,undefined",
                        "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include"),
                        os.path.join(ROOT, "tests", "abi_errors.c"), "-o", exe, lib,
                        "-Wl,-rpath," + str(tmp_path), "-lpthread"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", HIP_VISIBLE_DEVICES="")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    report = run.stdout + run.stderr
    assert run.returncode == 0 and run.stdout.strip().endswith("ok"), report
    assert "runtime error" not in report and "AddressSanitizer" not in report, report
