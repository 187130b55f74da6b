"""Build libawq_mi355x.so for gfx950 with hipcc (in-tree, no JIT cache).

    python -m post_weight_quantization_stats_amd.build
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT_DIR = os.path.join(PKG, "lib")
LIB_NAME = "libawq_mi355x.so"
LIB_PATH = os.path.join(OUT_DIR, LIB_NAME)

SOURCES = ["act_stats.hip", "candidate_scales.hip", "quantize_pack.hip", "w4a16_gemm.hip",
           "decode_gemm.hip", "dequant_packed.hip", "gram.hip", "block_ops.hip", "loss_argmin.hip", "noalloc.hip", "ceilings.hip",
           "api.cpp"]

ARCH = "gfx950"

# -ffp-contract=off: every fp32 step of the quantizer / dequantizer contract is
# a separately rounded operation (no fused multiply-add).
# -packed-fp32-ops off: the compiler must not form v_pk_{add,mul,fma}_f32.
COMMON_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off", "-Wall", "-Wno-unused-function",
    f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


# Per-source additions.  decode_gemm.hip: the matrix-core accumulators live in
# ordinary VGPRs (the fold after every group reads them; in AGPRs each read is
# an extra v_accvgpr_read per element).
SOURCE_FLAGS = {
    "decode_gemm.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def _compile(src: str, obj: str) -> None:
    cmd = [hipcc(), *COMMON_FLAGS, *SOURCE_FLAGS.get(src, []), "-x", "hip", "-c",
           os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")


def build(verbose: bool = False) -> str:
    """Compile every source and link the shared library; returns its path."""
    build_dir = os.path.join(PKG, "_build")
    os.makedirs(build_dir, exist_ok=True)
    os.makedirs(OUT_DIR, exist_ok=True)
    objs = [os.path.join(build_dir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        list(ex.map(_compile, SOURCES, objs))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
