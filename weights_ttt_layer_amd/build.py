"""Build libttt.so (HIP, gfx950) in-tree with hipcc.

    python -m weights_ttt_layer_amd.build

Every translation unit under csrc/ is compiled with --offload-arch=gfx950 and
packed-fp32 instruction selection disabled, then linked into
weights_ttt_layer_amd/libttt.so next to this file.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(HERE, "libttt.so")
SOURCES = ["ttt_abi.hip", "smallb_linear.hip", "smallb_chain.hip", "midb_linear.hip", "smallb_mlp.hip", "mlp_generic.hip",
           "large_chunk.hip", "decode.hip", "outer_layer.hip", "backward.hip"]
# the measurement calibration kernels (include/ttt_peak.h), a library of their own
PEAK_LIB_PATH = os.path.join(HERE, "libttt_peak.so")
PEAK_SOURCES = ["peak.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libttt.so)")


COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # no packed-fp32 (v_pk_*_f32) instruction selection
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # keep MFMA accumulators in ordinary VGPRs: the kernels read their state
    # tiles as operands every chunk, which AGPRs would force through copies
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-result", "-Wno-unused-variable",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *COMMON_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, path: str) -> None:
    tmp = path + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, path)


def build(verbose: bool = False) -> str:
    """Compile every HIP source for gfx950 and link libttt.so (and the calibration
    library libttt_peak.so). Returns the path of libttt.so."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = SOURCES + PEAK_SOURCES
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    _link(objs[:len(SOURCES)], LIB_PATH)
    _link(objs[len(SOURCES):], PEAK_LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH} and {PEAK_LIB_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
