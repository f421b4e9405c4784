"""Build libmla_absorb.so (HIP for gfx950) in-tree with hipcc.

    python -m mla_latent_kv_absorb_amd.build

Every source under csrc/ is compiled for gfx950 only, with packed-FP32 instruction
selection switched off, and linked into mla_latent_kv_absorb_amd/libmla_absorb.so.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
LIB_NAME = "libmla_absorb.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
BUILD_DIR = os.path.join(HERE, "_build")

SOURCES = ["mla_api.cpp", "timing.cpp", "plain_kernels.hip", "absorb_mfma.hip", "expand_mfma.hip", "cache_append.hip",
           "naive_mfma.hip", "noalloc.hip"]
# peak probes for the benchmark (streaming read and copy, matrix-core and LDS rates): a library of
# their own, never linked into the attention library
PEAKS_SOURCES = ["peaks.hip"]
PEAKS_LIB_PATH = os.path.join(HERE, "libmla_peaks.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-ffp-contract=fast",
    "-munsafe-fp-atomics",
    # packed FP32 instructions (v_pk_fma_f32 and friends) stay off
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd.insert(1, "-x")
        cmd.insert(2, "hip")
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, path: str) -> None:
    tmp = path + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, path)


def build(verbose: bool = True) -> str:
    """Compile every source and link the attention library and the probe library; returns the
    attention library's path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = [s for s in SOURCES + PEAKS_SOURCES if os.path.exists(os.path.join(CSRC, s))]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = dict(zip(srcs, ex.map(_compile, srcs)))
    _link([objs[s] for s in SOURCES if s in objs], LIB_PATH)
    _link([objs[s] for s in PEAKS_SOURCES if s in objs], PEAKS_LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH} and {PEAKS_LIB_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    build()
    sys.exit(0)
