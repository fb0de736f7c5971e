"""Build libso2attn.so (HIP for gfx950) in-tree with hipcc.

    python -m so_equivariant_graph_amd.build        # or build() from Python

Every source is compiled for gfx950 only, with packed-fp32 instruction
selection switched off (-Xclang -target-feature -Xclang -packed-fp32-ops),
then linked into one shared library next to this file."""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libso2attn.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)

SOURCES = [
    "abi.hip",
    "neighbors.hip",
    "attention_prep.hip",
    "norm.hip",
    "swiglu.hip",
    "attention_valu.hip",
    "attention_mfma.hip",
    "attention_batch.hip",
    "noalloc.hip",
]

HIPCC_FLAGS = [
    "-O3",
    "-std=c++17",
    "--offload-arch=gfx950",
    "-fPIC",
    "-Xclang",
    "-target-feature",
    "-Xclang",
    "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def _compile(src, hipcc, verbose):
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc, *HIPCC_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every HIP source for gfx950 and link LIB_PATH; returns it."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    hipcc = _hipcc()
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), 6)) as ex:
        objs = list(ex.map(lambda s: _compile(s, hipcc, verbose), SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
