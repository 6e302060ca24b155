"""Build libbsattn.so in-tree with hipcc for gfx950.

    python -m block_sparse_transformer_amd.build        # or build() from Python

Every HIP source is compiled to an object in parallel, then linked into
``block_sparse_transformer_amd/libbsattn.so``.  Packed-fp32 instructions are
disabled for device code (the target feature ``-packed-fp32-ops``).

``build(debug=True)`` (``--debug`` on the command line) builds
``libbsattn_debug.so`` with ``-DBSATTN_DEBUG``: the forward kernels bounds-check
every schedule entry they read and the backward passes every item and block-list
entry; each of those launches synchronises its stream and fails (BSATTN_ERR_HIP,
"device-side assert") if a check did not hold.
Setting ``BSATTN_LIBRARY`` to its path makes the binding load it instead.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libbsattn.so")
BUILD_DEBUG = os.path.join(ROOT, "_build_debug")
LIB_DEBUG = os.path.join(PKG, "libbsattn_debug.so")

SOURCES = [
    "api.cpp",
    "kernels/fwd_bf16.hip",
    "kernels/bwd_bf16.hip",
    "kernels/layer.hip",
    "kernels/fwd_f32.hip",
    "kernels/router.hip",
    "kernels/layout_build.hip",
    "kernels/adaptive.hip",
    "kernels/noalloc.hip",
    "kernels/topr.hip",
    "kernels/bwd_token.hip",
    "kernels/candidates.hip",
]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-I", INCLUDE, "-I", CSRC,
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form",   # MFMA accumulators in VGPRs: no AGPR copies around the softmax
    "-Wno-unused-command-line-argument",
]


def _compile(src: str, verbose: bool, debug: bool = False) -> str:
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD_DEBUG if debug else BUILD, src.replace("/", "_") + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC, *FLAGS, *(["-DBSATTN_DEBUG"] if debug else []), *lang, "-c", path, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, debug: bool = False) -> str:
    out_dir, lib = (BUILD_DEBUG, LIB_DEBUG) if debug else (BUILD, LIB)
    os.makedirs(out_dir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, debug), SOURCES))
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp,
           "-L/opt/rocm/lib", "-lrocblas", "-lhipblaslt", "-Wl,-rpath,/opt/rocm/lib"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, debug="--debug" in sys.argv))
