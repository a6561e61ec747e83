"""Build ``libqsa.so`` (HIP kernels for gfx950 + the C ABI) in-tree with hipcc.

    python -m route_sparse_gqa_amd.build

Objects go to ``_build/`` at the repository root; the shared library is
written next to this file so that it travels with the source tree.
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build", "libqsa")
LIB_PATH = os.path.join(PKG, "libqsa.so")
ARCH = "gfx950"

SOURCES = [
    "route_normalize.hip",
    "membership_tiles.hip",
    "gather_attention.hip",
    "attention_backward.hip",
    "dkdv.hip",
    "key_segments.hip",
    "tile_lists.hip",
    "route_select.hip",
    "qsa_api.cpp",
    "noalloc.hip",
]

COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fvisibility=hidden",
    "-Wall",
    # packed fp32 VALU forms are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}",
]

# MFMA accumulators in ordinary VGPRs: the online-softmax rescale then needs no
# AGPR round trips and the attention kernel fits two waves per SIMD.  dkdv.hip
# keeps them in AGPRs: its dK/dV sums only accumulate, and the freed VGPRs let
# the compiler read the staged operands ahead of the matrix instructions.
VGPR_FORM_FLAGS = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
AGPR_FORM_SOURCES = {"dkdv.hip"}


def flags_for(src: str) -> list:
    return COMMON_FLAGS + ([] if os.path.basename(src) in AGPR_FORM_SOURCES else VGPR_FORM_FLAGS)


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP toolchain is required to build libqsa")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc(), *flags_for(src), "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def _link(objs, path: str) -> None:
    tmp = path + f".tmp{os.getpid()}"
    # -z defs: an entry point whose kernel file is missing fails here, not at load time
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,-z,defs", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, path)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(6, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    _link(objs, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
