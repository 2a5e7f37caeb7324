"""Build the HIP library ``libmlp.so`` in-tree with hipcc for gfx950.

Usage: ``python -m mlp_neural_shading_amd.build`` (or ``__graft_entry__.build()``).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
CSRC = PKG / "csrc"
LIB = PKG / "libmlp.so"
BUILD_DIR = PKG.parent / "_build"

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = [
    "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    # no packed-FP32 instructions anywhere (hipcc's host pass warns that it does not know the feature)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # a single-lane LDS atomic claims the next tile and its result is read an iteration later; the
    # wave-aggregating rewrite of atomics would consume the result at once and stall the wave
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
]
SOURCES = ["mlp_kernels.hip", "mlp_kernels_fp8.hip", "mlp_layered.hip", "mlp_pack_device.hip", "mlp_api.cpp", "mlp_pack.cpp"]
CEILING_SOURCE = "mlp_ceiling.hip"
CEILING_LIB = PKG / "libmlp_ceiling.so"


INCLUDE = PKG.parent / "include"


def _compile(src: Path, obj: Path, extra) -> None:
    cmd = [HIPCC, "--offload-arch=" + ARCH, *COMMON, "-I", str(INCLUDE), *extra, "-x", "hip", "-c", str(src),
           "-o", str(obj)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src.name, " ".join(cmd), r.stderr[-8000:]))


def build(verbose: bool = False, extra=()) -> Path:
    BUILD_DIR.mkdir(exist_ok=True)
    objs = [BUILD_DIR / (Path(s).stem + ".o") for s in SOURCES]
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        list(ex.map(lambda so: _compile(CSRC / so[0], so[1], list(extra)), zip(SOURCES, objs)))
    tmp = LIB.with_name(LIB.name + ".tmp%d" % os.getpid())
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", *map(str, objs), "-o", str(tmp)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr[-8000:]))
    os.replace(tmp, LIB)
    # the benchmark's MFMA-ceiling probe, a separate small library
    cobj = BUILD_DIR / "mlp_ceiling.o"
    _compile(CSRC / CEILING_SOURCE, cobj, list(extra))
    tmp = CEILING_LIB.with_name(CEILING_LIB.name + ".tmp%d" % os.getpid())
    r = subprocess.run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", str(cobj), "-o", str(tmp)],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed for the ceiling probe:\n%s" % r.stderr[-8000:])
    os.replace(tmp, CEILING_LIB)
    if verbose:
        print("built", LIB, "and", CEILING_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
