"""Build libmosaic_bsa.so in-tree for gfx950 with hipcc.

    python -m spherical_block_sparse_amd.build          # always rebuilds

Each HIP source is compiled to an object in parallel, then linked into
spherical_block_sparse_amd/libmosaic_bsa.so (the BSA library, include/
mosaic_bsa.h) and spherical_block_sparse_amd/libmosaic_probe.so (the
measurement probes, include/mosaic_probe.h).  Packed fp32 VALU instructions
are disabled (-packed-fp32-ops).
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
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmosaic_bsa.so")
PROBE_LIB = os.path.join(PKG, "libmosaic_probe.so")
PROBE_SOURCES = ["peak_probe.hip"]

SOURCES = ["bsa_pool.hip", "bsa_compress_select.hip", "bsa_fine.hip", "bsa_backward.hip", "bsa_layer.hip",
           "healpix_coarsen.hip", "healpix_interp.hip", "bsa_scratch.hip", "mosaic_bsa_api.cpp"]
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libmosaic_bsa)")


# per-source extra flags: the fine-attention and selection kernels never rely on NaN
# semantics (masked scores are -inf, which stays honoured), and without this
# every fmaxf of an MFMA result is preceded by a NaN-quieting instruction.  The
# selection kernels keep their fp64 MFMA accumulators in VGPRs
# (-amdgpu-mfma-vgpr-form): in AGPRs each chunk pays 16 accumulator reads,
# and no vector work runs beside an fp64 MFMA to hide them.
EXTRA = {
    "bsa_fine.hip": ["-fno-honor-nans"],
    "bsa_backward.hip": ["-fno-honor-nans"],
    "bsa_compress_select.hip": ["-fno-honor-nans", "-mllvm", "-amdgpu-mfma-vgpr-form"],
    # the MFMA probe's loop is then its eight MFMAs alone (with AGPR
    # accumulators the compiler rotates them through VGPRs every iteration)
    "peak_probe.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *FLAGS, *EXTRA.get(src, []), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile of {src} failed:\n{' '.join(cmd)}\n{r.stdout}{r.stderr}")
    return obj


def _link(lib: str, objs: list) -> None:
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, SOURCES + PROBE_SOURCES))
    _link(LIB, objs[:len(SOURCES)])
    _link(PROBE_LIB, objs[len(SOURCES):])
    if verbose:
        print(f"built {LIB} and {PROBE_LIB}")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
