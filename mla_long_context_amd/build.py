"""Build libmla.so (gfx950) in-tree with hipcc.

    python -m mla_long_context_amd.build

Every HIP source under csrc/ is compiled to an object in csrc/../_build and
linked into mla_long_context_amd/libmla.so. Always recompiles.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmla.so")
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (need ROCm)")


FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
    # packed fp32 ops disabled for every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


# Per-source extra flags. The attention kernel's softmax reads and rewrites
# the MFMA accumulators every tile; keeping MFMA results in VGPRs (instead of
# AGPRs) saves the accumulator copies around each softmax.
EXTRA = {
    "attn.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *FLAGS, *EXTRA.get(os.path.basename(src), []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines()
            if "packed-fp32-ops' is not a recognized feature" not in ln]
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n" + "\n".join(msgs))
    if msgs:
        sys.stderr.write("\n".join(msgs) + "\n")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources")
    build_calib(verbose)
    return LIB


CALIB_SRC = os.path.join(PKG, "calib", "mfma_peak.hip")
CALIB_LIB = os.path.join(PKG, "libmla_calib.so")


def build_calib(verbose: bool = False) -> str:
    """The benchmark's MFMA calibration library (not part of libmla.so)."""
    tmp = CALIB_LIB + ".tmp"
    cmd = [hipcc(), *FLAGS, "-shared", CALIB_SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for the calibration library:\n" + r.stdout + r.stderr)
    os.replace(tmp, CALIB_LIB)
    if verbose:
        print(f"built {CALIB_LIB}")
    return CALIB_LIB


if __name__ == "__main__":
    build(verbose=True)
