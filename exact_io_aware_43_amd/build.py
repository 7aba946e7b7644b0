"""Build libfa.so in-tree with hipcc for gfx950.

Each ``csrc/*.hip`` file compiles to an object under ``_build/`` (in parallel),
then all objects link into ``exact_io_aware_43_amd/libfa.so``. Packed-fp32 VALU
instructions are disabled for device code.
"""

from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfa.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-Wno-unused-command-line-argument",
]


# MFMA results in ordinary VGPRs: avoids AGPR<->VGPR copies around the softmax.
# The backward files keep the compiler's own choice (the same VGPR form for
# every instance of two waves per SIMD): the dK/dV kernel keeps its
# accumulators in AGPRs where it runs one wave per SIMD, and the dQ instances
# of one wave per SIMD at head dim 256 do not compile with the VGPR form forced.
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form=true"]
FILE_FLAGS = {"fa_bwd_dkdv.hip": [], "fa_bwd.hip": []}


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile every HIP source and link libfa.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = [os.path.join(BUILD, os.path.basename(s)[:-4] + ".o") for s in srcs]

    def one(pair):
        src, obj = pair
        extra = FILE_FLAGS.get(os.path.basename(src), VGPR_FORM)
        return _run([HIPCC, *CFLAGS, *extra, "-c", src, "-o", obj])

    with ThreadPoolExecutor(max_workers=max(1, min(jobs, len(srcs)))) as ex:
        for out in ex.map(one, zip(srcs, objs)):
            if verbose and out.strip():
                print(out)
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
