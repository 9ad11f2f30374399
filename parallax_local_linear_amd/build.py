"""Build the gfx950 Parallax library (``libparallax.so``) in-tree with hipcc.

Run ``python -m parallax_local_linear_amd.build`` (or call ``build()``).  The
library is a plain C-ABI shared object; it does not link against torch.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(PKG, "libparallax.so")
BUILD_DIR = os.path.join(ROOT, "_build")

SOURCES = ["parallax_api.hip", "parallax_fwd.hip", "parallax_bwd.hip", "parallax_decode.hip",
           "parallax_proj.hip", "parallax_hadamard.hip", "parallax_based.hip", "parallax_f32.hip"]
# Kernel sources: no NaN ever reaches a max or compare (masking uses -inf and
# non-finite inputs are outside the contract), so max chains need no NaN
# canonicalisation.  The host API keeps IEEE NaN semantics for its argument
# checks.
KERNEL_FLAGS = {
    "parallax_fwd.hip": ["-fno-honor-nans"],
    "parallax_bwd.hip": ["-fno-honor-nans"],
    "parallax_decode.hip": ["-fno-honor-nans"],
    "parallax_proj.hip": ["-fno-honor-nans"],
    "parallax_hadamard.hip": ["-fno-honor-nans"],
    "parallax_based.hip": ["-fno-honor-nans"],
    "parallax_f32.hip": ["-fno-honor-nans"],
}
ARCH = "gfx950"

# Packed fp32 VALU forms are kept out of the generated code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON_FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH, "-Wall",
                "-Wno-unused-command-line-argument", "-I" + CSRC, "-I" + INCLUDE]


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; the ROCm toolchain is required to build")
    return exe


def build(verbose: bool = False, extra_flags=()) -> str:
    """Compile every HIP source for gfx950 and link ``libparallax.so``."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    objects = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        cmd = [hipcc(), *COMMON_FLAGS, *DEVICE_FLAGS, *KERNEL_FLAGS.get(src, []), *extra_flags, "-c",
               os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        # hipcc's host pass does not know the packed-fp32 feature and says so;
        # everything else it prints is shown.
        msgs = [ln for ln in (res.stdout + res.stderr).splitlines()
                if "packed-fp32-ops" not in ln]
        if res.returncode != 0:
            raise RuntimeError("hipcc failed on %s:\n%s" % (src, "\n".join(msgs)))
        if msgs and verbose:
            print("\n".join(msgs))
        objects.append(obj)
    tmp = LIBRARY + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "-shared", "-fPIC", "--offload-arch=" + ARCH, *objects, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
