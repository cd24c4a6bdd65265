"""Build the HIP library ``libswin_wmsa.so`` in-tree for gfx950.

    python -m shifted_window_attention_roll_amd.build

Every HIP source under ``csrc/`` is compiled with hipcc for gfx950 only.  Packed
float32 VALU instructions are disabled (``-packed-fp32-ops``); the host pass of
hipcc warns that it does not know that feature, which is harmless.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libswin_wmsa.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-fno-honor-nans",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-command-line-argument", "-parallel-jobs=4"]


def sources():
    return sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))


def build(verbose: bool = False) -> str:
    """Compile the library (always, even when a built copy exists) and return its path."""
    if not os.path.exists(HIPCC) and shutil.which("hipcc") is None:
        raise RuntimeError("hipcc not found: cannot build the gfx950 library")
    hipcc = HIPCC if os.path.exists(HIPCC) else shutil.which("hipcc")
    tmp = LIB + ".tmp"
    cmd = [hipcc, *FLAGS, "-I", os.path.join(ROOT, "include"), *sources(), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    errs = [l for l in res.stderr.splitlines()
            if "packed-fp32-ops" not in l and "hip-link" not in l and l.strip()]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(errs))
    if errs and verbose:
        print("\n".join(errs), file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
