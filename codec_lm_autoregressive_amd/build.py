"""Build step of the HIP library libqt.so (gfx950), in-tree.

    python -m codec_lm_autoregressive_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = [os.path.join(PKG, "csrc", "qt_kernels.hip"), os.path.join(PKG, "csrc", "qt_api.hip")]
LIB = os.path.join(PKG, "libqt.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def command(out=LIB):
    return [HIPCC, "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-shared",
            # packed fp32 instructions are kept out of generated code on purpose
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(PKG, "csrc"),
            *SRC, "-o", out]


def build(verbose=False):
    tmp = LIB + ".tmp"
    cmd = command(tmp)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building libqt.so")
    if verbose:
        sys.stderr.write(r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
