"""Build step of the HIP library libqt.so (gfx950), in-tree.

    python -m codec_lm_autoregressive_amd.build

Each source is compiled to its own object in parallel (hipcc, gfx950 only),
then the objects are linked into libqt.so next to this file.
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
SRC = [os.path.join(CSRC, n) for n in ("qt_linear.hip", "qt_attn.hip", "qt_select.hip", "qt_frontend.hip", "qt_codec.hip", "qt_api.hip")]
LIB = os.path.join(PKG, "libqt.so")
HIPCC = "/opt/rocm/bin/hipcc"

FLAGS = ["-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC",
         # packed fp32 instructions are kept out of generated code on purpose
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I" + os.path.join(ROOT, "include"), "-I" + CSRC]


def compile_cmd(src, obj):
    return [HIPCC, *FLAGS, "-c", src, "-o", obj]


def link_cmd(objs, out):
    return [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", out]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    return r.returncode, r.stdout + r.stderr


def build(verbose=False):
    with tempfile.TemporaryDirectory(prefix="qt_build_") as tmp:
        objs = [os.path.join(tmp, os.path.basename(s) + ".o") for s in SRC]
        with ThreadPoolExecutor(max_workers=len(SRC)) as ex:
            results = list(ex.map(_run, [compile_cmd(s, o) for s, o in zip(SRC, objs)]))
        for (rc, out), s in zip(results, SRC):
            if rc != 0 or verbose:
                sys.stderr.write(out)
            if rc != 0:
                raise RuntimeError(f"hipcc failed on {os.path.basename(s)}")
        tmp_lib = LIB + ".tmp"
        rc, out = _run(link_cmd(objs, tmp_lib))
        if rc != 0:
            sys.stderr.write(out)
            raise RuntimeError("linking libqt.so failed")
    os.replace(tmp_lib, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
