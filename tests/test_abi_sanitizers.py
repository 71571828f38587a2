"""The C-ABI's host code (argument validation, overflow-checked workspace
planning, the context state machine) under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU.

The host side of qt_api.hip is compiled with both sanitizers (device code is
built as usual: the instrumentation is host-only), linked with the kernel
objects into a temporary library, and tests/test_abi_cpu.py runs against it
in a child process with the sanitizer runtime preloaded; any report ends that
process with a failure. No GPU is touched (those tests make no device call).
"""
import glob
import os
import subprocess
import sys
import tempfile

import pytest

from codec_lm_autoregressive_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
RUNTIME = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]

pytestmark = pytest.mark.skipif(not RUNTIME or not os.path.exists(build.HIPCC),
                                reason="hipcc or the clang sanitizer runtime is missing")

CHILD = r"""
import sys
sys.path.insert(0, sys.argv[1])
from codec_lm_autoregressive_amd import binding
binding.LIB_PATH = sys.argv[2]
import pytest
sys.exit(pytest.main(["-q", "-p", "no:cacheprovider", sys.argv[3]]))
"""


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    return r


def test_abi_host_code_under_asan_and_ubsan():
    with tempfile.TemporaryDirectory(prefix="qt_asan_") as tmp:
        objs = []
        procs = []
        for src in build.SRC:
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            extra = HOST_SAN if src.endswith("qt_api.hip") else []
            procs.append(subprocess.Popen([build.HIPCC, *build.FLAGS, *extra, "-c", src, "-o", obj],
                                          stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
            objs.append(obj)
        for p in procs:
            out = p.communicate()[0]
            assert p.returncode == 0, out[-3000:]
        lib = os.path.join(tmp, "libqt_san.so")
        _run([build.HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
              "-Xarch_host", "-fsanitize=undefined", "-shared-libsan", *objs, "-o", lib])
        syms = _run(["nm", "-D", lib]).stdout
        assert "__asan_report" in syms and "__ubsan_handle" in syms   # the host code is instrumented
        env = dict(os.environ, LD_PRELOAD=RUNTIME[-1], LD_LIBRARY_PATH=os.path.dirname(RUNTIME[-1]),
                   ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
                   UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
        r = subprocess.run([sys.executable, "-c", CHILD, ROOT, lib, os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                           capture_output=True, text=True, env=env, cwd=ROOT, timeout=600)
        report = r.stdout[-4000:] + r.stderr[-4000:]
        assert r.returncode == 0, report
        assert "ERROR: AddressSanitizer" not in report and "runtime error" not in report, report
        assert " passed" in r.stdout
