"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

libgc is built again with the sanitizers on its host side only (each -fsanitize= behind
-Xarch_host: the gfx950 code is built as usual), and the CPU tests of the plan's host logic
(k from a ratio, the output layout, every argument check of gc_layout and gc_plan_create,
the exported symbols and status strings) run against that build in a child process with
clang's sanitizer runtime preloaded.  An out-of-bounds access or undefined behaviour in that
code fails the run.  A planted overflow (an out_off array one entry short handed to
gc_layout) shows that the harness does catch one.
"""
import glob
import os
import subprocess
import sys

import pytest

from gradient_compression_amd import build as gc_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _clang_asan_runtime():
    llvm = os.path.join(os.path.dirname(os.path.dirname(gc_build.hipcc())), "llvm")
    for base in (llvm, "/opt/rocm/llvm"):
        hits = sorted(glob.glob(os.path.join(base, "lib", "clang", "*", "lib", "linux",
                                             "libclang_rt.asan-x86_64.so")))
        if hits:
            return hits[-1]
    return None


@pytest.fixture(scope="module")
def sanitized(tmp_path_factory):
    rt = _clang_asan_runtime()
    if rt is None:
        pytest.skip("clang's AddressSanitizer runtime is not installed")
    so = str(tmp_path_factory.mktemp("san") / "libgc_san.so")
    cmd = [gc_build.hipcc(), *gc_build.flags(), "-g", "-fno-omit-frame-pointer",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-shared-libsan",
           *gc_build.SOURCES, "-o", so]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    env = dict(os.environ, GC_LIB_PATH=so, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    return so, env


def test_host_logic_tests_pass_under_sanitizers(sanitized):
    _, env = sanitized
    files = [os.path.join("tests", "test_layout_host.py"), os.path.join("tests", "test_abi.py")]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu",
                        "-p", "no:cacheprovider", "-k", "not variant", *files],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    log = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, log
    assert " passed" in r.stdout, log
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, log


def test_sanitized_build_catches_a_planted_overflow(sanitized):
    so, env = sanitized
    code = ("import numpy as np, gradient_compression_amd as gca\n"
            f"assert gca.LIB_PATH == {so!r}\n"
            "L = gca.lib()\n"
            "off = np.array([0, 10, 20, 30], np.int64); k = np.ones(3, np.int64)\n"
            "k_out = np.zeros(3, np.int64); out_off = np.zeros(3, np.int64)  # needs 4\n"
            "L.gc_layout(off.ctypes.data, 3, k.ctypes.data, None, k_out.ctypes.data,\n"
            "            out_off.ctypes.data)\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr, r.stderr[-2000:]
