"""The oracle's C code under AddressSanitizer and UndefinedBehaviorSanitizer (host only).

oracle.c is compiled with -fsanitize=address,undefined (gcc, the oracle's own arithmetic
flags otherwise), and the oracle's CPU tests run against that build in a child process
with the sanitizer runtimes preloaded into the interpreter.  Any out-of-bounds access or
undefined behaviour in the oracle fails the run.  A planted out-of-bounds read (a 2-word
counter handed to the 4-word Philox routine) shows that the harness does catch one.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")
ORACLE_TESTS = ["clip", "ef", "gathered", "qsgd", "quant", "randk", "ratio", "select", "sign",
                "threshold"]


def _runtime(name):
    r = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


@pytest.fixture(scope="module")
def sanitized(tmp_path_factory):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not (asan and ubsan):
        pytest.skip("gcc's sanitizer runtimes are not installed")
    so = str(tmp_path_factory.mktemp("san") / "liboracle_san.so")
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
                    "-fno-fast-math", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", SRC, "-o", so,
                    "-lm"], check=True)
    env = dict(os.environ, GC_ORACLE_LIB=so, LD_PRELOAD=f"{asan} {ubsan}",
               ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    return so, env


def test_oracle_tests_pass_under_sanitizers(sanitized):
    _, env = sanitized
    files = [os.path.join("tests", f"test_oracle_{t}.py") for t in ORACLE_TESTS]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu",
                        "-p", "no:cacheprovider", *files],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    log = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, log
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, log


def test_sanitized_build_catches_a_planted_overread(sanitized):
    so, env = sanitized
    code = ("import numpy as np, oracle\n"
            "L = oracle.lib()\n"
            "c = np.zeros(2, np.uint32); k = np.zeros(2, np.uint32); o = np.zeros(4, np.uint32)\n"
            "L.orc_philox4x32_10(c.ctypes.data, k.ctypes.data, o.ctypes.data)\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr, r.stderr[-2000:]
