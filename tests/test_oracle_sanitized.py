"""The C++ oracle under AddressSanitizer and UndefinedBehaviorSanitizer
(host code only).

The C++ oracle holds hand-written wide-integer arithmetic (the 512-bit exact
mean, the 2304-bit exact sums of squares and of binary64 values) and plain
loops over caller-sized buffers.  This test builds it a second time with
``-fsanitize=address,undefined`` (any report is fatal), and runs the C++
oracle's own pin tests through that build in a child Python process with
the sanitizer runtimes preloaded: exact ties, subnormals, NaN and Inf, the
largest and smallest exponents, the brute-force and cross-oracle checks.
The child fails on the first report.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "cpp", "onebit_ref.cpp")

# the release flags of oracle/cref.py, with the sanitizers and frame
# pointers added (-O1 keeps the reports precise)
FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-std=c++17", "-fPIC", "-shared",
         "-ffp-contract=off", "-fno-fast-math", "-fno-math-errno", "-Wall", "-Wextra",
         "-Werror", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]

CHILD = r"""
import sys
sys.path.insert(0, {root!r})
from oracle import cref
cref.LIB = {lib!r}       # the sanitized build (newer than the source: no rebuild)
cref.load()
import pytest
# --capture=sys: a sanitizer report goes to file descriptor 2, which must
# stay the process's own stderr
sys.exit(pytest.main(["-q", "-x", "-p", "no:cacheprovider", "--capture=sys", "-m", "not gpu",
                      {tests!r}]))
"""


def _runtime(name: str) -> str:
    out = subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True, text=True)
    path = out.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else ""


@pytest.mark.timeout(600)
def test_cpp_oracle_pins_under_asan_and_ubsan(tmp_path):
    if shutil.which("g++") is None:
        pytest.skip("no g++")
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("g++ sanitizer runtimes not installed")
    lib = str(tmp_path / "libonebit_ref_san.so")
    build = subprocess.run(["g++", *FLAGS, "-o", lib, SRC], capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    env = dict(os.environ)
    env["LD_PRELOAD"] = f"{asan}:{ubsan}"
    # Python itself is not built with the sanitizers: its allocations at exit
    # are not leaks of the oracle
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    tests = os.path.join(ROOT, "tests", "test_oracle_cref.py")
    code = CHILD.format(root=ROOT, lib=lib, tests=tests)
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                         env=env, cwd=ROOT, timeout=560)
    report = "\n".join((res.stdout + res.stderr).splitlines()[-40:])
    assert res.returncode == 0, report
    assert "ERROR: AddressSanitizer" not in res.stderr, report
    assert "runtime error" not in res.stderr, report
    assert " passed" in res.stdout, report
