"""The host code under the address and undefined-behaviour sanitizers (CPU).

* The C ABI's argument validation (csrc/validate.cpp, free of HIP) is built
  with g++ -fsanitize=address,undefined together with a driver
  (sanitize_validate.cpp) that calls every check over valid arguments and the
  edges of every range, including the int32 limits where a product could
  wrap; any report or wrong status fails the run.
* The fp64 oracle (oracle/oracle.c) is built with gcc and the same
  sanitizers, and the oracle's own pinned tests run against that build in a
  child process with the sanitizer runtimes preloaded.
Neither build involves hipcc or device code.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "load_balanced_split_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _runtime(name):
    path = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


pytestmark = pytest.mark.skipif(_runtime("libasan.so") is None,
                                reason="gcc's sanitizer runtimes are not installed")


def test_validation_under_sanitizers(tmp_path):
    exe = str(tmp_path / "sanitize_validate")
    subprocess.check_call(["g++", "-std=c++17", "-O1", "-g", "-Wall"] + SAN +
                          ["-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
                           os.path.join(CSRC, "validate.cpp"),
                           os.path.join(ROOT, "tests", "sanitize_validate.cpp"), "-o", exe])
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr)
    assert r.returncode == 0, r.stderr
    assert "all checks passed" in r.stdout


def test_oracle_suite_under_sanitizers(tmp_path):
    lib = str(tmp_path / "liboracle_san.so")
    subprocess.check_call(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-Wall", "-shared",
                           "-fPIC"] + SAN + [os.path.join(ROOT, "oracle", "oracle.c"), "-o", lib,
                                             "-lm"])
    env = dict(os.environ)
    env["ORACLE_LIB"] = lib
    env["LD_PRELOAD"] = ":".join(p for p in (_runtime("libasan.so"), _runtime("libubsan.so"))
                                 if p)
    # Python's own allocations are not ours to check for leaks.
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:exitcode=97"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1:exitcode=98"
    env["OMP_NUM_THREADS"] = "2"
    tests = [os.path.join(ROOT, "tests", t) for t in
             ("test_oracle.py", "test_plan_cpu.py", "test_oracle_mtp.py",
              "test_oracle_prologue.py")]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-m", "not gpu"] + tests, capture_output=True, text=True, env=env,
                       cwd=ROOT, timeout=600)
    print(r.stdout[-3000:], r.stderr[-3000:])
    assert r.returncode == 0, (r.returncode, r.stderr[-2000:])
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr
