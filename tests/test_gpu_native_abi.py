"""The C ABI driven from C++ alone: tests/native_abi.cpp includes only
include/hpcattn.h, runs plan -> decode -> combine, the fused call with
tickets and the no-allocation variant over a ragged paged batch (empty,
one-token, tile-edge and multi-bin requests), and compares each result
with the fp64 C oracle. The binary is built by __graft_entry__.build()."""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
BIN = os.path.join(HERE, "native_abi")


@pytest.mark.gpu
def test_native_cpp_caller_matches_oracle():
    if not os.path.exists(BIN):
        pytest.fail("tests/native_abi is not built; run __graft_entry__.build()")
    r = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    print(r.stdout)
    print(r.stderr)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all checks passed" in r.stdout
