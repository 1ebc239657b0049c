"""The standalone C++ test of the C ABI (tests/standalone/decode_tiny.cpp),
run as its own process: cache write, split-K + combine at three split
counts, the split-K pass with the cache write folded in (output and cache
bytes), the whole-decode call and the whole decode without a workspace, on
the tiny workload, against the oracle's output stored in
tests/golden/tiny_decode.txt."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
BIN = os.path.join(HERE, "standalone", "decode_tiny")
GOLDEN = os.path.join(HERE, "golden", "tiny_decode.txt")


def test_standalone_cpp_decode():
    if not os.path.exists(BIN):
        pytest.fail(f"{BIN} is missing: build it with __graft_entry__.build()")
    res = subprocess.run([BIN, GOLDEN], capture_output=True, text=True, timeout=120)
    print(res.stdout)
    assert res.returncode == 0, res.stdout + res.stderr
    assert res.stdout.strip().endswith("PASS")
