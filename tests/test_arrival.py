"""The decode step's generation-tagged arrival counters (csrc/pkv_arrival.h) on the host: the
native test interleaves the two atomic steps of every piece's arrival at random over thousands of
calls, some of which stop part-way, and requires exactly one last arrival per sequence in every
complete call.  Built alone with g++ AddressSanitizer + UBSan."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_arrival_counters_native(tmp_path):
    exe = tmp_path / "arrival_test"
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-Wall", "-Werror",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    os.path.join(ROOT, "tests", "native", "arrival_test.cpp"), "-o", str(exe)],
                   check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "arrival counters ok" in r.stdout
