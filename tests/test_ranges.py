"""Host check of the kernels' buffer-resource byte ranges (csrc/ranges.h).

A buffer resource's range field is 32 bits; the kernels saturate ranges of
2^31 bytes or more instead of narrowing them, so a query block of a tensor
whose remaining rows span 4 GiB or more still sees all of its rows.  The
header is plain C++ and is compiled here with g++ (no GPU needed).
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "transformer_attention_09_amd", "csrc")


def test_range_arithmetic(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path / "ranges_check")
    subprocess.run([gxx, "-std=c++17", "-O1", "-I", CSRC, os.path.join(HERE, "ranges_check.cpp"), "-o", exe],
                   check=True)
    r = subprocess.run([exe], capture_output=True, text=True)
    print(r.stdout)
    assert r.returncode == 0, r.stdout
    assert "FAIL" not in r.stdout and r.stdout.count("ok ") == 11
