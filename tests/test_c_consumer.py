"""The C ABI from plain C: tests/c_consumer/consumer.c includes only
include/calibatt.h, is compiled with gcc, links libcalibatt.so and runs its
host-side checks (no GPU, no Python in the loop)."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "calibrated_block_sparse_amd")
LIB = os.path.join(PKG, "libcalibatt.so")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_plain_c_consumer(tmp_path):
    if not os.path.exists(LIB):
        pytest.skip("libcalibatt.so not built")
    exe = str(tmp_path / "consumer")
    cmd = ["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c_consumer", "consumer.c"), "-o", exe,
           "-L", PKG, "-lcalibatt", f"-Wl,-rpath,{PKG}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe, str(tmp_path / "bank.cbsm")], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip() == "ok"
