"""GPU: the attention path driven from a plain C program
(tests/c_consumer/attn_gpu.c: HIP runtime API and include/calibatt.h only,
no torch in its process). It compiles the mask into kept lists on the
device and runs calibatt_sparse_attn_fwd; its output matches the oracle
(max-abs <= 2e-2, rel-Frobenius <= 1e-2), and calibatt_sparse_attn_fwd_noalloc
called from the same program gives the same bytes."""

import os
import shutil
import struct
import subprocess

import numpy as np
import pytest

import oracle
from synth import bernoulli_mask, bf16_bits, gaussian_bf16, n_blocks
from tests._util import assert_attn_close, say

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "calibrated_block_sparse_amd")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_attention_from_plain_c(tmp_path):
    H, N = 2, 1000
    R = n_blocks(N)
    scale = 128 ** -0.5
    say(f"case plain C attention H={H} N={N}")
    exe = str(tmp_path / "attn_gpu")
    cmd = ["gcc", "-std=c99", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
           "-I", "/opt/rocm/include", os.path.join(ROOT, "tests", "c_consumer", "attn_gpu.c"), "-o", exe,
           "-L", PKG, "-lcalibatt", "-L", "/opt/rocm/lib", "-lamdhip64", f"-Wl,-rpath,{PKG}",
           "-Wl,-rpath,/opt/rocm/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    q, k, v = (gaussian_bf16(520 + i, (H, N, 128)) for i in range(3))
    mask = bernoulli_mask(523, H, R, 0.4, True)
    mask[1, 2, :] = 0                                   # an empty list -> zeros
    bits = [np.stack([bf16_bits(t[h]) for h in range(H)]) for t in (q, k, v)]
    src, dst = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(src, "wb") as f:
        f.write(struct.pack("<iif", H, N, scale))
        for b in bits:
            f.write(np.ascontiguousarray(b, dtype=np.uint16).tobytes())
        f.write(np.ascontiguousarray(mask, dtype=np.uint8).tobytes())
    r = subprocess.run([exe, str(src), str(dst)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    say(f"  {r.stdout.strip()}")
    assert r.stdout.strip() == f"ok nnz={int(mask.sum())} noalloc=equal"
    out = np.fromfile(dst, dtype=np.uint16).reshape(H, N, 128)
    got = (out.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    for h in range(H):
        want = oracle.block_sparse_attention(bits[0][h], bits[1][h], bits[2][h], scale, mask[h])
        assert_attn_close(got[h], want, f"head {h}")
    assert not got[1, 256:384].any()
