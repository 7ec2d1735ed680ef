"""The C ABI on the host: the shared library loads, exports every function
include/calibatt.h declares, and rejects bad arguments before touching a
device. No GPU is needed."""

import ctypes
import os
import re

import numpy as np
import pytest
import torch

import calibrated_block_sparse_amd as cbs
import oracle
from synth import CALIB_WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "calibatt.h")


@pytest.fixture(scope="module")
def lib():
    return cbs.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(calibatt_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(cbs.SIGNATURES), "binding and header disagree"


def test_abi_version(lib):
    assert cbs.calibatt_abi_version() == 8


def fake(n=16):
    return ctypes.c_void_p(n * 4096)  # non-null, aligned; never dereferenced here


def attn(lib, **kw):
    args = dict(q=fake(), k=fake(), v=fake(), o=fake(), heads=2, n=1024, d=128, sh=1024 * 128,
                stok=128, scale=0.088, off=fake(), idx=fake(), nnz=10, flags=None, grid=None,
                ws=fake(), wsb=cbs.calibatt_sparse_attn_fwd_workspace(2, 1024))
    args.update(kw)
    return lib.calibatt_sparse_attn_fwd(args["q"], args["k"], args["v"], args["o"], args["heads"],
                                        args["n"], args["d"], args["sh"], args["stok"], args["scale"],
                                        args["off"], args["idx"], args["nnz"], args["flags"],
                                        args["grid"], args["ws"], args["wsb"], None)


def test_attention_workspace(lib):
    # one bf16 128 x 128 V^T tile per head and key block (R = ceil(N / 128))
    assert cbs.calibatt_sparse_attn_fwd_workspace(2, 1024) == 2 * 8 * 128 * 128 * 2
    assert cbs.calibatt_sparse_attn_fwd_workspace(40, 75600) == 40 * 591 * 128 * 128 * 2
    assert cbs.calibatt_sparse_attn_fwd_workspace(0, 100) == 0
    need = cbs.calibatt_sparse_attn_fwd_workspace(2, 1024)
    assert attn(lib, ws=None) == -4
    assert "workspace" in cbs.calibatt_last_error()
    assert attn(lib, wsb=need - 1) == -4
    assert attn(lib, ws=ctypes.c_void_p(4096 + 8)) == -4
    # the two halves check the same workspace
    assert lib.calibatt_prepare_vt(fake(), 2, 1024, 128, 1024 * 128, 128, fake(), need - 1, None) == -4
    assert lib.calibatt_prepare_vt(None, 2, 1024, 128, 1024 * 128, 128, fake(), need, None) == -1
    assert lib.calibatt_sparse_attn_fwd_vt(fake(), fake(), None, fake(), 2, 1024, 128, 1024 * 128,
                                           128, 0.088, fake(), fake(), 10, None, None, need,
                                           None) == -4


def test_attention_argument_errors(lib):
    assert attn(lib, d=64) == -2
    assert "head_dim" in cbs.calibatt_last_error()
    assert attn(lib, q=None) == -1
    assert attn(lib, q=ctypes.c_void_p(4096 + 2)) == -1
    assert attn(lib, stok=100) == -1
    assert attn(lib, stok=(1 << 23) + 8) == -2                 # 32-bit tile offsets
    assert "stride_token" in cbs.calibatt_last_error()
    assert attn(lib, scale=0.0) == -1
    assert attn(lib, scale=float("nan")) == -1
    assert attn(lib, nnz=-1) == -1
    assert attn(lib, off=None) == -1
    assert attn(lib, heads=-1) == -1
    flags = (ctypes.c_uint8 * 2)(0, 1)
    assert attn(lib, flags=flags) == -1                        # repeat head without grid
    g = cbs.Grid(2, 16, 30, 5)                                 # 960 != 1024 tokens
    assert attn(lib, flags=flags, grid=ctypes.byref(g)) == -1
    g = cbs.Grid(2, 16, 32, 17)                                # anchors > rows
    assert attn(lib, flags=flags, grid=ctypes.byref(g)) == -1
    g = cbs.Grid(2, 10, 50, 9)                                 # anchor row 1 would serve segment 0
    assert attn(lib, flags=flags, grid=ctypes.byref(g), n=1000, sh=1000 * 128,
                wsb=cbs.calibatt_sparse_attn_fwd_workspace(2, 1000)) == -2
    assert "anchor" in cbs.calibatt_last_error()
    g = cbs.Grid(2, 16, 32, 5)
    assert attn(lib, flags=(ctypes.c_uint8 * 2)(0, 3), grid=ctypes.byref(g)) == -1   # flag 3
    g = cbs.Grid(2, 450, 128, 5)                               # N = 115200: R = 900 > 896
    big = lambda **kw: attn(lib, n=115200, sh=115200 * 128,
                            wsb=cbs.calibatt_sparse_attn_fwd_workspace(2, 115200), **kw)
    assert big(flags=(ctypes.c_uint8 * 2)(0, 2), grid=ctypes.byref(g)) == -2
    # empty problems are no-ops and succeed
    assert attn(lib, heads=0) == 0 and attn(lib, n=0) == 0


def test_noalloc_argument_errors(lib):
    """calibatt_sparse_attn_fwd_noalloc checks its arguments as the full call
    does and rejects N beyond what its fixed scratch holds (8192 V^T tiles
    per head: N <= 1,048,576) before touching a device."""
    na = lambda **kw: lib.calibatt_sparse_attn_fwd_noalloc(
        kw.get("q", fake()), fake(), fake(), fake(), kw.get("heads", 2), kw.get("n", 1024), 128,
        kw.get("n", 1024) * 128, 128, kw.get("scale", 0.088), fake(), fake(), 10, None, None, None)
    assert na(n=8192 * 128 + 1) == -2
    assert "scratch" in cbs.calibatt_last_error()
    assert na(q=None) == -1
    assert na(scale=-1.0) == -1
    assert na(heads=0) == 0 and na(n=0) == 0


def test_energy_argument_errors(lib):
    ws = cbs.calibatt_block_energy_workspace(2, 1000)
    assert ws == 2 * 4 * 2 * 8 * 128 * (8 + 1)
    f = lambda **kw: lib.calibatt_block_energy(kw.get("q", fake()), fake(), kw.get("e", fake()),
                                               2, kw.get("n", 1000), kw.get("d", 128), 1000 * 128,
                                               128, 0.1, kw.get("ws", fake()), kw.get("wsb", ws), None)
    assert f(d=96) == -2
    assert f(q=None) == -1
    # a workspace for one head is enough (heads then go in chunks); less is not
    assert f(wsb=cbs.calibatt_block_energy_workspace(1, 1000) - 1) == -4
    assert f(ws=None) == -4
    assert f(ws=ctypes.c_void_p(4096 + 8)) == -4              # 16-byte alignment
    assert f(n=2048 * 128) == -2                               # R beyond the selection limit


def test_mask_argument_errors(lib):
    assert lib.calibatt_build_mask(fake(), 1, 1, 2048, 5, fake(), None, None) == -2
    assert lib.calibatt_build_mask(None, 1, 1, 8, 5, fake(), None, None) == -1
    assert lib.calibatt_build_mask(fake(), 0, 1, 8, 5, fake(), None, None) == 0
    fin = lambda n, rn, rd: lib.calibatt_finalize_mask(fake(), 1, 8, n, rn, rd, fake(), fake(),
                                                       fake(), None, None)
    assert fin(0, 1, 2) == -1 and fin(256, 1, 2) == -1 and fin(64, 3, 2) == -1 and fin(64, 1, 0) == -1
    assert lib.calibatt_compile_skiplist(fake(), 40, 8000, fake(), fake(), None, None) == -2


def test_similarity_argument_errors(lib):
    H, N = 2, 1000
    ws = cbs.calibatt_block_energy_workspace(H, N)
    good = cbs.Grid(2, 20, 25, 5)
    f = lambda **kw: lib.calibatt_spatial_similarity(kw.get("ws", fake()), kw.get("wsb", ws), H,
                                                     kw.get("n", N), kw.get("g", ctypes.byref(good)),
                                                     kw.get("prof", fake()), fake(), None)
    assert f(g=None) == -1
    assert f(g=ctypes.byref(cbs.Grid(2, 20, 24, 5))) == -1          # does not cover N
    assert f(g=ctypes.byref(cbs.Grid(2, 20, 25, 21))) == -1         # anchors > rows
    assert f(g=ctypes.byref(cbs.Grid(2, 20, 25, 19))) == -2         # anchors = rows - 1
    assert f(prof=None) == -1
    # a workspace for one head is enough (heads then go in chunks); less is not
    assert f(wsb=cbs.calibatt_block_energy_workspace(1, 1000) - 1) == -4
    assert f(ws=None) == -4
    assert lib.calibatt_spatial_similarity(None, 0, 0, N, None, None, None, None) == 0


def test_mfma_probe_argument_errors(lib):
    assert lib.calibatt_mfma_rate_probe(None, 10, 4, None) == -1
    assert lib.calibatt_mfma_rate_probe(fake(), -1, 4, None) == -1
    assert lib.calibatt_mfma_rate_probe(fake(), 10, -4, None) == -1
    assert lib.calibatt_mfma_rate_probe(fake(), 10, 0, None) == 0   # nothing to launch


def test_eps_fx_matches_oracle(lib):
    w = CALIB_WORKLOADS["calibration_480p"]
    for t in list(w.steps) + list(range(0, 50, 7)):
        eps = oracle.eps_schedule(t, w.total_steps, w.eps_floor, w.eps_start, w.eps_rate)
        assert cbs.calibatt_eps_fx(t, w.total_steps, w.eps_floor, w.eps_start, w.eps_rate) == oracle.eps_fx(eps)
    # LightX2V-style 4-step schedule
    for t in range(4):
        eps = oracle.eps_schedule(t, 4, 0.84, 0.99, 5.0)
        assert cbs.calibatt_eps_fx(t, 4, 0.84, 0.99, 5.0) == oracle.eps_fx(eps)


def test_validate_skiplist_host(lib):
    rng = np.random.Generator(np.random.PCG64(3))
    m = (rng.random((3, 9, 9)) < 0.4).astype(np.uint8)
    off, idx = oracle.compile_skiplist(m)
    cbs.calibatt_validate_skiplist(off, idx, 3, 9)
    bad = [
        (off, np.where(idx == idx.max(), 9, idx)),             # index out of range
        (off, idx[::-1].copy()),                               # not ascending
        (np.r_[1, off[1:]], idx),                              # offsets[0] != 0
    ]
    o2 = off.copy()
    o2[5] = o2[4] - 1                                          # decreasing offsets
    bad.append((o2, idx))
    for o, i in bad:
        with pytest.raises(cbs.CalibAttError) as e:
            cbs.calibatt_validate_skiplist(o, i, 3, 9)
        assert e.value.code == -3


def test_validate_skiplist_offsets_past_nnz(lib):
    """Offsets that rise past nnz and fall back (first row [0, R), nnz = 0)
    pass the checks on offsets[0], offsets[rows] and row 0's length; the
    validator must reject them before it reads any index."""
    R = 9
    off = np.zeros(2 * R + 1, np.int32)
    off[1] = R                                                 # [0, R, 0, ..., 0], nnz = 0
    with pytest.raises(cbs.CalibAttError) as e:
        cbs.calibatt_validate_skiplist(off, np.zeros(0, np.int32), 2, R)
    assert e.value.code == -3 and "outside" in str(e.value)
    # the same through the raw C entry point with a NULL index array (legal for nnz = 0)
    assert lib.calibatt_validate_skiplist(off.ctypes.data_as(ctypes.c_void_p), None, 0, 2, R) == -3
    # an offset past nnz in the middle of otherwise valid lists
    m = np.ones((1, R, R), np.uint8)
    o2, i2 = oracle.compile_skiplist(m)
    o2 = o2.copy()
    o2[4] = i2.size + 5
    with pytest.raises(cbs.CalibAttError) as e:
        cbs.calibatt_validate_skiplist(o2, i2, 1, R)
    assert e.value.code == -3


def test_launch_stream_rejects_host_tensors():
    # the binding refuses tensors that are not on a GPU before it asks for a
    # stream or calls the library
    with pytest.raises(ValueError, match="CUDA"):
        cbs._stream(None, torch.zeros(4))
