"""Mask bank on the host (no GPU): the file written by calibatt_bank_write
matches the documented layout byte for byte (rebuilt here with struct and an
FNV-1a-64 pinned to its published test vectors), every (t, l) reads back
bit-exact, and corrupt files and malformed lists are rejected."""

import os
import struct

import numpy as np
import pytest
import torch

import calibrated_block_sparse_amd as cbs
from calibrated_block_sparse_amd.bank import MaskBank, write_bank

import oracle
from synth import bernoulli_mask


def fnv1a64(data: bytes) -> int:
    h = 0xcbf29ce484222325
    for b in data:
        h ^= b
        h = (h * 0x100000001b3) & 0xFFFFFFFFFFFFFFFF
    return h


def test_fnv1a64_published_vectors():
    # test vectors of the FNV reference (Fowler / Noll / Vo): empty input is
    # the offset basis; "a" and "foobar" from the published FNV-1a 64 table
    assert fnv1a64(b"") == 0xcbf29ce484222325
    assert fnv1a64(b"a") == 0xaf63dc4c8601ec8c
    assert fnv1a64(b"foobar") == 0x85944171f73967e8


def make_entries(H, N, seeds, rep=None):
    """Kept-block lists compiled by the oracle from seeded Bernoulli masks."""
    R = cbs.n_blocks(N)
    out = []
    for i, s in enumerate(seeds):
        mask = bernoulli_mask(s, H, R, 0.4, True)
        off, idx = oracle.compile_skiplist(mask)
        flags = None if rep is None else np.array(rep[i], dtype=np.uint8)
        out.append((off.astype(np.int32), idx.astype(np.int32), flags))
    return out


def expected_bytes(T, L, H, N, grid, entry_of, entries):
    """The file as include/calibatt.h describes it, built independently."""
    R = cbs.n_blocks(N)
    E = len(entries)
    table_off = 128 + 4 * T * L
    pos = -(-(table_off + 24 * E) // 256) * 256
    payloads, offs = [], []
    for off, idx, fl in entries:
        f = bytes(H) if fl is None else bytes(fl.tolist())
        body = f + bytes(-H % 4) + off.astype("<i4").tobytes() + idx.astype("<i4").tobytes()
        offs.append(pos)
        payloads.append(body)
        pos = -(-(pos + len(body)) // 256) * 256
    size = pos
    buf = bytearray(size)
    buf[128:table_off] = np.asarray(entry_of, dtype="<i4").tobytes()
    for e, (body, o) in enumerate(zip(payloads, offs)):
        nnz = len(entries[e][1])
        buf[table_off + 24 * e: table_off + 24 * (e + 1)] = struct.pack("<qqQ", o, nnz, fnv1a64(body))
        buf[o:o + len(body)] = body
    g = grid or (0, 0, 0, 0)
    hdr = b"CBSMBNK1" + struct.pack("<II", 1, 128) + struct.pack("<10i", T, L, H, N, R, *g, E) + \
        struct.pack("<qq", table_off, size)
    hdr += struct.pack("<Q", fnv1a64(bytes(buf[128:])))
    buf[:len(hdr)] = hdr
    return bytes(buf)


@pytest.fixture
def bank_case(tmp_path):
    H, N, T, L = 3, 1000, 4, 2
    grid = (2, 20, 25, 5)
    entries = make_entries(H, N, [71, 72, 73], rep=[[0, 0, 0], [0, 1, 0], [1, 1, 1]])
    entry_of = [[0, 1], [0, 1], [2, 1], [2, 0]]
    path = str(tmp_path / "bank.cbsm")
    write_bank(path, T, L, H, N, entry_of, entries, grid)
    return path, (T, L, H, N, grid, entry_of, entries)


def test_file_layout_matches_spec(bank_case):
    path, (T, L, H, N, grid, entry_of, entries) = bank_case
    got = open(path, "rb").read()
    want = expected_bytes(T, L, H, N, grid, entry_of, entries)
    assert len(got) == len(want)
    assert got == want


def test_round_trip_every_step_and_layer(bank_case):
    path, (T, L, H, N, grid, entry_of, entries) = bank_case
    b = MaskBank(path)
    assert b.shape == (T, L, H, N) and b.grid == grid
    assert b.info.n_entries == 3 and b.info.total_nnz == sum(len(e[1]) for e in entries)
    for t in range(T):
        for l in range(L):
            e, off, idx, fl = b.lookup_host(t, l)
            assert e == entry_of[t][l]
            want = entries[e]
            assert np.array_equal(off, want[0]) and np.array_equal(idx, want[1])
            assert np.array_equal(fl, want[2])
    b.close()


def test_no_grid_and_empty_lists(tmp_path):
    H, N = 2, 300
    R = cbs.n_blocks(N)
    empty = (np.zeros(H * R + 1, np.int32), np.zeros(0, np.int32), None)
    full = make_entries(H, N, [5])[0]
    path = str(tmp_path / "b.cbsm")
    write_bank(path, 1, 2, H, N, [[1, 0]], [empty, full])
    b = MaskBank(path)
    assert b.grid is None
    e, off, idx, fl = b.lookup_host(0, 1)
    assert e == 0 and idx.size == 0 and not off.any() and not fl.any()
    assert open(path, "rb").read() == expected_bytes(1, 2, H, N, None, [[1, 0]], [empty, full])


def corrupt(path, at, value=None):
    data = bytearray(open(path, "rb").read())
    data[at] = (data[at] ^ 0x5A) if value is None else value
    open(path, "wb").write(bytes(data))


def test_corrupt_files_are_rejected(bank_case, tmp_path):
    path, (T, L, H, N, grid, entry_of, entries) = bank_case
    size = os.path.getsize(path)

    def code(p):
        with pytest.raises(cbs.CalibAttError) as ei:
            MaskBank(p)
        return ei.value.code

    assert code(str(tmp_path / "missing.cbsm")) == -6
    corrupt(path, size - 300)                        # inside the last payload
    assert code(path) == -6
    write_bank(path, T, L, H, N, entry_of, entries, grid)
    corrupt(path, 0)                                 # magic
    assert code(path) == -6
    write_bank(path, T, L, H, N, entry_of, entries, grid)
    corrupt(path, 8, 2)                              # version 2
    assert code(path) == -6
    write_bank(path, T, L, H, N, entry_of, entries, grid)
    open(path, "r+b").truncate(size - 256)           # truncated
    assert code(path) == -6


def test_header_fields_outside_the_checksum_are_checked(bank_case):
    """The file checksum covers bytes 128.. only; header fields that
    contradict the rest are still reported as a corrupt file."""
    path, (T, L, H, N, grid, entry_of, entries) = bank_case
    good = open(path, "rb").read()
    for at, value in ((16, 0),                  # steps = 0
                      (32, 9),                  # n_blocks != ceil(N / 128)
                      (36, grid[0] + 1)):       # grid no longer covers N
        data = bytearray(good)
        data[at:at + 4] = struct.pack("<i", value)
        open(path, "wb").write(bytes(data))
        with pytest.raises(cbs.CalibAttError) as ei:
            MaskBank(path)
        assert ei.value.code == -6, (at, value, ei.value)


def test_offsets_past_nnz_in_a_checksummed_file(tmp_path):
    """A bank whose lists have offsets rising past nnz and falling back
    ([0, R, 0, ...] with nnz = 0), written with correct checksums (anyone
    can recompute them), is rejected as a malformed list before any index
    is read."""
    H, N = 2, 1000
    R = cbs.n_blocks(N)
    off = np.zeros(H * R + 1, np.int32)
    off[1] = R
    entries = [(off, np.zeros(0, np.int32), None)]
    path = str(tmp_path / "crafted.cbsm")
    open(path, "wb").write(expected_bytes(1, 1, H, N, None, [[0]], entries))
    with pytest.raises(cbs.CalibAttError) as ei:
        MaskBank(path)
    assert ei.value.code == -3


def test_writer_rejects_bad_input(tmp_path):
    H, N = 2, 600
    path = str(tmp_path / "bad.cbsm")
    off, idx, _ = make_entries(H, N, [9])[0]
    bad_idx = idx.copy()
    bad_idx[[0, 1]] = bad_idx[[1, 0]]                # not ascending
    with pytest.raises(cbs.CalibAttError) as ei:
        write_bank(path, 1, 1, H, N, [[0]], [(off, bad_idx, None)])
    assert ei.value.code == -3
    with pytest.raises(cbs.CalibAttError) as ei:
        write_bank(path, 1, 1, H, N, [[1]], [(off, idx, None)])      # entry out of range
    assert ei.value.code == -1
    with pytest.raises(cbs.CalibAttError) as ei:
        write_bank(path, 1, 1, H, N, [[0]], [(off, idx, np.array([0, 3], np.uint8))])
    assert ei.value.code == -1
    with pytest.raises(cbs.CalibAttError) as ei:                     # repeat head, no grid
        write_bank(path, 1, 1, H, N, [[0]], [(off, idx, np.array([0, 1], np.uint8))])
    assert ei.value.code == -1
    with pytest.raises(cbs.CalibAttError) as ei:                     # grid not covering N
        write_bank(path, 1, 1, H, N, [[0]], [(off, idx, None)], grid=(2, 10, 10, 5))
    assert ei.value.code == -1
    with pytest.raises(cbs.CalibAttError) as ei:                     # anchors off their segments
        write_bank(path, 1, 1, H, N, [[0]], [(off, idx, np.array([0, 1], np.uint8))],
                   grid=(2, 10, 30, 9))
    assert ei.value.code == -2
    assert not os.path.exists(path) and not os.path.exists(path + ".tmp")


def test_lookup_errors(bank_case):
    path, (T, L, *_rest) = bank_case
    b = MaskBank(path)
    with pytest.raises(cbs.CalibAttError) as ei:
        b.lookup_host(T, 0)
    assert ei.value.code == -1
    with pytest.raises(cbs.CalibAttError) as ei:
        b.lookup_host(0, -1)
    assert ei.value.code == -1
    with pytest.raises(RuntimeError):
        b.lookup(0, 0)                               # not uploaded


def test_custom_op_fake_shape():
    from calibrated_block_sparse_amd import bank  # noqa: F401  (registers the op)
    q = torch.empty(2, 300, 128, dtype=torch.bfloat16, device="meta")
    off = torch.empty(2 * 3 + 1, dtype=torch.int32, device="meta")
    idx = torch.empty(5, dtype=torch.int32, device="meta")
    o = torch.ops.calibatt.sparse_attn(q, q, q, off, idx, None, None, 0.1, None)
    assert o.shape == q.shape and o.dtype == q.dtype and o.device.type == "meta"
    ws = torch.empty(2 * 3 * 128 * 128 * 2, dtype=torch.uint8, device="meta")
    o = torch.ops.calibatt.sparse_attn(q, q, q, off, idx, None, None, 0.1, ws)
    assert o.shape == q.shape
