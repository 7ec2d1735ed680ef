"""Mask bank and per-(timestep, layer) attention.

Calibration compiles one static mask per (timestep, layer, head); at
inference each attention call fetches the kept-block lists or repeat flags of
its (t, l, h) from a table and decides nothing at run time (zhichai.net
article on CalibAtt, §一 and §三 online inference). The bank file, its checks
and the lookup are native (calibatt_bank_* in libcalibatt.so, layout in
include/calibatt.h); this module marshals arguments, keeps the uploaded
lists in one torch-owned device buffer, and exposes the attention as a torch
custom op (calibatt::sparse_attn) and an nn.Module that selects by (t, l).
"""

from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import List, Optional, Sequence, Tuple

import numpy as np
import torch

from . import (BankEntry, BankInfo, Grid, _check, _stream, calibatt_sparse_attn_fwd,
               calibatt_sparse_attn_fwd_workspace, load_library, n_blocks)

_BANK_ALIGN = 256


def _host_i32(a) -> np.ndarray:
    if isinstance(a, torch.Tensor):
        a = a.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def write_bank(path: str, steps: int, layers: int, heads: int, n_tokens: int,
               entry_of: Sequence[Sequence[int]], entries: Sequence[tuple],
               grid: Optional[Tuple[int, int, int, int]] = None) -> None:
    """Write a bank file. entry_of[t][l] is the entry index of (t, l);
    entries[e] = (kv_offsets, kv_indices, repeat_flags or None), host or
    device arrays (copied to the host here). Raises CalibAttError when a
    list is malformed or the file cannot be written."""
    emap = _host_i32(entry_of).reshape(steps, layers)
    offs = [_host_i32(e[0]) for e in entries]
    idxs = [_host_i32(e[1]) for e in entries]
    flags = []
    for e in entries:
        f = e[2] if len(e) > 2 else None
        if isinstance(f, torch.Tensor):
            f = f.detach().cpu().numpy()
        flags.append(None if f is None else np.ascontiguousarray(np.asarray(f, dtype=np.uint8)))
    R = n_blocks(n_tokens)
    for e, (o, f) in enumerate(zip(offs, flags)):
        if o.shape != (heads * R + 1,):
            raise ValueError(f"entry {e}: kv_offsets must have heads*R+1 = {heads * R + 1} entries")
        if f is not None and f.shape != (heads,):
            raise ValueError(f"entry {e}: repeat_flags must have one entry per head")
    n = len(entries)
    P = ctypes.c_void_p
    off_ptrs = (P * n)(*[o.ctypes.data for o in offs])
    idx_ptrs = (P * n)(*[i.ctypes.data if i.size else None for i in idxs])
    flag_ptrs = (P * n)(*[None if f is None else f.ctypes.data for f in flags])
    g = None if grid is None else ctypes.byref(Grid(*[int(x) for x in grid]))
    rc = load_library().calibatt_bank_write(path.encode(), steps, layers, heads, n_tokens, g, n,
                                            emap.ctypes.data_as(P), flag_ptrs, off_ptrs, idx_ptrs)
    _check("calibatt_bank_write", rc)


@dataclass
class BankLookup:
    """One (t, l): the entry index, its kept-block lists (int32 CUDA tensor
    views into the bank's device buffer), repeat flags (host uint8) and the
    bank's grid (None when it has none)."""
    entry: int
    kv_offsets: torch.Tensor
    kv_indices: torch.Tensor
    repeat_flags: np.ndarray
    grid: Optional[Tuple[int, int, int, int]]

    @property
    def any_repeat(self) -> bool:
        return bool(self.repeat_flags.any())


class MaskBank:
    """An opened, checked bank file. With `device` (a CUDA device), its lists
    are uploaded once into a torch-allocated buffer on the current stream and
    `lookup` returns device views; `lookup_host` always works."""

    def __init__(self, path: str, device=None):
        lib = load_library()
        h = ctypes.c_void_p()
        _check("calibatt_bank_open", lib.calibatt_bank_open(path.encode(), ctypes.byref(h)))
        self._h = h
        info = BankInfo()
        _check("calibatt_bank_get_info", lib.calibatt_bank_get_info(self._h, ctypes.byref(info)))
        self.info = info
        g = info.grid
        self.grid = None if (g.frames, g.rows, g.cols, g.anchors) == (0, 0, 0, 0) else \
            (g.frames, g.rows, g.cols, g.anchors)
        self._buf = None
        self._views = {}
        if device is not None:
            self.upload(device)

    @property
    def shape(self) -> Tuple[int, int, int, int]:
        """(steps, layers, heads, n_tokens)."""
        return self.info.steps, self.info.layers, self.info.heads, self.info.n_tokens

    def upload(self, device, stream=None) -> None:
        n = max(int(self.info.device_bytes), 1)
        buf = torch.empty(n + _BANK_ALIGN, dtype=torch.uint8, device=device)
        shift = (-buf.data_ptr()) % _BANK_ALIGN
        buf = buf[shift:shift + n]
        rc = load_library().calibatt_bank_upload(self._h, ctypes.c_void_p(buf.data_ptr()), n,
                                                 _stream(stream, buf))
        _check("calibatt_bank_upload", rc)
        self._buf = buf
        self._views = {}

    def _entry(self, t: int, l: int, on_device: int) -> BankEntry:
        e = BankEntry()
        rc = load_library().calibatt_bank_lookup(self._h, t, l, on_device, ctypes.byref(e))
        _check("calibatt_bank_lookup", rc)
        return e

    def _flags(self, e: BankEntry) -> np.ndarray:
        return np.ctypeslib.as_array((ctypes.c_uint8 * self.info.heads).from_address(e.repeat_flags)).copy()

    def lookup(self, t: int, l: int) -> BankLookup:
        """Device lists of (t, l) (requires upload)."""
        if self._buf is None:
            raise RuntimeError("MaskBank.lookup needs the bank uploaded to a device")
        e = self._entry(t, l, 1)
        hit = self._views.get(e.entry)
        if hit is None:
            base = self._buf.data_ptr()
            H, R = self.info.heads, self.info.n_blocks
            o0 = e.kv_offsets - base
            i0 = e.kv_indices - base
            off = self._buf[o0:o0 + 4 * (H * R + 1)].view(torch.int32)
            idx = self._buf[i0:i0 + 4 * e.nnz].view(torch.int32)
            hit = BankLookup(e.entry, off, idx, self._flags(e), self.grid)
            self._views[e.entry] = hit
        return hit

    def lookup_host(self, t: int, l: int) -> Tuple[int, np.ndarray, np.ndarray, np.ndarray]:
        """(entry, kv_offsets, kv_indices, repeat_flags) of (t, l) as host copies."""
        e = self._entry(t, l, 0)
        H, R = self.info.heads, self.info.n_blocks
        off = np.ctypeslib.as_array((ctypes.c_int32 * (H * R + 1)).from_address(e.kv_offsets)).copy()
        idx = np.zeros(0, np.int32) if e.nnz == 0 else \
            np.ctypeslib.as_array((ctypes.c_int32 * e.nnz).from_address(e.kv_indices)).copy()
        return e.entry, off, idx, self._flags(e)

    def close(self) -> None:
        if getattr(self, "_h", None):
            load_library().calibatt_bank_close(self._h)
            self._h = None

    def __del__(self):
        self.close()


# ----------------------------------------------------------------------------
# torch custom op and module


@torch.library.custom_op("calibatt::sparse_attn", mutates_args=("workspace",))
def sparse_attn(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, kv_offsets: torch.Tensor,
                kv_indices: torch.Tensor, repeat_flags: Optional[torch.Tensor],
                grid: Optional[List[int]], scale: float,
                workspace: Optional[torch.Tensor]) -> torch.Tensor:
    """Block-sparse attention with repeat heads (calibatt_sparse_attn_fwd);
    repeat_flags is a host uint8 tensor [H] or None. workspace: a uint8 CUDA
    tensor of calibatt_sparse_attn_fwd_workspace(H, N) bytes kept by the
    caller across calls (its contents are scratch), or None to have one
    allocated for this call."""
    o = torch.empty_like(q)
    flags = None if repeat_flags is None else repeat_flags.cpu().numpy()
    calibatt_sparse_attn_fwd(q, k, v, o, kv_offsets, kv_indices, scale, flags, grid,
                             workspace=workspace)
    return o


@sparse_attn.register_fake
def _sparse_attn_fake(q, k, v, kv_offsets, kv_indices, repeat_flags, grid, scale, workspace):
    return torch.empty_like(q)


class CalibAttention(torch.nn.Module):
    """Attention of one DiT layer with the calibrated masks of a bank: the
    call for (t, l) fetches that entry's lists and repeat flags (no run-time
    decision) and runs calibatt::sparse_attn. q, k, v: [H][N][128] bf16 on
    the bank's device.

    The module keeps one V^T workspace (calibatt_sparse_attn_fwd_workspace
    bytes: 775 MB for 40 heads at N = 75600) for all its calls, allocated on
    the first call for a given (H, N, device); calls of one module therefore
    must not run concurrently on different streams. `workspace` passes a
    caller-owned buffer instead."""

    def __init__(self, bank: MaskBank, scale: Optional[float] = None,
                 workspace: Optional[torch.Tensor] = None):
        super().__init__()
        self.bank = bank
        self.scale = scale if scale is not None else 128 ** -0.5
        self._flags = {}
        self._ws = workspace
        self._ws_key = None if workspace is None else "caller"

    def _workspace(self, q: torch.Tensor) -> torch.Tensor:
        if self._ws_key == "caller":
            return self._ws
        H, N, _ = q.shape
        key = (H, N, q.device)
        if self._ws_key != key:
            self._ws = torch.empty(max(calibatt_sparse_attn_fwd_workspace(H, N), 16),
                                   dtype=torch.uint8, device=q.device)
            self._ws_key = key
        return self._ws

    def forward(self, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, t: int, l: int) -> torch.Tensor:
        e = self.bank.lookup(t, l)
        flags = None
        if e.any_repeat:
            flags = self._flags.get(e.entry)
            if flags is None:
                flags = self._flags[e.entry] = torch.from_numpy(e.repeat_flags.copy())
        grid = list(e.grid) if (e.any_repeat and e.grid is not None) else None
        return torch.ops.calibatt.sparse_attn(q, k, v, e.kv_offsets, e.kv_indices, flags, grid,
                                              float(self.scale), self._workspace(q))
