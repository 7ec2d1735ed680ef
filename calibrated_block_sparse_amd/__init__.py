"""Python binding of libcalibatt.so (calibrated block-sparse attention for
MI355X / gfx950).

Argument marshalling only: every step runs in the library's HIP kernels.
torch supplies device memory and the current stream. The functions keep
the C names of include/calibatt.h; each raises CalibAttError with the
library's message when the call fails, and load_library() raises when the
shared library has not been built (python -m calibrated_block_sparse_amd.build).
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np
import torch

BLOCK = 128
HEAD_DIM = 128
MAX_BLOCKS = 2047
NOALLOC_SCRATCH_BYTES = 268435456   # CALIBATT_NOALLOC_SCRATCH_BYTES

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libcalibatt.so")

# Every symbol include/calibatt.h declares, with its ctypes signature.
_c = ctypes
_p = _c.c_void_p
SIGNATURES = {
    "calibatt_last_error": (_c.c_char_p, []),
    "calibatt_abi_version": (_c.c_int32, []),
    "calibatt_sparse_attn_fwd": (_c.c_int, [_p, _p, _p, _p, _c.c_int32, _c.c_int32, _c.c_int32,
                                            _c.c_int64, _c.c_int64, _c.c_float, _p, _p,
                                            _c.c_int64, _p, _p, _p, _c.c_size_t, _p]),
    "calibatt_sparse_attn_fwd_workspace": (_c.c_size_t, [_c.c_int32, _c.c_int32]),
    "calibatt_prepare_vt": (_c.c_int, [_p, _c.c_int32, _c.c_int32, _c.c_int32, _c.c_int64,
                                       _c.c_int64, _p, _c.c_size_t, _p]),
    "calibatt_sparse_attn_fwd_vt": (_c.c_int, [_p, _p, _p, _p, _c.c_int32, _c.c_int32,
                                               _c.c_int32, _c.c_int64, _c.c_int64, _c.c_float,
                                               _p, _p, _c.c_int64, _p, _p, _c.c_size_t, _p]),
    "calibatt_sparse_attn_fwd_noalloc": (_c.c_int, [_p, _p, _p, _p, _c.c_int32, _c.c_int32,
                                                    _c.c_int32, _c.c_int64, _c.c_int64, _c.c_float,
                                                    _p, _p, _c.c_int64, _p, _p, _p]),
    "calibatt_block_energy_workspace": (_c.c_size_t, [_c.c_int32, _c.c_int32]),
    "calibatt_block_energy": (_c.c_int, [_p, _p, _p, _c.c_int32, _c.c_int32, _c.c_int32,
                                         _c.c_int64, _c.c_int64, _c.c_float, _p, _c.c_size_t, _p]),
    "calibatt_spatial_similarity": (_c.c_int, [_p, _c.c_size_t, _c.c_int32, _c.c_int32, _p, _p,
                                                _p, _p]),
    "calibatt_eps_fx": (_c.c_uint64, [_c.c_double] * 5),
    "calibatt_build_mask": (_c.c_int, [_p, _c.c_int32, _c.c_int32, _c.c_int32, _c.c_uint64, _p,
                                       _p, _p]),
    "calibatt_finalize_mask": (_c.c_int, [_p, _c.c_int32, _c.c_int32, _c.c_int32, _c.c_int32,
                                          _c.c_int32, _p, _p, _p, _p, _p]),
    "calibatt_compile_skiplist": (_c.c_int, [_p, _c.c_int32, _c.c_int32, _p, _p, _p, _p]),
    "calibatt_validate_skiplist": (_c.c_int, [_p, _p, _c.c_int64, _c.c_int32, _c.c_int32]),
    "calibatt_bank_write": (_c.c_int, [_c.c_char_p, _c.c_int32, _c.c_int32, _c.c_int32, _c.c_int32,
                                       _p, _c.c_int32, _p, _p, _p, _p]),
    "calibatt_bank_open": (_c.c_int, [_c.c_char_p, _p]),
    "calibatt_bank_close": (None, [_p]),
    "calibatt_bank_get_info": (_c.c_int, [_p, _p]),
    "calibatt_bank_upload": (_c.c_int, [_p, _p, _c.c_size_t, _p]),
    "calibatt_bank_lookup": (_c.c_int, [_p, _c.c_int32, _c.c_int32, _c.c_int32, _p]),
    "calibatt_mfma_rate_probe": (_c.c_int, [_p, _c.c_int64, _c.c_int32, _p]),
}

STATUS = {0: "OK", -1: "INVALID_ARG", -2: "UNSUPPORTED", -3: "BAD_SKIPLIST", -4: "WORKSPACE",
          -5: "HIP", -6: "IO"}


class CalibAttError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn} failed ({STATUS.get(code, code)}): {msg}")
        self.code = code


class Grid(ctypes.Structure):
    """calibatt_grid: token n = f*rows*cols + y*cols + x; `anchors` rows per
    frame are computed by repeat heads."""
    _fields_ = [("frames", ctypes.c_int32), ("rows", ctypes.c_int32),
                ("cols", ctypes.c_int32), ("anchors", ctypes.c_int32)]


class BankInfo(ctypes.Structure):
    """calibatt_bank_info."""
    _fields_ = [("steps", ctypes.c_int32), ("layers", ctypes.c_int32), ("heads", ctypes.c_int32),
                ("n_tokens", ctypes.c_int32), ("n_blocks", ctypes.c_int32),
                ("n_entries", ctypes.c_int32), ("grid", Grid), ("total_nnz", ctypes.c_int64),
                ("device_bytes", ctypes.c_size_t)]


class BankEntry(ctypes.Structure):
    """calibatt_bank_entry."""
    _fields_ = [("entry", ctypes.c_int32), ("repeat_flags", ctypes.c_void_p),
                ("kv_offsets", ctypes.c_void_p), ("kv_indices", ctypes.c_void_p),
                ("nnz", ctypes.c_int64)]


_lib = None


def load_library(path: Optional[str] = None):
    """Loads libcalibatt.so once; raises if it is missing or lacks a symbol.
    The environment variable CALIBATT_LIB names another build of the library
    to load instead (for example the host-sanitized libcalibatt_asan.so)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or os.environ.get("CALIBATT_LIB") or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} not found: build it with `python -m calibrated_block_sparse_amd.build`")
    lib = ctypes.CDLL(p)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib


def _check(fn: str, rc: int):
    if rc != 0:
        raise CalibAttError(fn, rc, load_library().calibatt_last_error().decode())


def _launch_stream(stream, *tensors) -> "torch.cuda.Stream":
    """The torch stream to launch on: `stream`, or the current stream of the
    device the tensors live on. Every CUDA tensor given must live on that
    device (the library launches on the stream's device and would otherwise
    be handed another device's memory)."""
    devs = {t.device for t in tensors if isinstance(t, torch.Tensor)}
    for t in tensors:
        if isinstance(t, torch.Tensor) and not t.is_cuda:
            raise ValueError(f"expected CUDA tensors, got one on {t.device}")
    if len(devs) > 1:
        raise ValueError(f"tensors on different devices: {sorted(str(d) for d in devs)}")
    dev = next(iter(devs)) if devs else None
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    elif dev is not None and stream.device != dev:
        raise ValueError(f"stream on {stream.device}, tensors on {dev}")
    return stream


def _stream(stream, *tensors) -> ctypes.c_void_p:
    """The stream handle to launch on (see _launch_stream)."""
    return ctypes.c_void_p(_launch_stream(stream, *tensors).cuda_stream)


def _empty_on(stream, *shape, dtype, device) -> torch.Tensor:
    """torch.empty allocated on `stream` (a torch stream): the caching
    allocator then hands the memory to another allocation only after the
    work enqueued on that stream, so a scratch buffer freed when the binding
    returns stays valid for the kernels still running on it."""
    with torch.cuda.stream(stream):
        return torch.empty(*shape, dtype=dtype, device=device)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def n_blocks(n_tokens: int) -> int:
    return (n_tokens + BLOCK - 1) // BLOCK


def _attn_layout(name: str, *ts: torch.Tensor):
    """[heads][N][128] bf16 CUDA tensors sharing one stride pattern."""
    t0 = ts[0]
    for t in ts:
        if t.dtype != torch.bfloat16 or not t.is_cuda or t.dim() != 3:
            raise ValueError(f"{name}: expected 3-d bf16 CUDA tensors [heads][N][128]")
        if t.shape != t0.shape or t.stride() != t0.stride():
            raise ValueError(f"{name}: q/k/v/o must share shape and strides")
        if t.stride(2) != 1:
            raise ValueError(f"{name}: the head dimension must be contiguous")
    H, N, D = t0.shape
    return H, N, D, t0.stride(0), t0.stride(1)


def calibatt_last_error() -> str:
    return load_library().calibatt_last_error().decode()


def calibatt_abi_version() -> int:
    return int(load_library().calibatt_abi_version())


def calibatt_sparse_attn_fwd_workspace(heads: int, n_tokens: int) -> int:
    return int(load_library().calibatt_sparse_attn_fwd_workspace(heads, n_tokens))


def calibatt_sparse_attn_fwd(q, k, v, o, kv_offsets, kv_indices, scale: float,
                             repeat_flags=None, grid=None, stream=None, workspace=None) -> None:
    """o <- block-sparse attention of q, k, v over the kept-block lists
    (kv_offsets int32 [H*R+1], kv_indices int32 [nnz], CUDA tensors).
    repeat_flags: host sequence of H ints (or None); grid: (frames, rows,
    cols, anchors) for repeat heads. workspace: uint8 CUDA tensor of
    calibatt_sparse_attn_fwd_workspace bytes (allocated here through torch
    when None)."""
    H, N, D, sh, stok = _attn_layout("calibatt_sparse_attn_fwd", q, k, v, o)
    nnz = _check_lists(H, N, kv_offsets, kv_indices)
    flags, g = _flags_grid(H, repeat_flags, grid)
    lib = load_library()
    st = _launch_stream(stream, q, k, v, o, kv_offsets, kv_indices, workspace)
    if workspace is None:
        need = calibatt_sparse_attn_fwd_workspace(H, N)
        workspace = _empty_on(st, max(need, 16), dtype=torch.uint8, device=q.device)
    rc = lib.calibatt_sparse_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), H, N, D, sh, stok,
                                      float(scale), _ptr(kv_offsets), _ptr(kv_indices), nnz,
                                      None if flags is None else flags.ctypes.data_as(ctypes.c_void_p),
                                      None if g is None else ctypes.byref(g), _ptr(workspace),
                                      workspace.numel() * workspace.element_size(),
                                      ctypes.c_void_p(st.cuda_stream))
    _check("calibatt_sparse_attn_fwd", rc)


def _check_lists(H: int, N: int, kv_offsets, kv_indices) -> int:
    """Kept-block lists as the kernels read them: contiguous int32 CUDA
    tensors, kv_offsets with at least H*R+1 entries. Returns nnz (the
    length of kv_indices). Either may be None (the library then requires
    every head to be a plain repeat head)."""
    for t in (kv_offsets, kv_indices):
        if t is not None and (t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous()):
            raise ValueError("kept-block lists must be contiguous int32 CUDA tensors")
    if kv_offsets is not None and kv_offsets.numel() < H * n_blocks(N) + 1:
        raise ValueError(f"kv_offsets needs H*R+1 = {H * n_blocks(N) + 1} entries, "
                         f"has {kv_offsets.numel()}")
    return 0 if kv_indices is None else kv_indices.numel()


def _flags_grid(H, repeat_flags, grid):
    flags = None
    if repeat_flags is not None:
        arr = np.ascontiguousarray(np.asarray(repeat_flags, dtype=np.uint8))
        if arr.shape != (H,):
            raise ValueError("repeat_flags must have one entry per head")
        flags = arr
    g = None if grid is None else Grid(*[int(x) for x in grid])
    return flags, g


def calibatt_prepare_vt(v, workspace, stream=None) -> None:
    """workspace (uint8 CUDA, calibatt_sparse_attn_fwd_workspace bytes) <- the
    V^T tiles of v ([H][N][128] bf16 CUDA)."""
    H, N, D, sh, stok = _attn_layout("calibatt_prepare_vt", v)
    rc = load_library().calibatt_prepare_vt(_ptr(v), H, N, D, sh, stok, _ptr(workspace),
                                            workspace.numel() * workspace.element_size(),
                                            _stream(stream, v, workspace))
    _check("calibatt_prepare_vt", rc)


def calibatt_sparse_attn_fwd_vt(q, k, vt, o, kv_offsets, kv_indices, scale: float,
                                repeat_flags=None, grid=None, stream=None) -> None:
    """o <- block-sparse attention of q, k and the V^T tiles in vt (filled by
    calibatt_prepare_vt); otherwise as calibatt_sparse_attn_fwd."""
    H, N, D, sh, stok = _attn_layout("calibatt_sparse_attn_fwd_vt", q, k, o)
    nnz = _check_lists(H, N, kv_offsets, kv_indices)
    flags, g = _flags_grid(H, repeat_flags, grid)
    rc = load_library().calibatt_sparse_attn_fwd_vt(
        _ptr(q), _ptr(k), _ptr(vt), _ptr(o), H, N, D, sh, stok, float(scale), _ptr(kv_offsets),
        _ptr(kv_indices), nnz, None if flags is None else flags.ctypes.data_as(ctypes.c_void_p),
        None if g is None else ctypes.byref(g), vt.numel() * vt.element_size(),
        _stream(stream, q, k, vt, o, kv_offsets, kv_indices))
    _check("calibatt_sparse_attn_fwd_vt", rc)


def calibatt_sparse_attn_fwd_noalloc(q, k, v, o, kv_offsets, kv_indices, scale: float,
                                     repeat_flags=None, grid=None, stream=None) -> None:
    """As calibatt_sparse_attn_fwd, with the V^T tiles in the library's own
    device scratch instead of a workspace (nothing is allocated; calls that
    overlap on one device race)."""
    H, N, D, sh, stok = _attn_layout("calibatt_sparse_attn_fwd_noalloc", q, k, v, o)
    nnz = _check_lists(H, N, kv_offsets, kv_indices)
    flags, g = _flags_grid(H, repeat_flags, grid)
    rc = load_library().calibatt_sparse_attn_fwd_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), H, N, D, sh, stok, float(scale), _ptr(kv_offsets),
        _ptr(kv_indices), nnz, None if flags is None else flags.ctypes.data_as(ctypes.c_void_p),
        None if g is None else ctypes.byref(g), _stream(stream, q, k, v, o, kv_offsets, kv_indices))
    _check("calibatt_sparse_attn_fwd_noalloc", rc)


def calibatt_block_energy_workspace(heads: int, n_tokens: int) -> int:
    return int(load_library().calibatt_block_energy_workspace(heads, n_tokens))


ENERGY_WORKSPACE_CAP = 2 << 30   # bytes the binding allocates at most (heads then go in chunks)


def calibatt_block_energy(q, k, energy, scale: float, workspace=None, stream=None) -> None:
    """energy (fp32 CUDA [H][R][R]) <- block energies of softmax(scale q k^T).
    workspace: uint8 CUDA tensor of at least calibatt_block_energy_workspace(1,
    N) bytes (heads are processed in chunks of as many as it holds); when
    None, one of min(all heads, max(one head, 2 GiB)) is allocated here
    through torch."""
    H, N, D, sh, stok = _attn_layout("calibatt_block_energy", q, k)
    R = n_blocks(N)
    if energy.dtype != torch.float32 or not energy.is_contiguous() or energy.shape != (H, R, R):
        raise ValueError("energy must be a contiguous fp32 tensor [H][R][R]")
    need = calibatt_block_energy_workspace(H, N)
    st = _launch_stream(stream, q, k, energy, workspace)
    if workspace is None:
        size = min(need, max(calibatt_block_energy_workspace(1, N), ENERGY_WORKSPACE_CAP))
        workspace = _empty_on(st, max(size, 1), dtype=torch.uint8, device=q.device)
    rc = load_library().calibatt_block_energy(_ptr(q), _ptr(k), _ptr(energy), H, N, D, sh, stok,
                                              float(scale), _ptr(workspace),
                                              workspace.numel() * workspace.element_size(),
                                              ctypes.c_void_p(st.cuda_stream))
    _check("calibatt_block_energy", rc)


def calibatt_spatial_similarity(energy_workspace, heads: int, n_tokens: int, grid, row_profiles,
                                similarity, stream=None) -> None:
    """row_profiles ([H][frames*rows][R] fp32 CUDA) and similarity ([H] fp32
    CUDA) from the workspace of a preceding calibatt_block_energy call on the
    same stream; grid = (frames, rows, cols, anchors)."""
    for t in (row_profiles, similarity):
        if t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous():
            raise ValueError("row_profiles and similarity must be contiguous float32 CUDA tensors")
    R = n_blocks(n_tokens)
    if row_profiles.numel() < heads * grid[0] * grid[1] * R or similarity.numel() < heads:
        raise ValueError("row_profiles needs heads*frames*rows*R and similarity heads elements")
    g = Grid(*[int(x) for x in grid])
    rc = load_library().calibatt_spatial_similarity(
        _ptr(energy_workspace), energy_workspace.numel() * energy_workspace.element_size(), heads,
        n_tokens, ctypes.byref(g), _ptr(row_profiles), _ptr(similarity),
        _stream(stream, energy_workspace, row_profiles, similarity))
    _check("calibatt_spatial_similarity", rc)


def calibatt_eps_fx(t: float, T: float, A: float, C: float, k: float) -> int:
    return int(load_library().calibatt_eps_fx(float(t), float(T), float(A), float(C), float(k)))


def calibatt_build_mask(energy, eps_fx: int, votes, n_sel=None, stream=None) -> None:
    """votes (uint8 [H][R][R]) += greedy selections at eps_fx of every draw in
    energy (fp32 [n_draws][H][R][R] or [H][R][R]); n_sel (int32
    [n_draws][H][R]) receives the selected counts when given."""
    e = energy if energy.dim() == 4 else energy.unsqueeze(0)
    D_, H, R, R2 = e.shape
    if e.dtype != torch.float32 or not e.is_contiguous() or R != R2:
        raise ValueError("energy must be contiguous fp32 [n_draws][H][R][R]")
    if votes.dtype != torch.uint8 or votes.shape != (H, R, R) or not votes.is_contiguous():
        raise ValueError("votes must be contiguous uint8 [H][R][R]")
    if n_sel is not None and (n_sel.dtype != torch.int32 or n_sel.numel() != D_ * H * R):
        raise ValueError("n_sel must be int32 with n_draws*H*R entries")
    rc = load_library().calibatt_build_mask(_ptr(e), D_, H, R, int(eps_fx), _ptr(votes),
                                            _ptr(n_sel), _stream(stream, e, votes, n_sel))
    _check("calibatt_build_mask", rc)


def calibatt_finalize_mask(votes, n_prompts: int, rho_num: int, rho_den: int, mask,
                           kv_offsets, kv_indices, stream=None) -> int:
    """Binarise votes at rho = rho_num/rho_den into mask and compile the
    kept-block lists; returns nnz (waits for the stream)."""
    if votes.dtype != torch.uint8 or votes.dim() != 3 or votes.shape[1] != votes.shape[2] or \
            not votes.is_contiguous():
        raise ValueError("votes must be contiguous uint8 [H][R][R]")
    H, R, _ = votes.shape
    if mask.dtype != torch.uint8 or mask.shape != votes.shape or not mask.is_contiguous():
        raise ValueError("mask must be contiguous uint8 with the shape of votes")
    for t in (kv_offsets, kv_indices):
        if t.dtype != torch.int32 or not t.is_contiguous():
            raise ValueError("kv_offsets and kv_indices must be contiguous int32 tensors")
    if kv_offsets.numel() < H * R + 1 or kv_indices.numel() < H * R * R:
        raise ValueError("kv_offsets needs H*R+1 entries and kv_indices H*R*R")
    nnz = ctypes.c_int64(0)
    rc = load_library().calibatt_finalize_mask(_ptr(votes), H, R, int(n_prompts), int(rho_num),
                                               int(rho_den), _ptr(mask), _ptr(kv_offsets),
                                               _ptr(kv_indices), ctypes.byref(nnz),
                                               _stream(stream, votes, mask, kv_offsets, kv_indices))
    _check("calibatt_finalize_mask", rc)
    return int(nnz.value)


def calibatt_compile_skiplist(mask, kv_offsets, kv_indices, stream=None) -> int:
    """Compile a uint8 [H][R][R] block mask into kept-block lists; returns
    nnz (waits for the stream)."""
    H, R, R2 = mask.shape
    if mask.dtype != torch.uint8 or R != R2 or not mask.is_contiguous():
        raise ValueError("mask must be contiguous uint8 [H][R][R]")
    for t in (kv_offsets, kv_indices):
        if t.dtype != torch.int32 or not t.is_contiguous():
            raise ValueError("kv_offsets and kv_indices must be contiguous int32 tensors")
    if kv_offsets.numel() < H * R + 1 or kv_indices.numel() < H * R * R:
        raise ValueError("kv_offsets needs H*R+1 entries and kv_indices H*R*R")
    nnz = ctypes.c_int64(0)
    rc = load_library().calibatt_compile_skiplist(_ptr(mask), H, R, _ptr(kv_offsets),
                                                  _ptr(kv_indices), ctypes.byref(nnz),
                                                  _stream(stream, mask, kv_offsets, kv_indices))
    _check("calibatt_compile_skiplist", rc)
    return int(nnz.value)


def calibatt_validate_skiplist(kv_offsets, kv_indices, heads: int, n_blocks_: int) -> None:
    """Host-side check of a kept-block list (numpy int32 arrays or CPU
    tensors); raises CalibAttError(BAD_SKIPLIST) on the first defect."""
    off = np.ascontiguousarray(np.asarray(kv_offsets, dtype=np.int32))
    idx = np.ascontiguousarray(np.asarray(kv_indices, dtype=np.int32))
    if off.size != heads * n_blocks_ + 1:
        raise ValueError("kv_offsets must have heads*R+1 entries")
    rc = load_library().calibatt_validate_skiplist(off.ctypes.data_as(ctypes.c_void_p),
                                                   idx.ctypes.data_as(ctypes.c_void_p),
                                                   idx.size, heads, n_blocks_)
    _check("calibatt_validate_skiplist", rc)


def calibatt_mfma_rate_probe(sink, iters: int, workgroups: int, stream=None) -> int:
    """Enqueue the matrix-core rate probe; returns the FLOP it performs
    (workgroups * 4 waves * iters * 8 MFMAs * 32768)."""
    if sink.dtype != torch.float32 or not sink.is_cuda or sink.numel() < 1:
        raise ValueError("sink must be a CUDA float32 tensor with at least one element")
    rc = load_library().calibatt_mfma_rate_probe(_ptr(sink), iters, workgroups, _stream(stream, sink))
    _check("calibatt_mfma_rate_probe", rc)
    return int(workgroups) * 4 * int(iters) * 8 * 32768


# ----------------------------------------------------------------------------
# Allocating conveniences (torch allocations + the calls above)


# Results and scratch buffers are allocated on the stream the work is
# enqueued on (the current stream unless `stream` is given).


def compile_skiplist(mask: torch.Tensor, stream=None):
    """(kv_offsets, kv_indices[:nnz]) on mask's device."""
    H, R, _ = mask.shape
    st = _launch_stream(stream, mask)
    off = _empty_on(st, H * R + 1, dtype=torch.int32, device=mask.device)
    idx = _empty_on(st, max(H * R * R, 1), dtype=torch.int32, device=mask.device)
    nnz = calibatt_compile_skiplist(mask, off, idx, st)
    return off, idx[:nnz]


def sparse_attention(q, k, v, kv_offsets, kv_indices, scale: float, repeat_flags=None,
                     grid=None, stream=None) -> torch.Tensor:
    st = _launch_stream(stream, q)
    with torch.cuda.stream(st):
        o = torch.empty_like(q)
    calibatt_sparse_attn_fwd(q, k, v, o, kv_offsets, kv_indices, scale, repeat_flags, grid, st)
    return o


def energy_and_similarity(q, k, scale: float, grid, stream=None):
    """One Q K^T pass: (energy [H][R][R], similarity [H], row profiles
    [H][frames*rows][R]) of q, k for grid (frames, rows, cols, anchors)."""
    H, N, _ = q.shape
    R = n_blocks(N)
    st = _launch_stream(stream, q, k)
    e = _empty_on(st, H, R, R, dtype=torch.float32, device=q.device)
    ws = _empty_on(st, max(calibatt_block_energy_workspace(H, N), 8), dtype=torch.uint8,
                   device=q.device)
    calibatt_block_energy(q, k, e, scale, ws, st)
    prof = _empty_on(st, H, grid[0] * grid[1], R, dtype=torch.float32, device=q.device)
    sim = _empty_on(st, H, dtype=torch.float32, device=q.device)
    calibatt_spatial_similarity(ws, H, N, grid, prof, sim, st)
    return e, sim, prof


def block_energy(q, k, scale: float, stream=None) -> torch.Tensor:
    H, N, _ = q.shape
    R = n_blocks(N)
    st = _launch_stream(stream, q, k)
    e = _empty_on(st, H, R, R, dtype=torch.float32, device=q.device)
    calibatt_block_energy(q, k, e, scale, None, st)
    return e
