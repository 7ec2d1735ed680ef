"""Seeded synthetic workloads shaped like the pages' video models.

The pages measure CalibAtt inside Wan 2.1 14B (480p, 720p) and Mochi 1
(480p) generations over 64 calibration prompts ("Accelerating Text-to-Video
Generation with Calibrated Sparse Attention", zhichai.net summary, sections
三 and 四). None of those weights, prompts or videos exist here; the
generators below stand in for them with tensors of the same shapes, block
sparsities taken from the results table (section 四), and a frame-major,
row-major video token layout (section 六).

Everything here is random-number drawing and layout. Nothing computes
attention, energies, selections or skip lists.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional, Tuple

import numpy as np
import torch

BLOCK = 128
HEAD_DIM = 128

__all__ = [
    "BLOCK", "HEAD_DIM", "VideoGrid", "AttnWorkload", "CalibWorkload",
    "ATTN_WORKLOADS", "CALIB_WORKLOADS", "n_blocks", "bf16_bits",
    "gaussian_bf16", "qkv", "block_mask", "band_random_mask",
    "bernoulli_mask", "repeat_flags", "energy_rows", "calib_draw",
    "calib_basis", "mask_for_fraction",
]


def n_blocks(n_tokens: int) -> int:
    """Number of 128-token blocks covering n_tokens (the last may be ragged)."""
    return (n_tokens + BLOCK - 1) // BLOCK


@dataclasses.dataclass(frozen=True)
class VideoGrid:
    """Latent video grid: token n = f*rows*cols + y*cols + x (frame-major,
    row-major inside a frame)."""
    frames: int
    rows: int
    cols: int

    @property
    def n_tokens(self) -> int:
        return self.frames * self.rows * self.cols


@dataclasses.dataclass(frozen=True)
class AttnWorkload:
    name: str
    heads: int
    n_tokens: int
    grid: Optional[VideoGrid]
    sparsity: Optional[float]          # fraction of skipped blocks per head
    seeds: Tuple[int, int, int]        # q, k, v
    mask_seed: int                     # per-head mask seed = mask_seed + h
    repeat_every: int = 0              # heads with h % repeat_every == repeat_every-1 repeat
    anchors: int = 5
    head_dim: int = HEAD_DIM

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def n_blocks(self) -> int:
        return n_blocks(self.n_tokens)

    def keep_per_head(self) -> int:
        R = self.n_blocks
        return int(round((1.0 - self.sparsity) * R * R))


ATTN_WORKLOADS = {
    # One head, N=1024 (8x8 blocks), Bernoulli(0.5) block mask, diagonal kept.
    "single_head_1k": AttnWorkload("single_head_1k", 1, 1024, None, None,
                                   (11, 12, 13), 14),
    # Wan 2.1 14B self-attention layer at 480p: 21 frames x 30x52 latent grid.
    "wan21_480p_layer": AttnWorkload("wan21_480p_layer", 40, 32760,
                                     VideoGrid(21, 30, 52), 0.68,
                                     (21, 22, 23), 200),
    # Wan 2.1 14B self-attention layer at 720p: 21 frames x 45x80 grid.
    "wan21_720p_layer": AttnWorkload("wan21_720p_layer", 40, 75600,
                                     VideoGrid(21, 45, 80), 0.625,
                                     (31, 32, 33), 300),
    # Mochi 1 layer at 480p: 28 frames x 30x53 grid; every 4th head repeats.
    "mochi1_480p_layer": AttnWorkload("mochi1_480p_layer", 24, 44520,
                                      VideoGrid(28, 30, 53), 0.691,
                                      (41, 42, 43), 400, repeat_every=4),
}


@dataclasses.dataclass(frozen=True)
class CalibWorkload:
    name: str
    heads: int
    grid: VideoGrid
    draws: int
    draw_seed: int        # draw p uses draw_seed + p
    basis_seed: int       # shared positional code
    proj_seed: int        # per-head projections of the code
    alpha: float          # strength of the shared low-rank component
    steps: Tuple[int, ...]
    total_steps: int
    eps_floor: float      # A: late-step threshold
    eps_start: float      # C: first-step threshold
    eps_rate: float       # k: decay rate
    rho: Tuple[int, int]  # binarisation threshold as num/den
    rank: int = 16
    head_dim: int = HEAD_DIM

    @property
    def n_tokens(self) -> int:
        return self.grid.n_tokens

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


CALIB_WORKLOADS = {
    "calibration_480p": CalibWorkload(
        "calibration_480p", 40, VideoGrid(21, 30, 52), 64,
        5000, 4999, 4998, alpha=1.5, steps=(0, 25, 49), total_steps=50,
        eps_floor=0.84, eps_start=0.99, eps_rate=5.0, rho=(1, 2)),
    # Same recipe at a size a CPU finishes in seconds.
    "calibration_small": CalibWorkload(
        "calibration_small", 2, VideoGrid(4, 8, 24), 8,
        6000, 5999, 5998, alpha=1.5, steps=(0, 25, 49), total_steps=50,
        eps_floor=0.84, eps_start=0.99, eps_rate=5.0, rho=(1, 2)),
}


# ----------------------------------------------------------------------------
# bf16 helpers (storage only)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Raw bf16 bit patterns of a torch bf16 tensor as a numpy uint16 array."""
    assert t.dtype == torch.bfloat16
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def _generator(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def gaussian_bf16(seed: int, shape, device="cpu", std: float = 1.0) -> torch.Tensor:
    """N(0, std^2) samples drawn in fp32 from a seeded torch generator on
    `device`, rounded to bf16 (round-to-nearest-even). CPU and GPU generators
    give different streams for one seed; every caller hands the same tensor to
    both sides of a comparison."""
    g = _generator(seed, device)
    x = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(torch.bfloat16)


def qkv(w: AttnWorkload, device="cpu", heads: Optional[int] = None):
    """Q, K, V as contiguous bf16 [heads][N][D] tensors."""
    H = w.heads if heads is None else heads
    shape = (H, w.n_tokens, w.head_dim)
    return tuple(gaussian_bf16(s, shape, device) for s in w.seeds)


# ----------------------------------------------------------------------------
# Block masks (input structure: which 128x128 blocks a head keeps)


def bernoulli_mask(seed: int, heads: int, R: int, keep: float = 0.5,
                   diagonal: bool = True) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed))
    m = (rng.random((heads, R, R)) < keep).astype(np.uint8)
    if diagonal:
        idx = np.arange(R)
        m[:, idx, idx] = 1
    return m


def _frame_band(grid: VideoGrid, n_tokens: int, width: int) -> np.ndarray:
    """Blocks whose token spans come within `width` frames of each other."""
    R = n_blocks(n_tokens)
    ft = grid.rows * grid.cols
    t0 = np.arange(R, dtype=np.int64) * BLOCK
    t1 = np.minimum(t0 + BLOCK, n_tokens) - 1
    f0, f1 = t0 // ft, t1 // ft
    gap = np.maximum(0, np.maximum(f0[None, :] - f1[:, None],
                                   f0[:, None] - f1[None, :]))
    return gap <= width


def band_random_mask(grid: VideoGrid, n_tokens: int, heads: int,
                     keep_per_head: int, seed0: int,
                     band_width: int = 2) -> np.ndarray:
    """Per-head mask: the frame band |frame distance| <= band_width (which
    holds the diagonal), plus blocks drawn uniformly without replacement from
    outside the band until exactly keep_per_head blocks are kept. Head h uses
    seed seed0 + h."""
    R = n_blocks(n_tokens)
    band = _frame_band(grid, n_tokens, band_width)
    nb = int(band.sum())
    if keep_per_head < nb:
        raise ValueError(f"band alone keeps {nb} > {keep_per_head} blocks")
    outside = np.flatnonzero(~band.ravel())
    out = np.empty((heads, R, R), dtype=np.uint8)
    for h in range(heads):
        rng = np.random.Generator(np.random.PCG64(seed0 + h))
        pick = rng.choice(outside.size, size=keep_per_head - nb, replace=False)
        m = band.ravel().astype(np.uint8)
        m[outside[pick]] = 1
        out[h] = m.reshape(R, R)
    return out


def block_mask(w: AttnWorkload, heads: Optional[int] = None) -> np.ndarray:
    """The workload's uint8 [heads][R][R] block mask (1 = keep)."""
    H = w.heads if heads is None else heads
    if w.grid is None:
        return bernoulli_mask(w.mask_seed, H, w.n_blocks, 0.5, True)
    return band_random_mask(w.grid, w.n_tokens, H, w.keep_per_head(), w.mask_seed)


def mask_for_fraction(w: AttnWorkload, keep_fraction: float,
                      heads: Optional[int] = None, seed_offset: int = 0) -> np.ndarray:
    """Band + random mask of the workload's grid at another kept fraction
    (1.0 keeps everything). Used for the kept-fraction sweep."""
    H = w.heads if heads is None else heads
    R = w.n_blocks
    if keep_fraction >= 1.0:
        return np.ones((H, R, R), dtype=np.uint8)
    keep = int(round(keep_fraction * R * R))
    band = _frame_band(w.grid, w.n_tokens, 2)
    if keep < int(band.sum()):
        # Thinner band: keep the diagonal and draw the rest at random.
        out = np.zeros((H, R, R), dtype=np.uint8)
        idx = np.arange(R)
        for h in range(H):
            rng = np.random.Generator(np.random.PCG64(w.mask_seed + seed_offset + h))
            m = np.zeros((R, R), dtype=np.uint8)
            m[idx, idx] = 1
            off = np.flatnonzero(m.ravel() == 0)
            pick = rng.choice(off.size, size=keep - R, replace=False)
            m.ravel()[off[pick]] = 1
            out[h] = m
        return out
    return band_random_mask(w.grid, w.n_tokens, H, keep, w.mask_seed + seed_offset)


def repeat_flags(w: AttnWorkload, heads: Optional[int] = None) -> np.ndarray:
    H = w.heads if heads is None else heads
    f = np.zeros(H, dtype=np.uint8)
    if w.repeat_every:
        f[np.arange(H) % w.repeat_every == w.repeat_every - 1] = 1
    return f


# ----------------------------------------------------------------------------
# Energy-like rows for exercising selection on its own


def energy_rows(seed: int, heads: int, R: int, kind: str = "dirichlet") -> np.ndarray:
    """fp32 [heads][R][R] non-negative rows that sum to about one.

    kind: "dirichlet" (smooth random rows), "peaky" (a few large entries),
    "ties" (values drawn from a handful of levels so equal entries are
    common), "uniform" (every entry of a row equal), "onehot".
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    if kind == "dirichlet":
        x = rng.gamma(1.0, size=(heads, R, R))
    elif kind == "peaky":
        x = rng.gamma(0.1, size=(heads, R, R))
    elif kind == "ties":
        x = rng.integers(0, 4, size=(heads, R, R)).astype(np.float64)
        x[..., 0] += 1.0
    elif kind == "uniform":
        x = np.ones((heads, R, R))
    elif kind == "onehot":
        x = np.zeros((heads, R, R))
        cols = rng.integers(0, R, size=(heads, R))
        np.put_along_axis(x, cols[..., None], 1.0, axis=-1)
    else:
        raise ValueError(kind)
    x = x / x.sum(axis=-1, keepdims=True)
    return x.astype(np.float32)


# ----------------------------------------------------------------------------
# Calibration draws: per-prompt Q/K with a shared positional structure


def calib_basis(w: CalibWorkload, device="cpu"):
    """Shared positional code Phi [N][rank] (frame + row + column codebooks,
    each N(0, 1/16)) and per-head projections Wq, Wk [heads][rank][D]."""
    g = w.grid
    gen = _generator(w.basis_seed, "cpu")
    fc = torch.randn(g.frames, w.rank, generator=gen) / 4
    rc = torch.randn(g.rows, w.rank, generator=gen) / 4
    cc = torch.randn(g.cols, w.rank, generator=gen) / 4
    phi = (fc[:, None, None, :] + rc[None, :, None, :] + cc[None, None, :, :])
    phi = phi.reshape(g.n_tokens, w.rank)
    gp = _generator(w.proj_seed, "cpu")
    wq = torch.randn(w.heads, w.rank, w.head_dim, generator=gp)
    wk = torch.randn(w.heads, w.rank, w.head_dim, generator=gp)
    return phi.to(device), wq.to(device), wk.to(device)


def calib_draw(w: CalibWorkload, p: int, basis=None, device="cpu",
               heads: Optional[int] = None):
    """Prompt draw p: Q = Z + alpha*Phi Wq_h, K = Z' + alpha*Phi Wk_h as bf16
    [heads][N][D], with Z, Z' i.i.d. N(0,1) from seed draw_seed + p."""
    H = w.heads if heads is None else heads
    phi, wq, wk = basis if basis is not None else calib_basis(w, device)
    gen = _generator(w.draw_seed + p, device)
    N, D = w.n_tokens, w.head_dim
    out = []
    for proj in (wq, wk):
        z = torch.randn(H, N, D, generator=gen, device=device, dtype=torch.float32)
        z.add_(torch.matmul(phi, proj[:H]).mul_(w.alpha))
        out.append(z.to(torch.bfloat16))
    return tuple(out)
