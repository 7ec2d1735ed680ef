"""fp64 / integer oracle of the offline calibration: block energy, greedy
selection at the threshold eps(t), vote averaging across prompts with a
threshold rho, and compilation of a block mask into per-query-block kept
lists. TEST INFRASTRUCTURE (see the package docstring).

Readings of the pages where they leave a step open:

* Energy of a ragged last block-row is normalised by its true row count
  |I_r| (equal to B for every full block), so that each block-row's
  energies sum to one, which the "reach eps" rule presumes.
* Cumulative energies are compared at a resolution of 2^-40: every energy
  and the threshold are rounded to the nearest multiple of 2^-40 (ties to
  even) and summed as integers. The selection is then independent of the
  order of summation. "Reaches" means >=.
* Equal energies are taken in ascending column order.
* If no prefix reaches eps, every block of the row is selected.
* Averaged mask entries exactly at rho are kept. A block-row left empty by
  the threshold keeps its most-voted column (the lowest such column).
* Kept lists are in ascending column order.
"""

from __future__ import annotations

import math

import numpy as np

from .attention import BLOCK, as_f64

FX_BITS = 40


def block_energy_row(q, k, scale: float, r: int) -> np.ndarray:
    """E_{r,c} for every key block c of query block-row r ([CalibAtt blog] §三,
    offline calibration steps 1-2): P = softmax(scale Q K^T) row by row over
    all N keys (the post-softmax attention), then
    E_{r,c} = (1/|I_r|) * sum_{i in I_r} sum_{j in J_c} P_ij."""
    q, k = as_f64(q), as_f64(k)
    N = q.shape[0]
    R = (N + BLOCK - 1) // BLOCK
    rows = np.arange(r * BLOCK, min((r + 1) * BLOCK, N))
    s = (q[rows] @ k.T) * scale
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    e = np.zeros(R)
    for c in range(R):
        e[c] = p[:, c * BLOCK:min((c + 1) * BLOCK, N)].sum()
    return e / rows.size


def block_energy(q, k, scale: float, rows=None) -> np.ndarray:
    """E for one head, [R][R] (or only the listed block-rows, [len][R])."""
    q = as_f64(q)
    R = (q.shape[0] + BLOCK - 1) // BLOCK
    rr = range(R) if rows is None else rows
    return np.stack([block_energy_row(q, k, scale, r) for r in rr])


def quantize_energy(e) -> np.ndarray:
    """Energies as integer multiples of 2^-40, rounded to nearest (ties to
    even). Exact for fp32 and fp64 inputs in [0, 2^12)."""
    return np.rint(np.asarray(e, dtype=np.float64) * float(2 ** FX_BITS)).astype(np.int64)


def eps_schedule(t, T, A, C, k):
    """Energy threshold at sampling step t ([CalibAtt blog] §三):
    eps(t) = A + (C - A) * exp(-k * t / T). Step 0 is the first, noisiest
    step, where eps = C; eps decays towards A."""
    return A + (C - A) * np.exp(-k * np.asarray(t, dtype=np.float64) / T)


def eps_fx(eps: float) -> int:
    """Threshold as an integer multiple of 2^-40."""
    return int(np.rint(float(eps) * float(2 ** FX_BITS)))


def greedy_select_row(e_fx, eps_fx_value: int):
    """[CalibAtt blog] §三 step 3: the fewest key blocks whose cumulative
    energy reaches eps, taken greedily from the largest energy down.
    Pure-Python loop; returns (selected columns in greedy order, n*)."""
    e = [int(x) for x in e_fx]
    order = sorted(range(len(e)), key=lambda c: (-e[c], c))
    acc = 0
    for n, c in enumerate(order, start=1):
        acc += e[c]
        if acc >= eps_fx_value:
            return order[:n], n
    return order, len(order)


def greedy_select(E, eps_fx_value: int):
    """Vectorised greedy selection over the last axis of E (fp32/fp64
    energies, [..., R]). Returns (selection mask uint8 [..., R], n* int32
    [...]). Same rule as greedy_select_row."""
    e = quantize_energy(E)
    R = e.shape[-1]
    cols = np.broadcast_to(np.arange(R), e.shape)
    order = np.lexsort((cols, -e), axis=-1)          # energy desc, column asc
    csum = np.cumsum(np.take_along_axis(e, order, axis=-1), axis=-1)
    reached = csum >= eps_fx_value
    nstar = np.where(reached.any(axis=-1), reached.argmax(axis=-1) + 1, R)
    rank_sel = np.arange(R) < nstar[..., None]       # in sorted position
    sel = np.zeros(e.shape, dtype=np.uint8)
    np.put_along_axis(sel, order, rank_sel.astype(np.uint8), axis=-1)
    return sel, nstar.astype(np.int32)


def accumulate_votes(selections) -> np.ndarray:
    """Sum of per-prompt selection masks: |D| * M_bar ([CalibAtt blog] §三,
    the mean over calibration prompts), kept as an integer count."""
    sel = np.asarray(selections)
    return sel.astype(np.int64).sum(axis=0)


def binarize(votes, n_prompts: int, rho_num: int = 1, rho_den: int = 2) -> np.ndarray:
    """Keep block (r, c) iff M_bar >= rho, i.e. votes * rho_den >=
    rho_num * |D| ([CalibAtt blog] §三: binarised at rho = 0.5). A row with
    nothing kept keeps its most-voted column (lowest index on ties)."""
    v = np.asarray(votes, dtype=np.int64)
    keep = (v * rho_den >= rho_num * n_prompts).astype(np.uint8)
    empty = keep.sum(axis=-1) == 0
    if empty.any():
        top = v.argmax(axis=-1)  # first maximum = lowest column
        np.put_along_axis(keep, top[..., None],
                          np.maximum(np.take_along_axis(keep, top[..., None], -1),
                                     empty[..., None].astype(np.uint8)), axis=-1)
    return keep


def compile_skiplist(mask):
    """Per-query-block kept lists of a [H][R][R] mask in CSR form: offsets
    int32 [H*R+1], indices int32 [nnz], ascending within each row."""
    m = np.asarray(mask)
    H, R, R2 = m.shape
    assert R == R2
    flat = m.reshape(H * R, R) != 0
    counts = flat.sum(axis=1)
    offsets = np.zeros(H * R + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    indices = np.concatenate([np.flatnonzero(row) for row in flat]) if H * R else np.zeros(0)
    return offsets.astype(np.int32), indices.astype(np.int32)


def skiplist_to_mask(offsets, indices, H: int, R: int) -> np.ndarray:
    m = np.zeros((H * R, R), dtype=np.uint8)
    for row in range(H * R):
        m[row, indices[offsets[row]:offsets[row + 1]]] = 1
    return m.reshape(H, R, R)


__all__ = [n for n in dir() if not n.startswith("_") and n not in ("math", "np")]


# ----------------------------------------------------------------------------
# Spatial similarity of a head and its repeat classification ([CalibAtt
# blog] §二 observation 4: rows of one frame attend alike; §三: a spatial
# similarity score s per (t, l, h), above gamma = 0.87 the head is computed
# from k anchor rows and broadcast). The pages give no formula for s. The
# reading taken here, with the anchors of repeat_head_attention:
#
# * profile of spatial row (f, y): the mean over its W query tokens of the
#   post-softmax attention summed per key block (block granularity, as the
#   masks), rho_{f,y}[c] = (1/W) sum_{i in row (f,y)} sum_{j in J_c} P_ij;
# * s = mean over frames f and non-anchor rows y of the cosine similarity
#   between rho_{f,y} and the profile of its anchor row, rho_{f,a(y)}
#   (1 when every row is an anchor); averaged over prompts by the caller;
# * repeat iff s > gamma ("exceeds").
# PARITY UNPINNED as to the formula (the pages have none); the function is
# pinned to its reading by closed forms in tests/test_oracle_calibration.py.

GAMMA = 0.87


def row_profiles(q, k, scale: float, frames: int, rows: int, cols: int) -> np.ndarray:
    """rho: [frames*rows][R], one row per spatial row (f, y)."""
    q, k = as_f64(q), as_f64(k)
    N = q.shape[0]
    assert frames * rows * cols == N
    R = (N + BLOCK - 1) // BLOCK
    out = np.zeros((frames * rows, R))
    for fy in range(frames * rows):
        qi = q[fy * cols:(fy + 1) * cols]
        s = (qi @ k.T) * scale
        p = np.exp(s - s.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        for c in range(R):
            out[fy, c] = p[:, c * BLOCK:min((c + 1) * BLOCK, N)].sum() / cols
    return out


def spatial_similarity(q, k, scale: float, frames: int, rows: int, cols: int,
                       anchors: int) -> float:
    """s of one head for one prompt (see the reading above)."""
    from .attention import anchor_of_row
    prof = row_profiles(q, k, scale, frames, rows, cols)
    a = anchor_of_row(rows, anchors)
    total, count = 0.0, 0
    for f in range(frames):
        for y in range(rows):
            if a[y] == y:
                continue
            u = prof[f * rows + y]
            w = prof[f * rows + a[y]]
            total += float(u @ w) / (np.linalg.norm(u) * np.linalg.norm(w))
            count += 1
    return 1.0 if count == 0 else total / count


def classify_repeat(s_mean, gamma: float = GAMMA) -> np.ndarray:
    """Repeat flags (uint8) of heads whose prompt-averaged s exceeds gamma."""
    return (np.asarray(s_mean, dtype=np.float64) > gamma).astype(np.uint8)
