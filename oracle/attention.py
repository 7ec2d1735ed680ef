"""fp64 attention oracle: dense, block-sparse over kept-block lists, and
"repeat" heads. TEST INFRASTRUCTURE (see the package docstring).

Conventions (readings of the pages where they are silent):

* Blocks are 128 contiguous tokens in sequence order ([CalibAtt blog] §二,
  observation 1: the B x B block grid with B = 128). The last block of a
  sequence whose length is not a multiple of 128 is ragged: keys at or past
  N do not exist and take no part in any softmax; query rows past N are not
  outputs.
* A query block with an empty kept list produces zeros.
* Video tokens are frame-major and row-major inside a frame ([CalibAtt blog]
  §六: a frame of H x W tokens is unrolled row by row).
"""

from __future__ import annotations

import numpy as np

BLOCK = 128


def as_f64(x) -> np.ndarray:
    """fp64 view of an input (the array itself when it is already fp64,
    else a converted copy). uint16 / int16 arrays are raw bf16 bit patterns
    and are decoded exactly (bf16 is the top half of an fp32). Callers never
    write to the result."""
    a = np.asarray(x)
    if a.dtype in (np.uint16, np.int16):
        u32 = a.view(np.uint16).astype(np.uint32) << 16
        return u32.view(np.float32).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


def _attend(qr: np.ndarray, kk: np.ndarray, vv: np.ndarray, scale: float) -> np.ndarray:
    """softmax(scale * qr kk^T) vv, row by row, max-subtracted, in fp64."""
    s = (qr @ kk.T) * scale
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    return (p @ vv) / p.sum(axis=1, keepdims=True)


def dense_attention(q, k, v, scale: float, rows=None) -> np.ndarray:
    """Dense softmax attention of one head: O_i = sum_j softmax_j(scale q_i.k_j) v_j
    over all N keys. q, k, v: [N][D]. rows: optional query indices."""
    q, k, v = as_f64(q), as_f64(k), as_f64(v)
    qr = q if rows is None else q[np.asarray(rows)]
    return _attend(qr, k, v, scale)


def kept_keys(kept_blocks, n_tokens: int) -> np.ndarray:
    """Token indices of the kept key blocks, ascending, clipped to n_tokens."""
    blocks = np.sort(np.asarray(kept_blocks, dtype=np.int64))
    if blocks.size == 0:
        return np.zeros(0, dtype=np.int64)
    idx = (blocks[:, None] * BLOCK + np.arange(BLOCK)[None, :]).ravel()
    return idx[idx < n_tokens]


def block_sparse_attention_block(q, k, v, scale: float, kept_blocks, r: int) -> np.ndarray:
    """Output rows of query block r when it attends only to the key blocks in
    kept_blocks ([CalibAtt blog] §三 online inference: the skip list tells
    the kernel which blocks to compute and which to skip; [abstract]: selected
    connections are computed densely, unselected ones skipped).

    Equivalent to dense attention with the logits of skipped blocks at -inf.
    Returns [|I_r|][D]; zeros when kept_blocks is empty."""
    q, k, v = as_f64(q), as_f64(k), as_f64(v)
    N, D = q.shape
    rows = np.arange(r * BLOCK, min((r + 1) * BLOCK, N))
    keys = kept_keys(kept_blocks, N)
    if keys.size == 0:
        return np.zeros((rows.size, D))
    return _attend(q[rows], k[keys], v[keys], scale)


def block_sparse_attention(q, k, v, scale: float, mask) -> np.ndarray:
    """Whole-head block-sparse attention. mask: [R][R] (1 = keep block c for
    query block r)."""
    q, k, v = as_f64(q), as_f64(k), as_f64(v)
    N, D = q.shape
    mask = np.asarray(mask)
    R = (N + BLOCK - 1) // BLOCK
    assert mask.shape == (R, R)
    out = np.zeros((N, D))
    for r in range(R):
        cols = np.flatnonzero(mask[r])
        out[r * BLOCK:min((r + 1) * BLOCK, N)] = block_sparse_attention_block(
            q, k, v, scale, cols, r)
    return out


# ----------------------------------------------------------------------------
# Repeat heads ([CalibAtt blog] §二 observation 4, §三: a head flagged as
# spatially repeating computes only k = 5 anchor rows per frame and broadcasts
# them to the other rows of the same frame).


def check_anchor_geometry(rows: int, anchors: int) -> None:
    """The repeat head computes its anchor rows and hands each one's output
    to the other rows of its frame ([CalibAtt blog] §三), so every anchor
    row must keep its own output: A(m) must lie in the segment m it serves,
    floor(A(m) * anchors / rows) == m. Geometries where some anchor does not
    (possible only for rows / 2 < anchors < rows, e.g. 9 anchors in 10 rows)
    are rejected."""
    if not 1 <= anchors <= rows:
        raise ValueError(f"anchors {anchors} not in [1, rows={rows}]")
    for m in range(anchors):
        a = (2 * m + 1) * rows // (2 * anchors)
        if a * anchors // rows != m:
            raise ValueError(f"{anchors} anchors in {rows} rows: anchor row {a} would not serve "
                             f"its own segment {m}")


def anchor_rows(rows: int, anchors: int) -> np.ndarray:
    """Evenly spaced anchor rows of a frame with `rows` spatial rows: the
    middle row of each of `anchors` equal segments, A(m) = floor((2m+1) *
    rows / (2 * anchors))."""
    check_anchor_geometry(rows, anchors)
    m = np.arange(anchors)
    return (2 * m + 1) * rows // (2 * anchors)


def anchor_of_row(rows: int, anchors: int) -> np.ndarray:
    """Anchor serving each spatial row y: the anchor of y's segment,
    a(y) = A(floor(y * anchors / rows))."""
    y = np.arange(rows)
    return anchor_rows(rows, anchors)[y * anchors // rows]


def repeat_source_token(tokens, frames: int, rows: int, cols: int, anchors: int) -> np.ndarray:
    """For output token n = (f, y, x), the query token (f, a(y), x) whose
    attention output it receives."""
    n = np.asarray(tokens, dtype=np.int64)
    f, rem = np.divmod(n, rows * cols)
    y, x = np.divmod(rem, cols)
    return f * rows * cols + anchor_of_row(rows, anchors)[y] * cols + x


def repeat_head_attention(q, k, v, scale: float, frames: int, rows: int,
                          cols: int, anchors: int, tokens=None) -> np.ndarray:
    """Output of a repeat head: every token takes the dense-attention output
    (over all N keys) of its frame's anchor row at the same column.
    tokens: optional output token indices (default all)."""
    q, k, v = as_f64(q), as_f64(k), as_f64(v)
    N = q.shape[0]
    assert frames * rows * cols == N
    toks = np.arange(N) if tokens is None else np.asarray(tokens, dtype=np.int64)
    src = repeat_source_token(toks, frames, rows, cols, anchors)
    uniq, inv = np.unique(src, return_inverse=True)
    o = _attend(q[uniq], k, v, scale)
    return o[inv]


def repeat_head_attention_masked(q, k, v, scale: float, frames: int, rows: int, cols: int,
                                 anchors: int, mask, tokens=None) -> np.ndarray:
    """Repeat head that also keeps its block mask (a variant the pages leave
    open: [CalibAtt blog] §三 names no mask for repeat heads). Every token
    takes the output of its frame's anchor-row query at the same column, as
    in repeat_head_attention, but that anchor query n attends only to the keys
    of the blocks its own block-row floor(n / 128) keeps (mask [R][R]); an
    anchor query whose row keeps nothing yields zeros."""
    q, k, v = as_f64(q), as_f64(k), as_f64(v)
    N = q.shape[0]
    assert frames * rows * cols == N
    mask = np.asarray(mask)
    toks = np.arange(N) if tokens is None else np.asarray(tokens, dtype=np.int64)
    src = repeat_source_token(toks, frames, rows, cols, anchors)
    uniq, inv = np.unique(src, return_inverse=True)
    out = np.zeros((uniq.size, q.shape[1]))
    for r in np.unique(uniq // BLOCK):
        sel = np.flatnonzero(uniq // BLOCK == r)
        keys = kept_keys(np.flatnonzero(mask[r]), N)
        if keys.size:
            out[sel] = _attend(q[uniq[sel]], k[keys], v[keys], scale)
    return out[inv]
