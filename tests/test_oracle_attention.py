"""Pins of the attention oracle against things other than itself: a library
routine (torch's fp64 SDPA on the CPU), a textbook per-row softmax written
with the math module, closed forms, and invariants the method fixes.

Sources: [CalibAtt blog] = the zhichai.net article on CalibAtt; §二
observation 1 (B x B blocks, B = 128), §三 online inference (skip list for
non-repeat heads; k anchor rows broadcast within a frame for repeat heads),
§六 (row-major frame layout)."""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def rnd(seed, *shape):
    return np.random.Generator(np.random.PCG64(seed)).standard_normal(shape)


def sdpa(q, k, v, scale, mask=None):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))[None, None]
    m = None if mask is None else torch.from_numpy(mask)[None, None]
    o = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=m, scale=scale)
    return o[0, 0].numpy()


def test_block_size_matches_pages():
    const = json.load(open(os.path.join(GOLD, "paper_constants.json")))
    assert oracle.BLOCK == const["block_size"]


def test_dense_vs_torch_sdpa():
    q, k, v = rnd(1, 300, 128), rnd(2, 300, 128), rnd(3, 300, 128)
    for scale in (1 / math.sqrt(128), 0.5):
        np.testing.assert_allclose(oracle.dense_attention(q, k, v, scale), sdpa(q, k, v, scale),
                                   rtol=1e-12, atol=1e-12)


def test_dense_vs_textbook_loop():
    q, k, v = rnd(4, 5, 3), rnd(5, 7, 3), rnd(6, 7, 2)
    out = oracle.dense_attention(q, k, v, 0.7)
    for i in range(5):
        logits = [0.7 * sum(q[i, d] * k[j, d] for d in range(3)) for j in range(7)]
        w = [math.exp(x) for x in logits]
        z = sum(w)
        for e in range(2):
            assert abs(out[i, e] - sum(w[j] * v[j, e] for j in range(7)) / z) < 1e-12


def test_bf16_decode_is_exact():
    bits = np.array([0x3F80, 0xC000, 0x0000, 0x3E00, 0x4049, 0x8001], dtype=np.uint16)
    want = [1.0, -2.0, 0.0, 0.125, 3.140625, -(2.0 ** -133)]
    assert list(oracle.as_f64(bits)) == want


@pytest.mark.parametrize("N", [1024, 1000, 130])
def test_all_kept_equals_dense(N):
    q, k, v = rnd(7, N, 128), rnd(8, N, 128), rnd(9, N, 128)
    R = (N + 127) // 128
    got = oracle.block_sparse_attention(q, k, v, 0.09, np.ones((R, R), np.uint8))
    np.testing.assert_allclose(got, sdpa(q, k, v, 0.09), rtol=1e-11, atol=1e-12)


def test_token_level_mask_equivalence():
    """Block-sparse == SDPA with a boolean token mask expanded from the block
    mask (skipped blocks get -inf logits); ragged N."""
    N = 1000
    R = 8
    q, k, v = rnd(10, N, 128), rnd(11, N, 128), rnd(12, N, 128)
    rng = np.random.Generator(np.random.PCG64(13))
    bm = (rng.random((R, R)) < 0.4).astype(np.uint8)
    bm[np.arange(R), np.arange(R)] = 1
    tok = np.kron(bm, np.ones((128, 128), np.uint8))[:N, :N].astype(bool)
    np.testing.assert_allclose(oracle.block_sparse_attention(q, k, v, 0.1, bm),
                               sdpa(q, k, v, 0.1, tok), rtol=1e-11, atol=1e-12)


def test_single_block_list():
    N = 700
    q, k, v = rnd(14, N, 128), rnd(15, N, 128), rnd(16, N, 128)
    for r, c in [(0, 3), (5, 5), (2, 5)]:   # block 5 is the ragged tail (60 keys)
        got = oracle.block_sparse_attention_block(q, k, v, 0.2, [c], r)
        rows = slice(r * 128, min(r * 128 + 128, N))
        keys = slice(c * 128, min(c * 128 + 128, N))
        np.testing.assert_allclose(got, sdpa(q[rows], k[keys], v[keys], 0.2), rtol=1e-12, atol=1e-12)


def test_zero_queries_average_values():
    """Q = 0: every kept key gets the same weight, O_i = mean of V over the
    kept keys (closed form); the tail block has only N mod 128 keys."""
    N = 1000
    k, v = rnd(17, N, 128), rnd(18, N, 128)
    q = np.zeros((N, 128))
    cols = [1, 7]
    keys = np.r_[128:256, 896:1000]
    got = oracle.block_sparse_attention_block(q, k, v, 0.1, cols, 3)
    np.testing.assert_allclose(got, np.broadcast_to(v[keys].mean(0), got.shape), rtol=1e-12, atol=1e-13)


def test_skipped_blocks_have_no_influence():
    N = 1024
    q, k, v = rnd(19, N, 128), rnd(20, N, 128), rnd(21, N, 128)
    cols = [0, 2, 5]
    a = oracle.block_sparse_attention_block(q, k, v, 0.1, cols, 4)
    k2, v2 = k.copy(), v.copy()
    k2[128:256] += 50.0
    v2[384:512] = 1e6
    b = oracle.block_sparse_attention_block(q, k2, v2, 0.1, cols, 4)
    assert np.array_equal(a, b)


def test_empty_list_gives_zeros():
    q = rnd(22, 256, 128)
    assert not oracle.block_sparse_attention_block(q, q, q, 0.1, [], 1).any()


def test_anchor_rows_closed_form():
    # A(m) = floor((2m+1) Hs / (2k)): the centre row of each of k segments.
    assert list(oracle.anchor_rows(30, 5)) == [3, 9, 15, 21, 27]
    assert list(oracle.anchor_rows(45, 5)) == [4, 13, 22, 31, 40]
    a = oracle.anchor_of_row(30, 5)
    assert list(a) == [3] * 6 + [9] * 6 + [15] * 6 + [21] * 6 + [27] * 6
    # where k divides Hs, every row is served by a nearest anchor
    for Hs, k in ((30, 5), (45, 5), (12, 3), (5, 5)):
        A = oracle.anchor_rows(Hs, k)
        for y, ay in enumerate(oracle.anchor_of_row(Hs, k)):
            assert abs(y - ay) == min(abs(y - b) for b in A)


def test_every_anchor_serves_itself_where_supported():
    """Brute force over small geometries: the oracle accepts exactly the
    (rows, anchors) where every anchor row is served by itself (checked
    here by building the row -> anchor map and looking at each anchor),
    which includes every geometry with anchors == rows or rows >=
    2 anchors - 1; the rejected ones are those where some anchor row would
    take another anchor's output."""
    rejected = 0
    for Hs in range(1, 41):
        for k in range(1, Hs + 1):
            m = np.arange(k)
            A = (2 * m + 1) * Hs // (2 * k)              # the formula, restated independently
            a = A[np.arange(Hs) * k // Hs]
            self_served = all(a[y] == y for y in A)
            if k == Hs or Hs >= 2 * k - 1:
                assert self_served, (Hs, k)
            if self_served:
                assert list(oracle.anchor_of_row(Hs, k)) == list(a)
            else:
                rejected += 1
                with pytest.raises(ValueError):
                    oracle.anchor_rows(Hs, k)
    assert rejected > 0
    # the example of a rejected geometry: 10 rows, 9 anchors (row 1 would copy row 0);
    # 8 rows with 5 anchors is accepted (anchors 0, 2, 4, 5, 7 each serve themselves)
    with pytest.raises(ValueError):
        oracle.anchor_of_row(10, 9)
    assert list(oracle.anchor_rows(8, 5)) == [0, 2, 4, 5, 7]


def test_repeat_head_reduces_to_dense_when_every_row_is_an_anchor():
    F, Hs, W = 2, 5, 13
    N = F * Hs * W
    q, k, v = rnd(23, N, 128), rnd(24, N, 128), rnd(25, N, 128)
    np.testing.assert_allclose(oracle.repeat_head_attention(q, k, v, 0.1, F, Hs, W, Hs),
                               sdpa(q, k, v, 0.1), rtol=1e-12, atol=1e-12)


def test_repeat_head_exact_when_rows_repeat():
    """If every spatial row of a frame has the same queries, broadcasting the
    anchor rows reproduces dense attention."""
    F, Hs, W = 3, 10, 11
    N = F * Hs * W
    base = rnd(26, F, 1, W, 128)
    q = np.broadcast_to(base, (F, Hs, W, 128)).reshape(N, 128)
    k, v = rnd(27, N, 128), rnd(28, N, 128)
    np.testing.assert_allclose(oracle.repeat_head_attention(q, k, v, 0.1, F, Hs, W, 5),
                               sdpa(q, k, v, 0.1), rtol=1e-12, atol=1e-12)


def test_repeat_head_anchor_rows_are_dense_and_copies_exact():
    F, Hs, W = 2, 30, 7
    N = F * Hs * W
    q, k, v = rnd(29, N, 128), rnd(30, N, 128), rnd(31, N, 128)
    o = oracle.repeat_head_attention(q, k, v, 0.1, F, Hs, W, 5).reshape(F, Hs, W, 128)
    d = sdpa(q, k, v, 0.1).reshape(F, Hs, W, 128)
    for y in (3, 9, 15, 21, 27):
        np.testing.assert_allclose(o[:, y], d[:, y], rtol=1e-12, atol=1e-12)
    for y in range(Hs):
        assert np.array_equal(o[:, y], o[:, 3 + 6 * (y // 6)])


# Repeat head that also keeps its block mask (a variant; the pages name no
# mask for repeat heads): pinned to torch's fp64 SDPA with the token mask the
# block mask implies.


def token_mask(mask, N):
    b = np.arange(N) // oracle.BLOCK
    return mask[b][:, b].astype(bool)


def test_masked_repeat_anchor_rows_equal_masked_sdpa():
    F, Hs, W = 2, 12, 20                       # N = 480, R = 4 (last block 96 keys)
    N = F * Hs * W
    R = -(-N // 128)
    q, k, v = rnd(41, N, 128), rnd(42, N, 128), rnd(43, N, 128)
    mask = (np.random.default_rng(44).random((R, R)) < 0.5).astype(np.uint8)
    np.fill_diagonal(mask, 1)
    o = oracle.repeat_head_attention_masked(q, k, v, 0.1, F, Hs, W, 3, mask).reshape(F, Hs, W, 128)
    d = sdpa(q, k, v, 0.1, token_mask(mask, N)).reshape(F, Hs, W, 128)
    anchors = oracle.anchor_rows(Hs, 3)
    for y in anchors:
        np.testing.assert_allclose(o[:, y], d[:, y], rtol=1e-12, atol=1e-12)
    a = oracle.anchor_of_row(Hs, 3)
    for y in range(Hs):
        assert np.array_equal(o[:, y], o[:, a[y]])


def test_masked_repeat_full_mask_is_plain_repeat_and_empty_row_is_zero():
    F, Hs, W = 1, 8, 40                        # N = 320, R = 3
    N = F * Hs * W
    q, k, v = rnd(45, N, 128), rnd(46, N, 128), rnd(47, N, 128)
    full = np.ones((3, 3), np.uint8)
    np.testing.assert_allclose(oracle.repeat_head_attention_masked(q, k, v, 0.1, F, Hs, W, 2, full),
                               oracle.repeat_head_attention(q, k, v, 0.1, F, Hs, W, 2),
                               rtol=1e-12, atol=1e-12)
    m = full.copy()
    m[1] = 0                                   # block-row 1 keeps nothing
    o = oracle.repeat_head_attention_masked(q, k, v, 0.1, F, Hs, W, 2, m)
    src = oracle.repeat_source_token(np.arange(N), F, Hs, W, 2)
    zero = src // 128 == 1
    assert zero.any() and not o[zero].any()
    assert np.abs(o[~zero]).sum() > 0
