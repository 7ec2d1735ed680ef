"""GPU parity of calibatt_sparse_attn_fwd (through the C ABI) against the fp64
oracle on the same seeded bf16 inputs.

Bar: max-abs <= 2e-2 and relative Frobenius <= 1e-2 on every compared
output; kept-block lists bit-exact against the oracle's compilation.
Small cases compare every output; the full Wan / Mochi layer shapes compare
all heads on the first, the ragged last and seeded query blocks (and
sampled tokens of repeat heads)."""

import numpy as np
import pytest
import torch

import oracle
from synth import (ATTN_WORKLOADS, VideoGrid, bernoulli_mask, bf16_bits, block_mask,
                   gaussian_bf16, n_blocks, qkv, repeat_flags)
from tests._util import assert_attn_close, f64, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def run(cbs, q, k, v, mask_np, scale, flags=None, grid=None):
    mask = torch.from_numpy(mask_np).to(DEV)
    off, idx = cbs.compile_skiplist(mask)
    o = cbs.sparse_attention(q, k, v, off, idx, scale, flags, grid)
    torch.cuda.synchronize()
    return o, off, idx


def oracle_head_blocks(q, k, v, mask, scale, h, blocks):
    qb, kb, vb = (bf16_bits(t[h]) for t in (q, k, v))
    return [oracle.block_sparse_attention_block(qb, kb, vb, scale, np.flatnonzero(mask[h, r]), r)
            for r in blocks]


def full_compare(cbs, q, k, v, mask, scale, what):
    o, off, idx = run(cbs, q, k, v, mask, scale)
    H, N, _ = q.shape
    R = n_blocks(N)
    for h in range(H):
        got = f64(o[h])
        want = np.concatenate(oracle_head_blocks(q, k, v, mask, scale, h, range(R)))
        e = assert_attn_close(got, want, f"{what} head {h}")
        say(f"  {what} head {h}: max-abs {e[0]:.2e} rel-fro {e[1]:.2e}")
    return o, off, idx


def test_single_head_1k(gpu):
    w = ATTN_WORKLOADS["single_head_1k"]
    say("case single_head_1k")
    q, k, v = (t.to(DEV) for t in qkv(w))
    mask = block_mask(w)
    _, off, idx = full_compare(gpu, q, k, v, mask, w.scale, "single_head_1k")
    o_off, o_idx = oracle.compile_skiplist(mask)
    assert np.array_equal(off.cpu().numpy(), o_off) and np.array_equal(idx.cpu().numpy(), o_idx)


@pytest.mark.parametrize("N,H,seed", [(1000, 3, 1), (130, 2, 2), (128, 1, 3), (7, 1, 4), (2944, 2, 5)])
def test_ragged_and_tiny(gpu, N, H, seed):
    say(f"case ragged N={N} H={H}")
    q, k, v = (gaussian_bf16(seed * 10 + i, (H, N, 128)).to(DEV) for i in range(3))
    R = n_blocks(N)
    mask = bernoulli_mask(seed, H, R, 0.5, diagonal=True)
    if R > 2:
        mask[0, 1, :] = 0          # an empty kept list -> zeros
    o, _, _ = full_compare(gpu, q, k, v, mask, 1 / np.sqrt(128), f"N={N}")
    if R > 2:
        assert not f64(o[0, 128:256]).any()


def test_peaky_scores(gpu):
    """Scaled-up queries make softmax rows concentrated, so the tolerance
    bites on large outputs."""
    say("case peaky")
    N, H = 1024, 2
    q = gaussian_bf16(71, (H, N, 128), std=4.0).to(DEV)
    k, v = (gaussian_bf16(72 + i, (H, N, 128)).to(DEV) for i in range(2))
    mask = bernoulli_mask(73, H, 8, 0.4)
    full_compare(gpu, q, k, v, mask, 1 / np.sqrt(128), "peaky")


def test_all_kept_is_dense(gpu):
    say("case all-kept")
    N, H = 1000, 2
    q, k, v = (gaussian_bf16(80 + i, (H, N, 128), std=2.0).to(DEV) for i in range(3))
    o, _, _ = run(gpu, q, k, v, np.ones((H, 8, 8), np.uint8), 0.1)
    for h in range(H):
        want = oracle.dense_attention(*(bf16_bits(t[h]) for t in (q, k, v)), 0.1)
        assert_attn_close(f64(o[h]), want, "all-kept")


def test_skipped_blocks_do_not_matter_bitwise(gpu):
    say("case skipped-blocks")
    N, H = 1024, 2
    q, k, v = (gaussian_bf16(90 + i, (H, N, 128)).to(DEV) for i in range(3))
    mask = bernoulli_mask(93, H, 8, 0.5)
    o1, _, _ = run(gpu, q, k, v, mask, 0.09)
    k2, v2 = k.clone(), v.clone()
    for h in range(H):
        skipped_everywhere = [c for c in range(8) if not mask[h, :, c].any()]
        for c in skipped_everywhere:
            k2[h, c * 128:(c + 1) * 128] = 7.0
            v2[h, c * 128:(c + 1) * 128] = -3.0
    # Perturb a block that row 0 skips but others keep: only rows keeping it may change.
    c_pert = int(np.flatnonzero(mask[0, 0] == 0)[0])
    k2[0, c_pert * 128:(c_pert + 1) * 128] += 1.0
    o2, _, _ = run(gpu, q, k2, v2, mask, 0.09)
    assert torch.equal(o1[1], o2[1])
    for r in range(8):
        if not mask[0, r, c_pert]:
            assert torch.equal(o1[0, r * 128:(r + 1) * 128], o2[0, r * 128:(r + 1) * 128])


def test_deterministic(gpu):
    say("case deterministic")
    N, H = 2000, 4
    q, k, v = (gaussian_bf16(100 + i, (H, N, 128)).to(DEV) for i in range(3))
    mask = bernoulli_mask(103, H, n_blocks(N), 0.6)
    o1, _, _ = run(gpu, q, k, v, mask, 0.09)
    o2, _, _ = run(gpu, q, k, v, mask, 0.09)
    assert torch.equal(o1, o2)


def test_strided_layout(gpu):
    """[N][H][D] interleaved storage (stride_token = H*D) gives the same
    result as contiguous [H][N][D]."""
    say("case strided")
    N, H = 700, 3
    base = [gaussian_bf16(110 + i, (N, H, 128)).to(DEV) for i in range(3)]
    views = [t.permute(1, 0, 2) for t in base]
    mask = bernoulli_mask(113, H, n_blocks(N), 0.5)
    m = torch.from_numpy(mask).to(DEV)
    off, idx = gpu.compile_skiplist(m)
    o_view = torch.empty_like(base[0]).permute(1, 0, 2)
    gpu.calibatt_sparse_attn_fwd(*views, o_view, off, idx, 0.09)
    o_cont = gpu.sparse_attention(*(t.contiguous() for t in views), off, idx, 0.09)
    torch.cuda.synchronize()
    assert torch.equal(o_view.contiguous(), o_cont)


def test_split_calls_match_full_call(gpu):
    """calibatt_prepare_vt + calibatt_sparse_attn_fwd_vt give the full call's
    output bit for bit, including repeat heads and a ragged tail."""
    say("case split calls")
    F, Hs, W, kk = 2, 30, 7, 5
    N, H = F * Hs * W, 3
    q, k, v = (gaussian_bf16(130 + i, (H, N, 128)).to(DEV) for i in range(3))
    mask = bernoulli_mask(133, H, n_blocks(N), 0.5, diagonal=True)
    flags = np.array([0, 1, 0], np.uint8)
    off, idx = gpu.compile_skiplist(torch.from_numpy(mask).to(DEV))
    o_full = gpu.sparse_attention(q, k, v, off, idx, 0.09, flags, (F, Hs, W, kk))
    ws = torch.empty(gpu.calibatt_sparse_attn_fwd_workspace(H, N), dtype=torch.uint8, device=DEV)
    gpu.calibatt_prepare_vt(v, ws)
    o_split = torch.empty_like(q)
    gpu.calibatt_sparse_attn_fwd_vt(q, k, ws, o_split, off, idx, 0.09, flags, (F, Hs, W, kk))
    torch.cuda.synchronize()
    assert torch.equal(o_full, o_split)


@pytest.mark.parametrize("F,Hs,W,kk", [(2, 30, 7, 5), (3, 45, 4, 5), (2, 10, 13, 10), (1, 7, 9, 3)])
def test_repeat_heads_small(gpu, F, Hs, W, kk):
    say(f"case repeat grid {F}x{Hs}x{W} k={kk}")
    N = F * Hs * W
    H = 3
    q, k, v = (gaussian_bf16(120 + i, (H, N, 128), std=1.5).to(DEV) for i in range(3))
    R = n_blocks(N)
    mask = bernoulli_mask(124, H, R, 0.5)
    flags = np.array([0, 1, 1], np.uint8)
    o, _, _ = run(gpu, q, k, v, mask, 0.09, flags, (F, Hs, W, kk))
    want0 = oracle.block_sparse_attention(*(bf16_bits(t[0]) for t in (q, k, v)), 0.09, mask[0])
    assert_attn_close(f64(o[0]), want0, "non-repeat head")
    for h in (1, 2):
        want = oracle.repeat_head_attention(*(bf16_bits(t[h]) for t in (q, k, v)), 0.09, F, Hs, W, kk)
        assert_attn_close(f64(o[h]), want, f"repeat head {h}")
        # copies are exact: every row equals its anchor row bit for bit
        og = o[h].view(F, Hs, W, 128)
        arow = oracle.anchor_of_row(Hs, kk)
        for y in range(Hs):
            assert torch.equal(og[:, y], og[:, int(arow[y])])


def sampled_blocks(R, seed, n=14):
    rng = np.random.Generator(np.random.PCG64(seed))
    extra = rng.choice(np.arange(1, R - 1), size=min(n, R - 2), replace=False)
    return sorted(set([0, R - 1, *extra.tolist()]))


# (layer, part, parts): heads part, part + parts, ... of the layer, so each
# case stays well inside the per-test time limit
FULL_SIZE_CASES = [("wan21_480p_layer", p, 2) for p in range(2)] + \
    [("wan21_720p_layer", p, 4) for p in range(4)] + [("mochi1_480p_layer", p, 2) for p in range(2)]


@pytest.mark.parametrize("name,part,parts", FULL_SIZE_CASES)
def test_full_size_layer_sampled(gpu, name, part, parts):
    """Every head of the layer (one part of them per case): the first, the
    last and 14 seeded query blocks of each block-sparse head, and 897
    tokens of each repeat head, against the oracle."""
    w = ATTN_WORKLOADS[name]
    say(f"case full-size {name} part {part}/{parts}: H={w.heads} N={w.n_tokens}")
    q, k, v = qkv(w, device=DEV)
    mask = block_mask(w)
    flags = repeat_flags(w)
    grid = (w.grid.frames, w.grid.rows, w.grid.cols, w.anchors) if flags.any() else None
    o, off, idx = run(gpu, q, k, v, mask, w.scale, flags if flags.any() else None, grid)
    R = w.n_blocks
    kept = (mask.reshape(w.heads, -1).sum(1))
    assert (kept == w.keep_per_head()).all()
    o_off, o_idx = oracle.compile_skiplist(mask)
    assert np.array_equal(off.cpu().numpy(), o_off) and np.array_equal(idx.cpu().numpy(), o_idx)
    for h in range(part, w.heads, parts):
        qb, kb, vb = (bf16_bits(t[h]) for t in (q, k, v))
        if flags[h]:
            rng = np.random.Generator(np.random.PCG64(1000 + h))
            toks = np.r_[np.arange(128), rng.integers(0, w.n_tokens, 768), w.n_tokens - 1]
            want = oracle.repeat_head_attention(qb, kb, vb, w.scale, w.grid.frames, w.grid.rows,
                                                w.grid.cols, w.anchors, toks)
            got = f64(o[h][torch.from_numpy(toks).to(DEV)])
            assert_attn_close(got, want, f"{name} repeat head {h}")
            continue
        blocks = sampled_blocks(R, 500 + h)
        want = np.concatenate([oracle.block_sparse_attention_block(qb, kb, vb, w.scale,
                                                                   np.flatnonzero(mask[h, r]), r)
                               for r in blocks])
        rows = np.concatenate([np.arange(r * 128, min(r * 128 + 128, w.n_tokens)) for r in blocks])
        got = f64(o[h][torch.from_numpy(rows).to(DEV)])
        e = assert_attn_close(got, want, f"{name} head {h}")
        if h % 10 == 0:
            say(f"  {name} head {h}: max-abs {e[0]:.2e} rel-fro {e[1]:.2e}")


@pytest.mark.parametrize("name,head", [("wan21_720p_layer", 0), ("wan21_720p_layer", 39),
                                       ("wan21_480p_layer", 7), ("wan21_480p_layer", 33)])
def test_full_size_head_full_output(gpu, name, head):
    """Every output token of one head of the full layer (all query blocks,
    the launch covering all 40 heads as the bench times it) against the
    oracle, block by block."""
    w = ATTN_WORKLOADS[name]
    say(f"case full output {name} head {head}")
    q, k, v = qkv(w, device=DEV)
    mask = block_mask(w)
    o, _, _ = run(gpu, q, k, v, mask, w.scale)
    qb, kb, vb = (oracle.as_f64(bf16_bits(t[head])) for t in (q, k, v))
    want = np.concatenate([oracle.block_sparse_attention_block(qb, kb, vb, w.scale,
                                                               np.flatnonzero(mask[head, r]), r)
                           for r in range(w.n_blocks)])
    e = assert_attn_close(f64(o[head]), want, f"{name} head {head}")
    say(f"  max-abs {e[0]:.2e} rel-fro {e[1]:.2e} over {w.n_tokens} tokens")


MOCHI_REPEAT_CASES = [(flag, part) for flag in (1, 2) for part in range(2)]


@pytest.mark.parametrize("flag,part", MOCHI_REPEAT_CASES)
def test_mochi_repeat_heads_full_output(gpu, flag, part):
    """Every output token (all 44,520) of the Mochi 480p layer's repeat heads
    (three of the six per case), plain (flag 1) or keeping the head's block
    mask (flag 2), against the oracle; and every spatial row equals its
    anchor row bit for bit at this shape."""
    w = ATTN_WORKLOADS["mochi1_480p_layer"]
    say(f"case Mochi repeat heads full output flag={flag} part {part}/2")
    q, k, v = qkv(w, device=DEV)
    mask = block_mask(w)
    flags = repeat_flags(w) * flag
    F, Hs, W, kk = w.grid.frames, w.grid.rows, w.grid.cols, w.anchors
    o, _, _ = run(gpu, q, k, v, mask, w.scale, flags, (F, Hs, W, kk))
    arow = oracle.anchor_of_row(Hs, kk)
    heads = np.flatnonzero(flags)[part::2]
    assert heads.size == 3
    for h in heads:
        og = o[h].view(F, Hs, W, 128)
        for y in range(Hs):
            assert torch.equal(og[:, y], og[:, int(arow[y])]), (h, y)
        qb, kb, vb = (oracle.as_f64(bf16_bits(t[h])) for t in (q, k, v))
        got = f64(o[h])
        want = np.empty_like(got)
        step = 4 * Hs * W                                      # four frames per oracle call
        for t0 in range(0, w.n_tokens, step):
            toks = np.arange(t0, min(t0 + step, w.n_tokens))
            if flag == 1:
                want[toks] = oracle.repeat_head_attention(qb, kb, vb, w.scale, F, Hs, W, kk, toks)
            else:
                want[toks] = oracle.repeat_head_attention_masked(qb, kb, vb, w.scale, F, Hs, W, kk,
                                                                 mask[h], toks)
        e = assert_attn_close(got, want, f"repeat head {h} flag {flag}")
        say(f"  head {h}: max-abs {e[0]:.2e} rel-fro {e[1]:.2e} over {w.n_tokens} tokens")


def test_mfma_rate_probe(gpu):
    """The matrix-core probe runs through the C ABI and reports a rate
    between a tenth of the published dense bf16 peak and that peak."""
    sink = torch.zeros(1, dtype=torch.float32, device=DEV)
    gpu.calibatt_mfma_rate_probe(sink, 100, 512)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    flop = gpu.calibatt_mfma_rate_probe(sink, 2000, 2048)
    e1.record()
    torch.cuda.synchronize()
    assert flop == 2048 * 4 * 2000 * 8 * 32768
    tflops = flop / (e0.elapsed_time(e1) * 1e-3) / 1e12
    say(f"  mfma probe: {tflops:.0f} TFLOP/s")
    assert 251.7 < tflops < 2516.6 * 1.02
    assert float(sink[0]) == 0.0


def test_more_heads_than_one_launch(gpu):
    """300 heads (launches hold at most 256), every seventh a repeat head:
    each head against the oracle."""
    F, Hs, W, kk = 2, 4, 32, 2
    N, H = F * Hs * W, 300
    say(f"case {H} heads N={N}")
    q, k, v = (gaussian_bf16(400 + i, (H, N, 128)).to(DEV) for i in range(3))
    R = n_blocks(N)
    mask = bernoulli_mask(404, H, R, 0.5, diagonal=True)
    flags = (np.arange(H) % 7 == 6).astype(np.uint8)
    o, _, _ = run(gpu, q, k, v, mask, 0.1, flags, (F, Hs, W, kk))
    for h in range(H):
        qb, kb, vb = (bf16_bits(t[h]) for t in (q, k, v))
        if flags[h]:
            want = oracle.repeat_head_attention(qb, kb, vb, 0.1, F, Hs, W, kk)
        else:
            want = oracle.block_sparse_attention(qb, kb, vb, 0.1, mask[h])
        assert_attn_close(f64(o[h]), want, f"head {h}")


def test_out_of_range_entries_are_skipped(gpu):
    """Indices outside [0, R) are skipped and offsets are clamped to
    [0, nnz): the output equals the oracle over the in-range entries."""
    N, H = 700, 2
    R = n_blocks(N)
    say(f"case out-of-range list entries N={N}")
    q, k, v = (gaussian_bf16(410 + i, (H, N, 128)).to(DEV) for i in range(3))
    mask = bernoulli_mask(414, H, R, 0.5, diagonal=True)
    off, idx = oracle.compile_skiplist(mask)
    # insert -1, R and R+7 after the first entry of every row (still "ascending" order is not needed)
    new_idx, new_off = [], [0]
    for row in range(H * R):
        ent = idx[off[row]:off[row + 1]].tolist()
        ent = ent[:1] + [-1, R, R + 7] + ent[1:]
        new_idx += ent
        new_off.append(len(new_idx))
    nnz = len(new_idx)
    off_t = torch.tensor(new_off, dtype=torch.int32, device=DEV)
    idx_t = torch.tensor(new_idx, dtype=torch.int32, device=DEV)
    o = torch.empty_like(q)
    gpu.calibatt_sparse_attn_fwd(q, k, v, o, off_t, idx_t, 0.1)
    # offsets past nnz: the last row's range is clamped to [.., nnz)
    off_big = off_t.clone()
    off_big[-1] = nnz + 1000
    o2 = torch.empty_like(q)
    gpu.calibatt_sparse_attn_fwd(q, k, v, o2, off_big, idx_t, 0.1)
    torch.cuda.synchronize()
    assert torch.equal(o, o2)
    for h in range(H):
        want = oracle.block_sparse_attention(*(bf16_bits(t[h]) for t in (q, k, v)), 0.1, mask[h])
        assert_attn_close(f64(o[h]), want, f"head {h}")


@pytest.mark.parametrize("F,Hs,W,kk", [(2, 30, 7, 5), (3, 12, 40, 3), (1, 8, 100, 2), (2, 10, 13, 10)])
def test_masked_repeat_heads_small(gpu, F, Hs, W, kk):
    """Flags 0 / 1 / 2 in one call: block-sparse, repeat, and repeat heads
    whose anchor queries keep their block-row's list (one block-row keeps
    nothing, so its anchor queries give zeros)."""
    N = F * Hs * W
    H = 4
    R = n_blocks(N)
    say(f"case masked repeat grid {F}x{Hs}x{W} k={kk} R={R}")
    q, k, v = (gaussian_bf16(430 + i, (H, N, 128), std=1.5).to(DEV) for i in range(3))
    mask = bernoulli_mask(434, H, R, 0.5, diagonal=True)
    if R > 2:
        mask[3, 1, :] = 0
    flags = np.array([0, 1, 2, 2], np.uint8)
    o, _, _ = run(gpu, q, k, v, mask, 0.09, flags, (F, Hs, W, kk))
    for h in range(H):
        qb, kb, vb = (bf16_bits(t[h]) for t in (q, k, v))
        if flags[h] == 0:
            want = oracle.block_sparse_attention(qb, kb, vb, 0.09, mask[h])
        elif flags[h] == 1:
            want = oracle.repeat_head_attention(qb, kb, vb, 0.09, F, Hs, W, kk)
        else:
            want = oracle.repeat_head_attention_masked(qb, kb, vb, 0.09, F, Hs, W, kk, mask[h])
        assert_attn_close(f64(o[h]), want, f"head {h} flag {flags[h]}")
    if R > 2:
        src = oracle.repeat_source_token(np.arange(N), F, Hs, W, kk)
        assert not f64(o[3])[src // 128 == 1].any()


def test_masked_repeat_with_every_block_kept_is_plain_repeat(gpu):
    F, Hs, W, kk = 2, 30, 13, 5
    N = F * Hs * W
    R = n_blocks(N)
    say("case masked repeat, full mask")
    q, k, v = (gaussian_bf16(440 + i, (2, N, 128)).to(DEV) for i in range(3))
    mask = np.ones((2, R, R), np.uint8)
    o1, _, _ = run(gpu, q, k, v, mask, 0.1, np.array([1, 1], np.uint8), (F, Hs, W, kk))
    o2, _, _ = run(gpu, q, k, v, mask, 0.1, np.array([2, 2], np.uint8), (F, Hs, W, kk))
    assert torch.equal(o1, o2)


def test_masked_repeat_mochi_shape_sampled(gpu):
    """Mochi 480p layer with its repeat heads also keeping their masks:
    sampled tokens of every repeat head against the oracle."""
    w = ATTN_WORKLOADS["mochi1_480p_layer"]
    say(f"case masked repeat {w.name}")
    q, k, v = qkv(w, device=DEV)
    mask = block_mask(w)
    flags = repeat_flags(w) * 2
    grid = (w.grid.frames, w.grid.rows, w.grid.cols, w.anchors)
    o, _, _ = run(gpu, q, k, v, mask, w.scale, flags, grid)
    for h in np.flatnonzero(flags):
        qb, kb, vb = (bf16_bits(t[h]) for t in (q, k, v))
        rng = np.random.Generator(np.random.PCG64(2000 + h))
        toks = np.r_[np.arange(64), rng.integers(0, w.n_tokens, 448), w.n_tokens - 1]
        want = oracle.repeat_head_attention_masked(qb, kb, vb, w.scale, *grid, mask[h], toks)
        got = f64(o[h][torch.from_numpy(toks).to(DEV)])
        e = assert_attn_close(got, want, f"masked repeat head {h}")
    say(f"  last head max-abs {e[0]:.2e}")


def test_masked_repeat_at_the_block_limit(gpu):
    """Masked repeat heads at the largest supported R (896 blocks: the
    per-query bitmaps and the union list fill the LDS left beside the two
    tiles), one masked repeat head beside a block-sparse head; sampled
    tokens against the oracle, the block-sparse head on sampled blocks."""
    F, Hs, W, kk = 28, 32, 128, 5
    N = F * Hs * W                       # 114,688 tokens = 896 blocks
    R = n_blocks(N)
    assert R == 896
    say(f"case masked repeat at R={R}")
    q, k, v = (gaussian_bf16(470 + i, (2, N, 128)).to(DEV) for i in range(3))
    mask = bernoulli_mask(473, 2, R, 0.3, True)
    flags = np.array([2, 0], np.uint8)
    o, _, _ = run(gpu, q, k, v, mask, 128 ** -0.5, flags, (F, Hs, W, kk))
    qb, kb, vb = (bf16_bits(t[0]) for t in (q, k, v))
    rng = np.random.Generator(np.random.PCG64(474))
    toks = np.r_[np.arange(32), rng.integers(0, N, 96), N - 1]
    want = oracle.repeat_head_attention_masked(qb, kb, vb, 128 ** -0.5, F, Hs, W, kk, mask[0], toks)
    e = assert_attn_close(f64(o[0][torch.from_numpy(toks).to(DEV)]), want, "masked repeat head")
    blocks = [0, 447, R - 1]
    want1 = oracle_head_blocks(q, k, v, mask, 128 ** -0.5, 1, blocks)
    for r, wb in zip(blocks, want1):
        assert_attn_close(f64(o[1][r * 128:(r + 1) * 128]), wb, f"sparse head block {r}")
    say(f"  masked head max-abs {e[0]:.2e}")


@pytest.mark.parametrize("kind", ["sparse", "repeat", "masked"])
def test_graph_capture_replays_match_eager(gpu, kind):
    """calibatt_sparse_attn_fwd captured in a HIP graph (V^T pre-pass and
    attention; no memset nodes): three replays, each after new inputs are
    written eagerly, equal the eager call on those inputs bit for bit."""
    H, N = 3, 1000
    grid = (2, 20, 25, 5)
    scale = 128 ** -0.5
    say(f"case graph capture {kind}")
    flags = {"sparse": None, "repeat": np.array([0, 1, 0], np.uint8),
             "masked": np.array([2, 0, 1], np.uint8)}[kind]
    g_arg = None if flags is None else grid
    q, k, v = (gaussian_bf16(480 + i, (H, N, 128)).to(DEV) for i in range(3))
    mask = bernoulli_mask(484, H, n_blocks(N), 0.35, True)
    off, idx = gpu.compile_skiplist(torch.from_numpy(mask).to(DEV))
    ws = torch.empty(gpu.calibatt_sparse_attn_fwd_workspace(H, N), dtype=torch.uint8, device=DEV)
    o = torch.empty_like(q)

    def call(out):
        gpu.calibatt_sparse_attn_fwd(q, k, v, out, off, idx, scale, flags, g_arg, workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(o)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(o)
    torch.cuda.synchronize()
    for rep in range(3):
        for i, t in enumerate((q, k, v)):
            t.copy_(gaussian_bf16(490 + 10 * rep + i, (H, N, 128)).to(DEV))
        want = torch.empty_like(q)
        call(want)
        torch.cuda.synchronize()
        o.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, want), f"replay {rep}"


def test_side_stream_scratch_is_not_reused_early(gpu):
    """Calls on an explicit side stream with library scratch allocated by the
    binding (V^T workspace, energy workspace): right after each call returns,
    the current stream allocates and overwrites a large buffer while the side
    stream may still be running. The scratch is allocated on the side
    stream, so the allocator cannot hand it out before that work is done;
    the results equal the same calls made on the current stream."""
    say("case side-stream scratch")
    H, N = 8, 9000
    q, k, v = (gaussian_bf16(520 + i, (H, N, 128)).to(DEV) for i in range(3))
    mask = bernoulli_mask(523, H, n_blocks(N), 0.6, True)
    off, idx = gpu.compile_skiplist(torch.from_numpy(mask).to(DEV))
    want = gpu.sparse_attention(q, k, v, off, idx, 0.1)
    want_e = gpu.block_energy(q[:2], k[:2], 0.1)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    for rep in range(3):
        o = torch.empty_like(q)
        o.record_stream(side)
        e = torch.empty_like(want_e)
        e.record_stream(side)
        gpu.calibatt_sparse_attn_fwd(q, k, v, o, off, idx, 0.1, stream=side)
        junk = torch.full((gpu.calibatt_sparse_attn_fwd_workspace(H, N) // 2,), 7.0,
                          dtype=torch.bfloat16, device=DEV)
        gpu.calibatt_block_energy(q[:2], k[:2], e, 0.1, stream=side)
        junk2 = torch.full((gpu.calibatt_block_energy_workspace(2, N) // 4,), -1.0,
                           dtype=torch.float32, device=DEV)
        side.synchronize()
        torch.cuda.synchronize()
        assert torch.equal(o, want), rep
        assert torch.equal(e, want_e), rep
        del junk, junk2


def test_two_streams_in_flight_at_once(gpu):
    """Independent calls on two streams with nothing ordering them (their own
    workspaces and outputs; the library keeps no state between calls): the
    results equal the same calls made one after the other."""
    say("case two streams at once")
    cases = []
    for i, (H, N, p) in enumerate(((6, 12000, 0.5), (4, 9000, 0.3))):
        q, k, v = (gaussian_bf16(560 + 10 * i + j, (H, N, 128)).to(DEV) for j in range(3))
        mask = bernoulli_mask(565 + i, H, n_blocks(N), p, True)
        off, idx = gpu.compile_skiplist(torch.from_numpy(mask).to(DEV))
        ws = torch.empty(gpu.calibatt_sparse_attn_fwd_workspace(H, N), dtype=torch.uint8, device=DEV)
        cases.append((q, k, v, off, idx, ws))
    want = [gpu.sparse_attention(q, k, v, off, idx, 0.1) for q, k, v, off, idx, _ in cases]
    want_e = gpu.block_energy(cases[1][0][:2], cases[1][1][:2], 0.1)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [torch.full_like(w, 3.0) for w in want]
    e = torch.full_like(want_e, -1.0)
    ews = torch.empty(gpu.calibatt_block_energy_workspace(2, cases[1][0].shape[1]), dtype=torch.uint8,
                      device=DEV)
    for st in streams:
        st.wait_stream(torch.cuda.current_stream())
    for rep in range(2):
        for i, (q, k, v, off, idx, ws) in enumerate(cases):
            gpu.calibatt_sparse_attn_fwd(q, k, v, outs[i], off, idx, 0.1, workspace=ws,
                                         stream=streams[i])
        gpu.calibatt_block_energy(cases[1][0][:2], cases[1][1][:2], e, 0.1, ews, stream=streams[1])
        for st in streams:
            st.synchronize()
        for i in range(2):
            assert torch.equal(outs[i], want[i]), (rep, i)
        assert torch.equal(e, want_e), rep


@pytest.mark.parametrize("N,H", [(1000, 2), (75600, 1)])
def test_mask_that_keeps_nothing(gpu, N, H):
    """Every list empty (nnz = 0, an empty index tensor): the call succeeds
    and every output row is zero, with the output buffer pre-filled with
    non-zeros so that unwritten rows would show."""
    say(f"case empty mask N={N} H={H}")
    q, k, v = (gaussian_bf16(500 + i, (H, N, 128)).to(DEV) for i in range(3))
    R = n_blocks(N)
    off, idx = gpu.compile_skiplist(torch.zeros(H, R, R, dtype=torch.uint8, device=DEV))
    assert idx.numel() == 0 and not off.any()
    o = torch.full_like(q, 3.0)
    gpu.calibatt_sparse_attn_fwd(q, k, v, o, off, idx, 128 ** -0.5)
    torch.cuda.synchronize()
    assert not o.float().any()
