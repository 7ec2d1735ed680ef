"""calibatt_sparse_attn_fwd_noalloc (V^T tiles in the library's static device
scratch, no workspace, no allocation) against calibatt_sparse_attn_fwd with a
workspace, through the C ABI: bit for bit, over consecutive calls whose
inputs shrink (the scratch keeps the previous call's contents), including
calls that need several head chunks (more V^T tiles than the scratch holds)
and repeat heads of both kinds."""

import numpy as np
import pytest
import torch

import oracle
from synth import ATTN_WORKLOADS, bernoulli_mask, bf16_bits, block_mask, gaussian_bf16, n_blocks, qkv
from tests._util import assert_attn_close, f64, say

pytestmark = pytest.mark.gpu
DEV = "cuda"
TILES = 268435456 // (128 * 128 * 2)


def both(cbs, q, k, v, off, idx, scale, flags=None, grid=None):
    o_ws = torch.empty_like(q)
    cbs.calibatt_sparse_attn_fwd(q, k, v, o_ws, off, idx, scale, flags, grid)
    o_na = torch.full_like(q, 5.0)
    cbs.calibatt_sparse_attn_fwd_noalloc(q, k, v, o_na, off, idx, scale, flags, grid)
    torch.cuda.synchronize()
    return o_ws, o_na


def test_noalloc_matches_workspace_call_on_shrinking_inputs(gpu):
    assert gpu.NOALLOC_SCRATCH_BYTES == 268435456
    # 1) Wan 480p layer: 40 heads x 256 blocks = 10240 tiles > 8192: two chunks of 20 heads
    w = ATTN_WORKLOADS["wan21_480p_layer"]
    assert w.heads * w.n_blocks > TILES
    say(f"case noalloc {w.name} (two head chunks)")
    q, k, v = qkv(w, device=DEV)
    off, idx = gpu.compile_skiplist(torch.from_numpy(block_mask(w)).to(DEV))
    o_ws, o_na = both(gpu, q, k, v, off, idx, w.scale)
    assert torch.equal(o_ws, o_na)
    del q, k, v, o_ws, o_na
    # 2) a smaller call right after: 3 heads, N = 1000, flags 0 / 1 / 2, against
    #    the workspace call bit for bit and the oracle within the attention bar
    H, N, grid = 3, 1000, (2, 20, 25, 5)
    say("case noalloc small, repeat heads")
    q, k, v = (gaussian_bf16(530 + i, (H, N, 128)).to(DEV) for i in range(3))
    mask = bernoulli_mask(533, H, n_blocks(N), 0.4, True)
    off, idx = gpu.compile_skiplist(torch.from_numpy(mask).to(DEV))
    flags = np.array([0, 1, 2], np.uint8)
    o_ws, o_na = both(gpu, q, k, v, off, idx, 0.09, flags, grid)
    assert torch.equal(o_ws, o_na)
    qb, kb, vb = (bf16_bits(t[0]) for t in (q, k, v))
    assert_attn_close(f64(o_na[0]), oracle.block_sparse_attention(qb, kb, vb, 0.09, mask[0]), "head 0")
    # 3) smaller still: one head, N = 300
    say("case noalloc one head N=300")
    q, k, v = (gaussian_bf16(540 + i, (1, 300, 128)).to(DEV) for i in range(3))
    off, idx = gpu.compile_skiplist(torch.ones(1, 3, 3, dtype=torch.uint8, device=DEV))
    o_ws, o_na = both(gpu, q, k, v, off, idx, 0.1)
    assert torch.equal(o_ws, o_na)


def test_noalloc_headline_layer(gpu):
    """Wan 720p layer (40 heads x 591 blocks: four chunks of 10 heads), then
    the Mochi layer (24 heads x 348 blocks: two chunks of 12, three repeat
    heads in each) with its repeat heads plain (flag 1) and keeping their
    block masks (flag 2): bit for bit against the workspace call."""
    from synth import repeat_flags
    for name, flag in (("wan21_720p_layer", 1), ("mochi1_480p_layer", 1), ("mochi1_480p_layer", 2)):
        w = ATTN_WORKLOADS[name]
        say(f"case noalloc {name} repeat flag {flag}")
        q, k, v = qkv(w, device=DEV)
        off, idx = gpu.compile_skiplist(torch.from_numpy(block_mask(w)).to(DEV))
        fl = repeat_flags(w) * np.uint8(flag)
        grid = (w.grid.frames, w.grid.rows, w.grid.cols, w.anchors) if fl.any() else None
        o_ws, o_na = both(gpu, q, k, v, off, idx, w.scale, fl if fl.any() else None, grid)
        assert torch.equal(o_ws, o_na), (name, flag)
        del q, k, v, o_ws, o_na


def test_noalloc_captured_in_a_graph(gpu):
    """After a first eager call on the device, the no-alloc call captured in
    a HIP graph (two head chunks: 40 heads x 256 blocks > 8192 tiles)
    replays bit-identical to the workspace call on fresh inputs, with eager
    work and synchronisation between the replays."""
    H, N = 40, 32760
    say("case noalloc graph capture")
    q, k, v = (gaussian_bf16(600 + i, (H, N, 128)).to(DEV) for i in range(3))
    mask = bernoulli_mask(603, H, n_blocks(N), 0.3, True)
    off, idx = gpu.compile_skiplist(torch.from_numpy(mask).to(DEV))
    o = torch.empty_like(q)
    gpu.calibatt_sparse_attn_fwd_noalloc(q, k, v, o, off, idx, 0.1)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        gpu.calibatt_sparse_attn_fwd_noalloc(q, k, v, o, off, idx, 0.1, stream=side)
    torch.cuda.synchronize()
    for rep in range(3):
        for i, t in enumerate((q, k, v)):
            t.copy_(gaussian_bf16(610 + 10 * rep + i, (H, N, 128)).to(DEV))
        want = torch.empty_like(q)
        gpu.calibatt_sparse_attn_fwd(q, k, v, want, off, idx, 0.1)
        torch.cuda.synchronize()
        o.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, want), f"replay {rep}"
