"""Seeded random cases through the C ABI against the fp64 oracle (hypothesis,
derandomised, so every run draws the same cases).

Attention ([CalibAtt blog] = the zhichai.net article on CalibAtt, §三 online
inference and repeat heads): random head counts, token counts given as a
video grid (frames x rows x cols, any anchor count the geometry rule
accepts), block masks of any density including empty block-rows, and a
random mix of block-sparse heads, repeat heads and repeat heads that keep
their mask, in one call; every output token against the oracle within the
attention bar (max-abs 2e-2, relative Frobenius 1e-2).

Calibration (§三 offline steps 1-3): random token counts and query scales;
block energies against the oracle within 1e-4 E + 1e-7, then the greedy
selection at a random eps on the GPU's own energies, votes and counts bit
for bit against the oracle's selection on the same fp32 values."""

import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle
from synth import bf16_bits, gaussian_bf16, n_blocks
from tests._util import assert_attn_close, assert_energy_close, f64, say

pytestmark = pytest.mark.gpu
DEV = "cuda"
SETTINGS = settings(max_examples=60, deadline=None, derandomize=True, database=None,
                    suppress_health_check=[HealthCheck.too_slow,
                                           HealthCheck.function_scoped_fixture])


def _valid_anchors(rows):
    ok = []
    for a in range(1, rows + 1):
        try:
            oracle.check_anchor_geometry(rows, a)
            ok.append(a)
        except ValueError:
            pass
    return ok


@st.composite
def attention_cases(draw):
    frames = draw(st.integers(1, 3))
    rows = draw(st.integers(1, 12))
    cols = draw(st.integers(1, 40))
    anchors = draw(st.sampled_from(_valid_anchors(rows)))
    heads = draw(st.integers(1, 3))
    flags = draw(st.lists(st.integers(0, 2), min_size=heads, max_size=heads))
    keep = draw(st.sampled_from([0.0, 0.2, 0.5, 0.9, 1.0]))
    seed = draw(st.integers(0, 2 ** 30))
    std = draw(st.sampled_from([0.5, 1.0, 2.0]))
    scale = draw(st.sampled_from([0.05, 128 ** -0.5, 0.15]))
    return frames, rows, cols, anchors, heads, flags, keep, seed, std, scale


@SETTINGS
@given(attention_cases())
def test_random_attention_calls(gpu, case):
    F, rows, cols, anchors, H, flags, keep, seed, std, scale = case
    N = F * rows * cols
    R = n_blocks(N)
    say(f"case random attention F={F} rows={rows} cols={cols} k={anchors} H={H} "
        f"flags={flags} keep={keep} seed={seed} std={std} scale={scale:.4f}")
    q = gaussian_bf16(seed, (H, N, 128), std=std).to(DEV)
    k = gaussian_bf16(seed + 1, (H, N, 128)).to(DEV)
    v = gaussian_bf16(seed + 2, (H, N, 128)).to(DEV)
    mask = (np.random.default_rng(seed).random((H, R, R)) < keep).astype(np.uint8)
    fl = np.asarray(flags, dtype=np.uint8)
    grid = (F, rows, cols, anchors) if fl.any() else None
    off, idx = gpu.compile_skiplist(torch.from_numpy(mask).to(DEV))
    o = gpu.sparse_attention(q, k, v, off, idx, scale, fl if fl.any() else None, grid)
    torch.cuda.synchronize()
    for h in range(H):
        qb, kb, vb = (bf16_bits(t[h]) for t in (q, k, v))
        if fl[h] == 0:
            want = oracle.block_sparse_attention(qb, kb, vb, scale, mask[h])
        elif fl[h] == 1:
            want = oracle.repeat_head_attention(qb, kb, vb, scale, F, rows, cols, anchors)
        else:
            want = oracle.repeat_head_attention_masked(qb, kb, vb, scale, F, rows, cols, anchors,
                                                       mask[h])
        assert_attn_close(f64(o[h]), want, f"head {h} flag {fl[h]}")


@st.composite
def energy_cases(draw):
    heads = draw(st.integers(1, 2))
    n = draw(st.integers(1, 900))
    seed = draw(st.integers(0, 2 ** 30))
    std = draw(st.sampled_from([0.3, 1.0, 2.5]))
    eps = draw(st.floats(0.3, 1.0))
    return heads, n, seed, std, eps


@SETTINGS
@given(energy_cases())
def test_random_energy_and_selection(gpu, case):
    H, N, seed, std, eps = case
    R = n_blocks(N)
    scale = 128 ** -0.5
    say(f"case random energy H={H} N={N} seed={seed} std={std} eps={eps:.4f}")
    q = gaussian_bf16(seed, (H, N, 128), std=std).to(DEV)
    k = gaussian_bf16(seed + 1, (H, N, 128)).to(DEV)
    e = gpu.block_energy(q, k, scale)
    efx = oracle.eps_fx(eps)
    votes = torch.zeros(H, R, R, dtype=torch.uint8, device=DEV)
    nsel = torch.zeros(H, R, dtype=torch.int32, device=DEV)
    gpu.calibatt_build_mask(e, efx, votes, nsel)
    torch.cuda.synchronize()
    e_np = e.cpu().numpy()
    for h in range(H):
        assert_energy_close(e_np[h].astype(np.float64),
                            oracle.block_energy(bf16_bits(q[h]), bf16_bits(k[h]), scale), f"head {h}")
    sel, n_star = oracle.greedy_select(e_np.astype(np.float64).reshape(H * R, R), efx)
    assert np.array_equal(votes.cpu().numpy().reshape(H * R, R), sel)
    assert np.array_equal(nsel.cpu().numpy().reshape(-1), n_star)
