"""GPU parity of the calibration path (calibatt_block_energy,
calibatt_build_mask, calibatt_finalize_mask, calibatt_compile_skiplist)
against the oracle, through the C ABI.

Bars: energies per element within 1e-4 relative + 1e-7 absolute and row L1
within 1e-4; selections, selected counts, votes, masks and kept lists
bit-exact when both sides start from the same fp32 energies; end to end
(GPU energies vs oracle energies) selections may differ only on rows whose
oracle prefix sums lie within 1e-4 of eps."""

import numpy as np
import pytest
import torch

import oracle
from synth import (CALIB_WORKLOADS, bernoulli_mask, bf16_bits, calib_basis, calib_draw,
                   energy_rows, gaussian_bf16, n_blocks)
from tests._util import assert_energy_close, f64, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def gpu_energy(cbs, q, k, scale):
    e = cbs.block_energy(q, k, scale)
    torch.cuda.synchronize()
    return e


@pytest.mark.parametrize("N,H,std", [(1024, 1, 1.0), (1024, 2, 4.0), (1000, 3, 2.0), (7, 1, 1.0),
                                     (2944, 2, 3.0)])
def test_energy_full(gpu, N, H, std):
    say(f"case energy N={N} H={H} std={std}")
    q = gaussian_bf16(200 + N, (H, N, 128), std=std).to(DEV)
    k = gaussian_bf16(201 + N, (H, N, 128)).to(DEV)
    e = f64(gpu_energy(gpu, q, k, 1 / np.sqrt(128)))
    for h in range(H):
        want = oracle.block_energy(bf16_bits(q[h]), bf16_bits(k[h]), 1 / np.sqrt(128))
        assert_energy_close(e[h], want, f"energy head {h}")
        np.testing.assert_allclose(e[h].sum(axis=1), 1.0, atol=1e-5)


def test_energy_zero_queries_closed_form(gpu):
    say("case energy Q=0")
    N = 1000
    q = torch.zeros(1, N, 128, dtype=torch.bfloat16, device=DEV)
    k = gaussian_bf16(210, (1, N, 128)).to(DEV)
    e = f64(gpu_energy(gpu, q, k, 0.1))[0]
    want = np.array([128] * 7 + [104]) / N
    np.testing.assert_allclose(e, np.broadcast_to(want, e.shape), rtol=1e-6)


@pytest.mark.parametrize("part", range(4))
def test_energy_calibration_size_sampled(gpu, part):
    """Calibration shape (40 heads, N = 32760 = 21 x 30 x 52), one draw:
    every head (heads part, part + 4, ... per case) on its first, last and
    14 seeded block-rows."""
    w = CALIB_WORKLOADS["calibration_480p"]
    say(f"case energy full-size part {part}/4 H={w.heads} N={w.n_tokens}")
    basis = calib_basis(w, DEV)
    q, k = calib_draw(w, 0, basis, DEV)
    e = gpu_energy(gpu, q, k, w.scale)
    R = n_blocks(w.n_tokens)
    assert np.allclose(f64(e).sum(axis=-1), 1.0, atol=1e-5)
    for h in range(part, w.heads, 4):
        rng = np.random.Generator(np.random.PCG64(700 + h))
        rows = sorted(set([0, R - 1, *rng.choice(np.arange(1, R - 1), 14, replace=False).tolist()]))
        want = oracle.block_energy(bf16_bits(q[h]), bf16_bits(k[h]), w.scale, rows)
        assert_energy_close(f64(e[h])[rows], want, f"energy head {h}")


@pytest.mark.parametrize("name,heads_per_chunk", [("calibration_480p", 7), ("wan21_720p_layer", 3)])
def test_energy_chunked_by_heads_is_bit_identical(gpu, name, heads_per_chunk):
    """A workspace holding only a few heads makes calibatt_block_energy run
    the heads in chunks; the energies equal those of one call over all heads
    bit for bit (480p calibration shape, and the 720p layer shape whose full
    workspace is 14.3 GB)."""
    from synth import ATTN_WORKLOADS, qkv
    if name in CALIB_WORKLOADS:
        w = CALIB_WORKLOADS[name]
        q, k = calib_draw(w, 1, calib_basis(w, DEV), DEV)
        scale = w.scale
    else:
        w = ATTN_WORKLOADS[name]
        q, k, _ = qkv(w, device=DEV)
        scale = w.scale
    H, N = q.shape[0], q.shape[1]
    R = n_blocks(N)
    say(f"case energy chunked {name} H={H} N={N}, {heads_per_chunk} heads per chunk")
    full = torch.empty(H, R, R, dtype=torch.float32, device=DEV)
    ws = torch.empty(gpu.calibatt_block_energy_workspace(H, N), dtype=torch.uint8, device=DEV)
    gpu.calibatt_block_energy(q, k, full, scale, ws)
    torch.cuda.synchronize()
    del ws
    part = torch.empty_like(full)
    ws = torch.empty(gpu.calibatt_block_energy_workspace(heads_per_chunk, N) + 100,
                     dtype=torch.uint8, device=DEV)
    gpu.calibatt_block_energy(q, k, part, scale, ws)
    torch.cuda.synchronize()
    assert torch.equal(full, part)
    assert np.allclose(full.sum(dim=-1).cpu().numpy(), 1.0, atol=1e-5)


def test_calibration_chain_on_gpu_energies_480p(gpu):
    """The calibration shape (40 heads, N = 32760, R = 256), four prompt
    draws: the library's own fp32 energies of all 40 heads go through
    calibatt_build_mask at eps(0), eps(25) and eps(49); votes and selected
    counts equal the oracle's greedy selection on those same energies bit
    for bit, and calibatt_finalize_mask at rho = 1/2 gives exactly
    oracle.binarize's masks and oracle.compile_skiplist's lists."""
    w = CALIB_WORKLOADS["calibration_480p"]
    R = n_blocks(w.n_tokens)
    draws = 4
    say(f"case calibration chain H={w.heads} N={w.n_tokens} draws={draws}")
    basis = calib_basis(w, DEV)
    E = torch.empty(draws, w.heads, R, R, dtype=torch.float32, device=DEV)
    for p in range(draws):
        q, k = calib_draw(w, p, basis, DEV)
        gpu.calibatt_block_energy(q, k, E[p], w.scale)
    torch.cuda.synchronize()
    E_host = E.cpu().numpy()
    assert np.allclose(E_host.sum(axis=-1), 1.0, atol=1e-5)
    for t in w.steps:
        efx = gpu.calibatt_eps_fx(t, w.total_steps, w.eps_floor, w.eps_start, w.eps_rate)
        assert efx == oracle.eps_fx(oracle.eps_schedule(t, w.total_steps, w.eps_floor,
                                                        w.eps_start, w.eps_rate))
        votes = torch.zeros(w.heads, R, R, dtype=torch.uint8, device=DEV)
        nsel = torch.zeros(draws, w.heads, R, dtype=torch.int32, device=DEV)
        gpu.calibatt_build_mask(E, efx, votes, nsel)
        sel_o, nstar_o = oracle.greedy_select(E_host, efx)
        votes_o = oracle.accumulate_votes(sel_o)
        assert np.array_equal(nsel.cpu().numpy(), nstar_o), f"n* differ at t={t}"
        assert np.array_equal(votes.cpu().numpy(), votes_o), f"votes differ at t={t}"
        mask = torch.empty_like(votes)
        off = torch.empty(w.heads * R + 1, dtype=torch.int32, device=DEV)
        idx = torch.empty(w.heads * R * R, dtype=torch.int32, device=DEV)
        nnz = gpu.calibatt_finalize_mask(votes, draws, *w.rho, mask, off, idx)
        want_mask = oracle.binarize(votes_o, draws, *w.rho)
        want_off, want_idx = oracle.compile_skiplist(want_mask)
        assert np.array_equal(mask.cpu().numpy(), want_mask), f"mask differs at t={t}"
        assert nnz == want_idx.size
        assert np.array_equal(off.cpu().numpy(), want_off)
        assert np.array_equal(idx.cpu().numpy()[:nnz], want_idx)
        say(f"  t={t}: eps {efx / 2 ** 40:.6f}, mean n* {nstar_o.mean():.1f}, kept {nnz / (w.heads * R * R):.4f}")


@pytest.mark.parametrize("kind", ["dirichlet", "peaky", "ties", "uniform", "onehot"])
@pytest.mark.parametrize("R", [8, 64, 100, 591, 2047])
def test_select_bit_exact(gpu, kind, R):
    say(f"case select {kind} R={R}")
    H = 2 if R < 1000 else 1
    draws = 3 if R <= 591 else 1
    E = np.stack([energy_rows(300 + 7 * d + R, H, R, kind) for d in range(draws)])
    if R == 2047:
        E = E[:, :, :64]  # 64 of the 2047 rows keep the case small
        E = np.ascontiguousarray(E)
    rows = E.shape[2]
    for eps in (0.5, 0.84, 0.9, 0.99):
        efx = gpu.calibatt_eps_fx(0, 1, eps, eps, 0)
        assert efx == oracle.eps_fx(eps)
        sel, nstar = oracle.greedy_select(E, efx)
        want_votes = oracle.accumulate_votes(sel)
        # The GPU takes [n_draws][H][R][R]; pad the row count to R with zero rows.
        Ep = np.zeros((draws, H, R, R), np.float32)
        Ep[:, :, :rows] = E
        votes = torch.zeros(H, R, R, dtype=torch.uint8, device=DEV)
        nsel = torch.zeros(draws, H, R, dtype=torch.int32, device=DEV)
        gpu.calibatt_build_mask(torch.from_numpy(Ep).to(DEV), efx, votes, nsel)
        torch.cuda.synchronize()
        v = votes.cpu().numpy()[:, :rows]
        assert np.array_equal(v, want_votes), f"votes differ (eps {eps})"
        assert np.array_equal(nsel.cpu().numpy()[:, :, :rows], nstar), f"n* differ (eps {eps})"


def test_votes_accumulate_and_saturate(gpu):
    say("case votes saturate")
    R, H = 16, 1
    E = energy_rows(400, H, R, "peaky")
    votes = torch.full((H, R, R), 250, dtype=torch.uint8, device=DEV)
    efx = oracle.eps_fx(0.9)
    Ed = torch.from_numpy(np.stack([E] * 10)).to(DEV)
    gpu.calibatt_build_mask(Ed, efx, votes)
    torch.cuda.synchronize()
    sel, _ = oracle.greedy_select(E, efx)
    want = np.minimum(250 + 10 * sel.astype(np.int64), 255)
    assert np.array_equal(votes.cpu().numpy(), want)


@pytest.mark.parametrize("H,R,n,rho", [(2, 8, 64, (1, 2)), (3, 100, 64, (1, 2)), (2, 591, 37, (3, 10)),
                                       (1, 33, 1, (1, 2)), (2, 50, 255, (7, 10))])
def test_finalize_bit_exact(gpu, H, R, n, rho):
    say(f"case finalize H={H} R={R} n={n} rho={rho}")
    rng = np.random.Generator(np.random.PCG64(R + n))
    votes = rng.integers(0, n + 1, size=(H, R, R)).astype(np.uint8)
    votes[0, 0] = 0                       # empty row -> fallback to column 0
    votes[0, 1] = 0
    votes[0, 1, R // 2] = 1 if n > 1 else 0  # below rho -> fallback to its argmax
    if n == 64:
        votes[-1, -1, :3] = [32, 31, 33]  # the rho tie is kept
    want_mask = oracle.binarize(votes, n, *rho)
    want_off, want_idx = oracle.compile_skiplist(want_mask)
    vd = torch.from_numpy(votes).to(DEV)
    mask = torch.empty_like(vd)
    off = torch.empty(H * R + 1, dtype=torch.int32, device=DEV)
    idx = torch.empty(H * R * R, dtype=torch.int32, device=DEV)
    nnz = gpu.calibatt_finalize_mask(vd, n, rho[0], rho[1], mask, off, idx)
    assert nnz == want_idx.size
    assert np.array_equal(mask.cpu().numpy(), want_mask)
    assert np.array_equal(off.cpu().numpy(), want_off)
    assert np.array_equal(idx.cpu().numpy()[:nnz], want_idx)


@pytest.mark.parametrize("H,R,p", [(40, 591, 0.375), (1, 1, 1.0), (3, 64, 0.0), (5, 2047, 0.01)])
def test_compile_bit_exact(gpu, H, R, p):
    say(f"case compile H={H} R={R}")
    m = bernoulli_mask(500 + R, H, R, p, diagonal=False)
    want_off, want_idx = oracle.compile_skiplist(m)
    off, idx = gpu.compile_skiplist(torch.from_numpy(m).to(DEV))
    assert np.array_equal(off.cpu().numpy(), want_off)
    assert np.array_equal(idx.cpu().numpy(), want_idx)


def test_calibration_end_to_end_small(gpu):
    """Small calibration run: energies -> selections at eps(t) for three
    steps -> votes over all draws -> binarised masks -> kept lists. GPU
    (energies included) vs oracle; selections may differ only on rows whose
    oracle prefix sums come within 1e-4 of eps."""
    w = CALIB_WORKLOADS["calibration_small"]
    say(f"case calibration small H={w.heads} N={w.n_tokens} draws={w.draws}")
    R = n_blocks(w.n_tokens)
    basis = calib_basis(w, "cpu")
    votes_g = {t: torch.zeros(w.heads, R, R, dtype=torch.uint8, device=DEV) for t in w.steps}
    votes_o = {t: np.zeros((w.heads, R, R), np.int64) for t in w.steps}
    near = 0
    for p in range(w.draws):
        q, k = calib_draw(w, p, basis, "cpu")
        e_g = gpu_energy(gpu, q.to(DEV), k.to(DEV), w.scale)
        e_o = np.stack([oracle.block_energy(bf16_bits(q[h]), bf16_bits(k[h]), w.scale)
                        for h in range(w.heads)])
        assert_energy_close(f64(e_g), e_o, f"draw {p}")
        for t in w.steps:
            efx = gpu.calibatt_eps_fx(t, w.total_steps, w.eps_floor, w.eps_start, w.eps_rate)
            nsel = torch.zeros(1, w.heads, R, dtype=torch.int32, device=DEV)
            before = votes_g[t].clone()
            gpu.calibatt_build_mask(e_g, efx, votes_g[t], nsel)
            sel_g = (votes_g[t] - before).cpu().numpy()
            sel_o, _ = oracle.greedy_select(e_o, efx)
            votes_o[t] += sel_o
            diff = np.flatnonzero((sel_g != sel_o).any(axis=-1).ravel())
            srt = -np.sort(-e_o, axis=-1)
            cs = np.cumsum(srt, axis=-1).reshape(-1, R)
            eps = efx / 2.0 ** 40
            for row in diff:
                assert np.min(np.abs(cs[row] - eps)) < 1e-4, f"draw {p} t {t} row {row}"
            near += diff.size
    say(f"  rows differing near eps: {near}")
    for t in w.steps:
        vg = votes_g[t].cpu().numpy()
        if near == 0:
            assert np.array_equal(vg, votes_o[t])
        mask = torch.empty(w.heads, R, R, dtype=torch.uint8, device=DEV)
        off = torch.empty(w.heads * R + 1, dtype=torch.int32, device=DEV)
        idx = torch.empty(w.heads * R * R, dtype=torch.int32, device=DEV)
        nnz = gpu.calibatt_finalize_mask(votes_g[t], w.draws, *w.rho, mask, off, idx)
        want = oracle.binarize(votes_o[t], w.draws, *w.rho)
        same_rows = (vg == votes_o[t]).all(axis=-1)
        assert np.array_equal(mask.cpu().numpy()[same_rows], want[same_rows])
        say(f"  t={t}: kept fraction {nnz / (w.heads * R * R):.3f}")


# ----------------------------------------------------------------------------
# Spatial similarity (calibatt_spatial_similarity after calibatt_block_energy).
# Bars: row profiles per element within 1e-4 relative + 1e-7 absolute (the
# energy bar), s within 1e-5 absolute.


def gpu_similarity(cbs, q, k, scale, grid):
    e, s, prof = cbs.energy_and_similarity(q, k, scale, grid)
    torch.cuda.synchronize()
    return f64(s), f64(prof)


@pytest.mark.parametrize("F,Hs,W,kk,H,std", [(2, 20, 25, 5, 2, 1.5), (1, 8, 32, 2, 1, 1.0),
                                             (3, 10, 13, 3, 2, 2.5), (2, 30, 7, 5, 1, 4.0),
                                             (1, 4, 150, 2, 1, 1.5)])
def test_similarity_matches_oracle(gpu, F, Hs, W, kk, H, std):
    N = F * Hs * W
    say(f"case similarity F={F} rows={Hs} cols={W} anchors={kk} H={H} std={std}")
    q = gaussian_bf16(300 + N, (H, N, 128), std=std).to(DEV)
    k = gaussian_bf16(301 + N, (H, N, 128)).to(DEV)
    scale = 1 / np.sqrt(128)
    s, prof = gpu_similarity(gpu, q, k, scale, (F, Hs, W, kk))
    for h in range(H):
        qb, kb = bf16_bits(q[h]), bf16_bits(k[h])
        want_p = oracle.row_profiles(qb, kb, scale, F, Hs, W)
        err = np.abs(prof[h] - want_p)
        assert (err <= 1e-4 * np.abs(want_p) + 1e-7).all(), f"head {h}: profile max err {err.max():.2e}"
        want_s = oracle.spatial_similarity(qb, kb, scale, F, Hs, W, kk)
        assert abs(s[h] - want_s) < 1e-5, (h, s[h], want_s)
        say(f"  head {h}: s {s[h]:.6f} (oracle {want_s:.6f})")


def test_similarity_closed_forms(gpu):
    say("case similarity closed forms")
    # one-hot attention (see the oracle pin): s = 4/6
    F, Hs, W = 1, 8, 32
    N = F * Hs * W
    pattern = [0, 0, 0, 1, 1, 0, 1, 1]
    k = torch.zeros(1, N, 128)
    k[0, :128, 0] = 1.0
    k[0, 128:, 1] = 1.0
    q = torch.zeros(1, N, 128)
    for y in range(Hs):
        q[0, y * W:(y + 1) * W, pattern[y]] = 64.0
    s, prof = gpu_similarity(gpu, q.to(torch.bfloat16).to(DEV), k.to(torch.bfloat16).to(DEV), 1.0,
                             (F, Hs, W, 2))
    np.testing.assert_allclose(prof[0], np.eye(2)[pattern], atol=1e-6)
    assert abs(s[0] - 4 / 6) < 1e-6
    # Q = 0: all profiles |J_c| / N, s = 1
    F, Hs, W = 2, 5, 40
    k = gaussian_bf16(320, (2, F * Hs * W, 128)).to(DEV)
    s, prof = gpu_similarity(gpu, torch.zeros_like(k), k, 0.1, (F, Hs, W, 2))
    np.testing.assert_allclose(prof, np.broadcast_to(np.array([128, 128, 128, 16]) / 400, prof.shape),
                               rtol=1e-6)
    np.testing.assert_allclose(s, 1.0, atol=1e-6)
    # every row an anchor: s = 1 exactly
    s, _ = gpu_similarity(gpu, gaussian_bf16(321, (1, 128, 128)).to(DEV),
                          gaussian_bf16(322, (1, 128, 128)).to(DEV), 0.1, (1, 4, 32, 4))
    assert s[0] == 1.0


def test_similarity_calibration_shape_small(gpu):
    """The small calibration recipe (low-rank positional code): one draw,
    every head against the oracle, then the classification at gamma."""
    w = CALIB_WORKLOADS["calibration_small"]
    g = w.grid
    grid = (g.frames, g.rows, g.cols, 5)
    say(f"case similarity calibration_small H={w.heads} N={w.n_tokens}")
    basis = calib_basis(w, "cpu")
    q, k = calib_draw(w, 0, basis, "cpu")
    s, _ = gpu_similarity(gpu, q.to(DEV), k.to(DEV), w.scale, grid)
    want = np.array([oracle.spatial_similarity(bf16_bits(q[h]), bf16_bits(k[h]), w.scale, *grid)
                     for h in range(w.heads)])
    np.testing.assert_allclose(s, want, atol=1e-5)
    assert np.array_equal(oracle.classify_repeat(s), oracle.classify_repeat(want)) or \
        np.min(np.abs(want - oracle.GAMMA)) < 1e-5
    say(f"  s = {np.round(s, 4).tolist()}")
