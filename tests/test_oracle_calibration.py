"""Pins of the calibration oracle: block energy against an explicit
softmax matrix and closed forms, greedy selection against brute force over
all subsets, the eps(t) schedule against the differential equation it
solves, binarisation and kept-list compilation against hand-worked cases.

Sources: [CalibAtt blog] = the zhichai.net article on CalibAtt, §三 offline
calibration (energy E_{r,c}, greedy selection to eps(t), mean over prompts
binarised at rho = 0.5, eps(t) = A + (C - A) exp(-k t / T))."""

import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")
FX = 2 ** 40


def rnd(seed, *shape):
    return np.random.Generator(np.random.PCG64(seed)).standard_normal(shape)


# ---------------------------------------------------------------- energy


@pytest.mark.parametrize("N", [1024, 1000, 200])
def test_energy_rows_sum_to_one_and_nonnegative(N):
    q, k = rnd(1, N, 128) * 2, rnd(2, N, 128)
    E = oracle.block_energy(q, k, 1 / math.sqrt(128))
    assert (E >= 0).all()
    np.testing.assert_allclose(E.sum(axis=1), 1.0, rtol=0, atol=1e-12)


def test_energy_zero_queries_closed_form():
    """Q = 0: P_ij = 1/N, so E_rc = |J_c| / N for every row (ragged last
    block has N mod 128 keys)."""
    N = 1000
    E = oracle.block_energy(np.zeros((N, 128)), rnd(3, N, 128), 0.1)
    want = np.array([128] * 7 + [104]) / N
    np.testing.assert_allclose(E, np.broadcast_to(want, E.shape), rtol=1e-13)


def test_energy_vs_explicit_softmax_matrix():
    """E from torch's softmax of the full fp64 score matrix, summed block by
    block with plain loops (tiny, ragged shape)."""
    N = 300
    q, k = rnd(4, N, 128), rnd(5, N, 128)
    P = torch.softmax(torch.from_numpy(q) @ torch.from_numpy(k).T * 0.15, dim=1).numpy()
    R = 3
    want = np.zeros((R, R))
    for r in range(R):
        rows = range(r * 128, min(r * 128 + 128, N))
        for c in range(R):
            want[r, c] = sum(P[i, j] for i in rows for j in range(c * 128, min(c * 128 + 128, N))) / len(rows)
    np.testing.assert_allclose(oracle.block_energy(q, k, 0.15), want, rtol=1e-11, atol=1e-15)


def test_energy_full_rows_use_block_size():
    """For full block-rows 1/|I_r| is the pages' 1/B with B = 128."""
    const = json.load(open(os.path.join(GOLD, "paper_constants.json")))
    N = 256
    q, k = rnd(6, N, 128), rnd(7, N, 128)
    P = torch.softmax(torch.from_numpy(q) @ torch.from_numpy(k).T * 0.1, dim=1).numpy()
    E = oracle.block_energy(q, k, 0.1)
    assert abs(E[1, 0] - P[128:, :128].sum() / const["block_size"]) < 1e-13


# ---------------------------------------------------------------- quantisation


def test_quantize_is_round_half_even_exact():
    vals = np.array([2.0 ** -41, 3 * 2.0 ** -41, 5 * 2.0 ** -41, 1.0, 0.0], dtype=np.float64)
    assert list(oracle.quantize_energy(vals)) == [0, 2, 2, FX, 0]
    rng = np.random.Generator(np.random.PCG64(8))
    f32 = rng.random(2000).astype(np.float32) ** 6
    want = [round(Fraction(float(x)) * FX) for x in f32]  # Python rounds Fractions half-to-even
    assert list(oracle.quantize_energy(f32)) == want


# ---------------------------------------------------------------- greedy


def brute_force(e, eps):
    """Smallest n such that SOME n-subset reaches eps (exhaustive)."""
    R = len(e)
    for n in range(1, R + 1):
        if any(sum(e[c] for c in sub) >= eps for sub in itertools.combinations(range(R), n)):
            return n
    return R


@pytest.mark.parametrize("kind", ["dirichlet", "peaky", "ties"])
def test_greedy_minimal_by_brute_force(kind):
    from synth import energy_rows
    E = energy_rows(9, 3, 8, kind)
    for eps in (0.5, 0.84, 0.9, 0.99, 1.0):
        efx = oracle.eps_fx(eps)
        sel, nstar = oracle.greedy_select(E, efx)
        for h in range(3):
            for r in range(8):
                e = oracle.quantize_energy(E[h, r])
                n = brute_force(list(e), efx)
                if sum(e) >= efx:
                    assert nstar[h, r] == n
                    chosen = np.flatnonzero(sel[h, r])
                    assert len(chosen) == n and e[chosen].sum() >= efx
                    # tie rule: the chosen set is a top-n set, lowest columns first among equals
                    thr = np.sort(e)[::-1][n - 1]
                    assert (e[chosen] >= thr).all()
                    eq = np.flatnonzero(e == thr)
                    assert list(np.intersect1d(chosen, eq)) == list(eq[:len(np.intersect1d(chosen, eq))])
                else:
                    assert nstar[h, r] == 8 and sel[h, r].all()


def test_greedy_vectorised_matches_row_loop():
    from synth import energy_rows
    E = energy_rows(10, 2, 40, "ties")
    efx = oracle.eps_fx(0.9)
    sel, nstar = oracle.greedy_select(E, efx)
    for h in range(2):
        for r in range(40):
            cols, n = oracle.greedy_select_row(oracle.quantize_energy(E[h, r]), efx)
            assert n == nstar[h, r]
            assert sorted(cols) == list(np.flatnonzero(sel[h, r]))


def test_greedy_special_cases():
    R = 16
    onehot = np.zeros((1, R), np.float32)
    onehot[0, 5] = 1.0
    s, n = oracle.greedy_select(onehot, oracle.eps_fx(0.99))
    assert n[0] == 1 and np.flatnonzero(s[0]).tolist() == [5]
    # uniform row e_c = u: n* = ceil(eps_fx / u)
    u = 1.0 / R
    for eps in (0.3, 0.5, 0.84, 0.99):
        efx = oracle.eps_fx(eps)
        s, n = oracle.greedy_select(np.full((1, R), u, np.float32), efx)
        ufx = int(u * FX)
        assert n[0] == -(-efx // ufx)
        assert np.flatnonzero(s[0]).tolist() == list(range(n[0]))   # ties -> lowest columns
    # eps at or below the largest energy -> one block
    row = np.array([[0.05, 0.6, 0.35]], np.float32)
    assert oracle.greedy_select(row, oracle.eps_fx(0.6))[1][0] == 1
    # eps above the row sum -> every block
    assert oracle.greedy_select(row * 0.5, oracle.eps_fx(0.9))[1][0] == 3


def test_greedy_agrees_with_real_arithmetic_away_from_threshold():
    from synth import energy_rows
    E = energy_rows(11, 4, 64, "dirichlet").astype(np.float64)
    eps = 0.9
    sel, nstar = oracle.greedy_select(E, oracle.eps_fx(eps))
    for h in range(4):
        for r in range(64):
            srt = np.sort(E[h, r])[::-1]
            cs = np.cumsum(srt)
            n_real = int(np.argmax(cs >= eps)) + 1 if cs[-1] >= eps else 64
            if min(abs(cs - eps)) > 1e-8:
                assert n_real == nstar[h, r]


# ---------------------------------------------------------------- eps(t)


def test_eps_schedule_properties():
    const = json.load(open(os.path.join(GOLD, "paper_constants.json")))
    A, C, k, T = const["eps_late"], const["eps_early"], 5.0, 50.0
    e = lambda t: float(oracle.eps_schedule(t, T, A, C, k))
    assert e(0) == pytest.approx(C, abs=1e-15)
    assert e(1e6) == pytest.approx(A, abs=1e-15)
    # half-way between C and A after t = T ln 2 / k
    assert e(T * math.log(2) / k) == pytest.approx((A + C) / 2, abs=1e-14)
    # solves d eps/dt = -(k/T)(eps - A): central differences
    for t in (3.0, 25.0, 49.0):
        h = 1e-4
        assert (e(t + h) - e(t - h)) / (2 * h) == pytest.approx(-(k / T) * (e(t) - A), rel=1e-6)
    ts = np.arange(50)
    assert np.all(np.diff(oracle.eps_schedule(ts, T, A, C, k)) < 0)


def test_eps_fx_rounding():
    assert oracle.eps_fx(0.5) == FX // 2
    assert oracle.eps_fx(1.0) == FX
    assert abs(oracle.eps_fx(0.84) - 0.84 * FX) <= 0.5


# ---------------------------------------------------------------- votes / binarise


def test_single_prompt_mask_is_its_selection():
    from synth import energy_rows
    E = energy_rows(12, 2, 16, "dirichlet")
    sel, _ = oracle.greedy_select(E, oracle.eps_fx(0.84))
    votes = oracle.accumulate_votes(sel[None])
    assert np.array_equal(oracle.binarize(votes, 1), sel)


def test_identical_prompts_reproduce_the_mask():
    from synth import energy_rows
    sel, _ = oracle.greedy_select(energy_rows(13, 2, 16, "peaky"), oracle.eps_fx(0.9))
    votes = oracle.accumulate_votes(np.stack([sel] * 64))
    assert votes.max() == 64
    assert np.array_equal(oracle.binarize(votes, 64), sel)


def test_rho_half_threshold_and_tie():
    votes = np.array([[[32, 31, 64, 0], [0, 0, 0, 0], [5, 9, 9, 2]]])
    m = oracle.binarize(votes, 64, 1, 2)
    assert m[0, 0].tolist() == [1, 0, 1, 0]           # 32/64 = rho is kept
    assert m[0, 1].tolist() == [1, 0, 0, 0]           # empty row: lowest of the maxima
    assert m[0, 2].tolist() == [0, 1, 0, 0]           # empty row: most-voted column
    m3 = oracle.binarize(votes, 64, 3, 10)            # rho = 0.3: votes >= 19.2
    assert m3[0, 0].tolist() == [1, 1, 1, 0]


# ---------------------------------------------------------------- compile


def test_compile_hand_example():
    mask = np.array([[[1, 0, 1], [0, 0, 0], [0, 1, 1]],
                     [[1, 1, 1], [0, 0, 1], [1, 0, 0]]], np.uint8)
    off, idx = oracle.compile_skiplist(mask)
    assert off.tolist() == [0, 2, 2, 4, 7, 8, 9]
    assert idx.tolist() == [0, 2, 1, 2, 0, 1, 2, 2, 0]


def test_compile_roundtrip():
    rng = np.random.Generator(np.random.PCG64(14))
    m = (rng.random((3, 37, 37)) < 0.3).astype(np.uint8)
    off, idx = oracle.compile_skiplist(m)
    assert np.array_equal(oracle.skiplist_to_mask(off, idx, 3, 37), m)
    for row in range(3 * 37):
        assert np.all(np.diff(idx[off[row]:off[row + 1]]) > 0)


# ----------------------------------------------------------------------------
# Spatial similarity (reading of [CalibAtt blog] §二 observation 4 / §三; the
# pages give no formula, so these pins tie the oracle to the stated reading).


def _onehot_case(pattern):
    """frames 1 x rows 8 x cols 32 (N = 256, two key blocks): every query of
    spatial row y points along unit direction e_{pattern[y]} with length 64,
    keys of block b are e_b, scale 1, so row y attends to block pattern[y]
    up to e^-64 and its profile is that one-hot vector."""
    F, Hs, W = 1, 8, 32
    N = F * Hs * W
    k = np.zeros((N, 128))
    k[:128, 0] = 1.0
    k[128:, 1] = 1.0
    q = np.zeros((N, 128))
    for y in range(Hs):
        q[y * W:(y + 1) * W, pattern[y]] = 64.0
    return q, k, (F, Hs, W)


def test_spatial_similarity_onehot_closed_form():
    # anchors 2 of 8 rows: A(m) = floor((2m+1)*8/4) = {2, 6}; rows 0-3 -> 2, 4-7 -> 6.
    # non-anchor rows 0,1,3,4,5,7 agree with their anchor's block in 4 cases.
    pattern = [0, 0, 0, 1, 1, 0, 1, 1]
    q, k, (F, Hs, W) = _onehot_case(pattern)
    assert list(oracle.anchor_rows(Hs, 2)) == [2, 6]
    prof = oracle.row_profiles(q, k, 1.0, F, Hs, W)
    np.testing.assert_allclose(prof, np.eye(2)[pattern], atol=1e-12)
    s = oracle.spatial_similarity(q, k, 1.0, F, Hs, W, 2)
    assert abs(s - 4 / 6) < 1e-12


def test_spatial_similarity_zero_queries_is_one():
    F, Hs, W = 2, 5, 40                       # N = 400, R = 4, last block 16 keys
    k = np.random.default_rng(3).standard_normal((F * Hs * W, 128))
    q = np.zeros_like(k)
    prof = oracle.row_profiles(q, k, 0.1, F, Hs, W)
    np.testing.assert_allclose(prof, np.broadcast_to(np.array([128, 128, 128, 16]) / 400, prof.shape),
                               atol=1e-15)
    assert abs(oracle.spatial_similarity(q, k, 0.1, F, Hs, W, 2) - 1.0) < 1e-12


def test_spatial_similarity_rows_alike_within_frames_is_one():
    F, Hs, W = 2, 6, 24
    rng = np.random.default_rng(4)
    k = rng.standard_normal((F * Hs * W, 128))
    base = rng.standard_normal((F, 1, W, 128))
    q = np.broadcast_to(base, (F, Hs, W, 128)).reshape(-1, 128)
    assert abs(oracle.spatial_similarity(q, k, 0.2, F, Hs, W, 3) - 1.0) < 1e-12


def test_spatial_similarity_every_row_an_anchor():
    F, Hs, W = 1, 4, 32
    rng = np.random.default_rng(5)
    q, k = rng.standard_normal((2, F * Hs * W, 128))
    assert list(oracle.anchor_of_row(Hs, Hs)) == list(range(Hs))
    assert oracle.spatial_similarity(q, k, 0.1, F, Hs, W, Hs) == 1.0


def test_spatial_similarity_bounds_and_profile_sums():
    F, Hs, W = 2, 6, 30
    rng = np.random.default_rng(6)
    q, k = rng.standard_normal((2, F * Hs * W, 128)) * 1.5
    prof = oracle.row_profiles(q, k, 0.3, F, Hs, W)
    np.testing.assert_allclose(prof.sum(axis=1), 1.0, atol=1e-12)
    assert (prof >= 0).all()
    s = oracle.spatial_similarity(q, k, 0.3, F, Hs, W, 2)
    assert 0.0 < s < 1.0


def test_classify_repeat_is_strictly_above_gamma():
    assert oracle.GAMMA == 0.87
    got = oracle.classify_repeat([0.86, 0.87, np.nextafter(0.87, 1.0), 0.99])
    assert got.tolist() == [0, 0, 1, 1] and got.dtype == np.uint8
