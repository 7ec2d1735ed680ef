"""Property-based tests (hypothesis) of the selection, binarisation and
kept-list rules on tiny rows, and of the host-side list validator, on
random inputs including ties and malformed lists. CPU only.

Rules ([CalibAtt blog] = the zhichai.net article on CalibAtt, §三 offline
calibration): the fewest blocks, largest energy first, whose cumulative
energy reaches eps; the mean of the selections over prompts binarised at
rho; static per-query-block lists of the kept blocks."""

import itertools

import numpy as np
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import calibrated_block_sparse_amd as cbs
import oracle

SETTINGS = settings(max_examples=150, deadline=None,
                    suppress_health_check=[HealthCheck.too_slow])

# energies as integer multiples of 2^-40 drawn from a small set, so ties are common
small_rows = st.lists(st.integers(min_value=0, max_value=6), min_size=1, max_size=7)


def as_energy(vals):
    x = np.asarray(vals, dtype=np.float64)
    s = x.sum()
    return x / s if s > 0 else x


@SETTINGS
@given(small_rows, st.integers(min_value=0, max_value=2 ** 40 + 5))
def test_greedy_is_minimal_and_top_ranked(vals, eps):
    """n* is the smallest subset size whose sum reaches eps (brute force over
    every subset), the selected set is the top n* by (energy desc, column
    asc), and when nothing reaches eps the whole row is selected."""
    e = as_energy(vals)
    efx = oracle.quantize_energy(e)
    sel, nstar = oracle.greedy_select(e[None, :], eps)
    sel, nstar = sel[0], int(nstar[0])
    R = len(vals)
    best = None
    for n in range(1, R + 1):
        if any(sum(int(efx[c]) for c in comb) >= eps for comb in itertools.combinations(range(R), n)):
            best = n
            break
    assert nstar == (best if best is not None else R)
    assert sel.sum() == nstar
    order = sorted(range(R), key=lambda c: (-int(efx[c]), c))
    assert set(np.flatnonzero(sel)) == set(order[:nstar])
    # the row-by-row and vectorised forms agree
    cols, n2 = oracle.greedy_select_row(efx, eps)
    assert n2 == nstar and set(cols) == set(order[:nstar])


@SETTINGS
@given(small_rows, st.integers(min_value=0, max_value=2 ** 40), st.integers(min_value=0, max_value=2 ** 39))
def test_larger_eps_selects_a_superset(vals, eps, extra):
    e = as_energy(vals)[None, :]
    lo, _ = oracle.greedy_select(e, eps)
    hi, _ = oracle.greedy_select(e, eps + extra)
    assert (hi >= lo).all()


votes_arrays = st.integers(min_value=1, max_value=6).flatmap(
    lambda R: st.tuples(st.integers(min_value=1, max_value=255), st.just(R),
                        st.lists(st.integers(0, 255), min_size=R * R, max_size=R * R)))


@SETTINGS
@given(votes_arrays, st.integers(1, 20), st.integers(1, 20))
def test_binarize_rule_fallback_and_monotone_in_rho(case, a, b):
    n, R, flat = case
    votes = np.minimum(np.asarray(flat, np.int64).reshape(1, R, R), n)
    num, den = min(a, b), max(a, b)
    keep = oracle.binarize(votes, n, num, den)
    rule = votes * den >= num * n
    for r in range(R):
        if rule[0, r].any():
            assert np.array_equal(keep[0, r].astype(bool), rule[0, r])
        else:  # exactly the most-voted column, the lowest on ties
            assert keep[0, r].sum() == 1 and keep[0, r, int(np.argmax(votes[0, r]))] == 1
    # a lower threshold keeps a superset of the rule's blocks
    lower = oracle.binarize(votes, n, max(num - 1, 0), den)
    assert (lower[rule] == 1).all()


masks = st.tuples(st.integers(1, 3), st.integers(1, 6)).flatmap(
    lambda hr: st.lists(st.integers(0, 1), min_size=hr[0] * hr[1] ** 2,
                        max_size=hr[0] * hr[1] ** 2).map(
        lambda v: np.asarray(v, np.uint8).reshape(hr[0], hr[1], hr[1])))


@SETTINGS
@given(masks)
def test_lists_round_trip_and_pass_the_validator(mask):
    H, R, _ = mask.shape
    off, idx = oracle.compile_skiplist(mask)
    assert off[0] == 0 and off[-1] == idx.size and (np.diff(off) >= 0).all()
    assert np.array_equal(oracle.skiplist_to_mask(off, idx, H, R), mask)
    cbs.calibatt_validate_skiplist(off, idx, H, R)          # the library's host check


@SETTINGS
@given(masks, st.data())
def test_validator_rejects_every_corruption(mask, data):
    """One corruption at a time (an offset moved outside [0, nnz] or made to
    decrease, an index out of range, two entries of a row out of order):
    the library's host validator reports a malformed list (and reads
    nothing outside the arrays it was given)."""
    H, R, _ = mask.shape
    off, idx = oracle.compile_skiplist(mask)
    off, idx = off.copy(), idx.copy()
    kind = data.draw(st.sampled_from(["offset_high", "offset_low", "index", "order"]))
    if kind == "offset_high":
        i = data.draw(st.integers(1, H * R - 1)) if H * R > 1 else None
        if i is None:
            return
        off[i] = idx.size + data.draw(st.integers(1, 50))
    elif kind == "offset_low":
        i = data.draw(st.integers(1, H * R))
        if off[i] == 0 and i < H * R:
            off[i] = -1
        elif off[i] > 0:
            off[i] = off[i - 1] - 1 if off[i - 1] > 0 else -1
        else:
            return
    elif kind == "index":
        if idx.size == 0:
            return
        j = data.draw(st.integers(0, idx.size - 1))
        idx[j] = data.draw(st.sampled_from([-1, R, R + 100]))
    else:
        rows = [r for r in range(H * R) if off[r + 1] - off[r] >= 2]
        if not rows:
            return
        r = data.draw(st.sampled_from(rows))
        idx[off[r]], idx[off[r] + 1] = idx[off[r] + 1], idx[off[r]]
    try:
        cbs.calibatt_validate_skiplist(off, idx, H, R)
    except cbs.CalibAttError as e:
        assert e.code == -3
    else:
        raise AssertionError(f"corruption {kind} accepted")


# ----------------------------------------------------------------------------
# The oracle's attention and block energy on random small heads: properties
# softmax attention has whatever the mask ([CalibAtt blog] §三 online
# inference: a query block attends to the keys of its kept blocks only).

ATT_SETTINGS = settings(max_examples=40, deadline=None,
                        suppress_health_check=[HealthCheck.too_slow])
heads = st.tuples(st.integers(min_value=1, max_value=400),      # N
                  st.integers(min_value=0, max_value=2 ** 31),    # seed
                  st.floats(min_value=0.0, max_value=1.0))        # keep probability


def _head(N, seed, p, D=16):
    rng = np.random.default_rng(seed)
    q, k, v = (rng.standard_normal((N, D)) for _ in range(3))
    R = (N + oracle.BLOCK - 1) // oracle.BLOCK
    mask = (rng.random((R, R)) < p).astype(np.uint8)
    return q, k, v, mask, 0.5 + rng.random()


@ATT_SETTINGS
@given(heads)
def test_sparse_attention_rows_are_convex_combinations_of_kept_values(h):
    """Every output row lies, coordinate by coordinate, between the least and
    the greatest value of V over the keys of its block-row's kept blocks;
    a block-row that keeps nothing is zero."""
    q, k, v, mask, scale = _head(*h)
    out = oracle.block_sparse_attention(q, k, v, scale, mask)
    N = q.shape[0]
    for r in range(mask.shape[0]):
        rows = slice(r * oracle.BLOCK, min((r + 1) * oracle.BLOCK, N))
        keys = oracle.kept_keys(np.flatnonzero(mask[r]), N)
        if keys.size == 0:
            assert not out[rows].any()
            continue
        lo, hi = v[keys].min(axis=0), v[keys].max(axis=0)
        assert (out[rows] >= lo - 1e-12).all() and (out[rows] <= hi + 1e-12).all()


@ATT_SETTINGS
@given(heads, st.floats(min_value=-3, max_value=3), st.floats(min_value=-3, max_value=3))
def test_sparse_attention_is_linear_in_the_values(h, a, b):
    q, k, v, mask, scale = _head(*h)
    v2 = np.random.default_rng(h[1] + 1).standard_normal(v.shape)
    lhs = oracle.block_sparse_attention(q, k, a * v + b * v2, scale, mask)
    rhs = a * oracle.block_sparse_attention(q, k, v, scale, mask) + \
        b * oracle.block_sparse_attention(q, k, v2, scale, mask)
    assert np.allclose(lhs, rhs, rtol=1e-10, atol=1e-10)


@ATT_SETTINGS
@given(heads)
def test_attention_and_energy_ignore_a_common_key_shift(h):
    """Adding one vector u to every key adds q_i.u to the whole score row i,
    which the softmax over keys removes: the outputs and the block energies
    are unchanged (a softmax taken over the wrong axis would not be)."""
    q, k, v, mask, scale = _head(*h)
    u = np.random.default_rng(h[1] + 2).standard_normal(k.shape[1])
    ks = k + u[None, :]
    assert np.allclose(oracle.block_sparse_attention(q, ks, v, scale, mask),
                       oracle.block_sparse_attention(q, k, v, scale, mask), rtol=1e-9, atol=1e-11)
    e0, e1 = oracle.block_energy(q, k, scale), oracle.block_energy(q, ks, scale)
    assert np.allclose(e0, e1, rtol=1e-9, atol=1e-13)
    assert np.allclose(e0.sum(axis=1), 1.0, atol=1e-12)
