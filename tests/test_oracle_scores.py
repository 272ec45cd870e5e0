"""Pins for the oracle's observation-window scores (SnapKV scoring named on the
citation-map page and in the companion page's "Two Ingredients, Fused").

Each test checks the oracle against something other than itself: a closed
form, an invariant, a library softmax, or a 50-digit brute force."""
import itertools

import mpmath
import numpy as np
import pytest
from scipy.special import softmax

from oracle import obs_column_scores


def _rand(rng, *shape):
    return rng.standard_normal(shape)


@pytest.mark.parametrize("G,W,L", [(1, 1, 7), (2, 4, 30), (4, 16, 512)])
def test_zero_queries_closed_form(G, W, L):
    # q = 0 -> every visible logit is 0 -> row r is uniform over its L-W+r+1
    # visible keys, so key i collects G * sum over rows that see it of 1/(L-W+r+1).
    rng = np.random.default_rng(1)
    d = 8
    col = obs_column_scores(np.zeros((G, W, d)), _rand(rng, L, d), 0.3)
    expect = np.zeros(L)
    for i in range(L):
        for r in range(W):
            if i <= L - W + r:
                expect[i] += G / (L - W + r + 1)
    np.testing.assert_allclose(col, expect, rtol=1e-13, atol=0)


@pytest.mark.parametrize("seed", range(4))
def test_column_sum_is_G_times_W(seed):
    # each softmax row sums to one -> all columns together sum to G*W
    rng = np.random.default_rng(seed)
    G, W, L, d = 3, 5, 200, 16
    col = obs_column_scores(_rand(rng, G, W, d), 2.0 * _rand(rng, L, d), 1 / np.sqrt(d))
    assert abs(col.sum() - G * W) < 1e-12 * G * W
    assert (col >= 0).all()


def test_single_row_equals_library_softmax():
    # G = W = 1: the only observation query is the last prompt position and
    # sees every key, so the column scores are exactly that row's softmax.
    rng = np.random.default_rng(5)
    L, d, scale = 64, 16, 0.25
    q, k = _rand(rng, 1, 1, d), _rand(rng, L, d)
    col = obs_column_scores(q, k, scale)
    np.testing.assert_allclose(col, softmax(scale * k @ q[0, 0]), rtol=1e-13)


def test_causal_visibility_of_window_keys():
    # G = 1, W = 2: the last key is visible only to the last row; row 0 sees
    # keys 0..L-2.  So col = softmax_row1 + [softmax_row0 over L-1 keys, 0].
    rng = np.random.default_rng(6)
    L, d, scale = 40, 8, 0.5
    q, k = _rand(rng, 1, 2, d), _rand(rng, L, d)
    col = obs_column_scores(q, k, scale)
    row0 = np.append(softmax(scale * k[:-1] @ q[0, 0]), 0.0)
    row1 = softmax(scale * k @ q[0, 1])
    np.testing.assert_allclose(col, row0 + row1, rtol=1e-13)


def test_dominant_key_takes_all_mass():
    # A key of huge norm aligned with every query takes (almost) all the
    # probability of every row: its score tends to G*W.
    rng = np.random.default_rng(7)
    G, W, L, d = 2, 4, 50, 8
    u = np.zeros(d)
    u[0] = 1.0
    q = 0.1 * _rand(rng, G, W, d)
    q[..., 0] = 1.0
    k = _rand(rng, L, d)
    k[20] = 400.0 * u
    col = obs_column_scores(q, k, 1 / np.sqrt(d))
    assert col[20] > G * W * (1 - 1e-9)
    assert col[20] <= G * W * (1 + 1e-12)


def _brute_force_mp(q, k, scale):
    """50-digit evaluation with explicit loops: for every head g and window row
    r, probability of key i = exp(z_i) / sum over visible keys exp(z_j)."""
    mpmath.mp.dps = 50
    G, W, d = q.shape
    L = k.shape[0]
    col = [mpmath.mpf(0)] * L
    for g, r in itertools.product(range(G), range(W)):
        last = L - W + r
        logits = []
        for i in range(last + 1):
            acc = mpmath.mpf(0)
            for t in range(d):
                acc += mpmath.mpf(float(q[g, r, t])) * mpmath.mpf(float(k[i, t]))
            logits.append(mpmath.mpf(float(scale)) * acc)
        den = mpmath.fsum(mpmath.exp(z) for z in logits)
        for i, z in enumerate(logits):
            col[i] += mpmath.exp(z) / den
    return np.array([float(c) for c in col])


@pytest.mark.parametrize("G,W,L,d", [(1, 1, 9, 2), (2, 3, 17, 4), (2, 4, 33, 2), (1, 4, 12, 4)])
def test_brute_force_50_digits(G, W, L, d):
    rng = np.random.default_rng(100 + L)
    q, k = 1.5 * _rand(rng, G, W, d), 1.5 * _rand(rng, L, d)
    scale = 1 / np.sqrt(d)
    np.testing.assert_allclose(obs_column_scores(q, k, scale), _brute_force_mp(q, k, scale),
                               rtol=1e-12, atol=1e-300)


def test_query_heads_are_summed_not_averaged():
    # two identical q-heads give exactly twice the single-head scores
    rng = np.random.default_rng(8)
    q, k = _rand(rng, 1, 3, 4), _rand(rng, 20, 4)
    one = obs_column_scores(q, k, 0.5)
    two = obs_column_scores(np.concatenate([q, q]), k, 0.5)
    np.testing.assert_allclose(two, 2 * one, rtol=1e-14)
