"""Pins for the oracle's forward pass (CPU only).

Each check ties ``oracle.attention_forward`` to something other than itself:
a hand-derived fixture, closed forms, invariants of softmax attention, scipy
routines, and the pages' block recurrence written independently in
``oracle.online``.
"""

import json
import os

import numpy as np
import pytest
import scipy.special

from oracle import attention_forward, attention_probs, visibility
from oracle.online import tiled_forward_kv_outer, tiled_forward_q_outer

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _butterfly(nb):
    i = np.arange(nb)[:, None]
    j = np.arange(nb)[None, :]
    x = i ^ j
    return ((x == 0) | ((x & (x - 1)) == 0)).astype(np.uint8)


@pytest.mark.parametrize("causal", [False, True])
def test_two_token_fixture(causal):
    g = json.load(open(os.path.join(GOLDEN, "two_token_closed_form.json")))
    inp = g["inputs"]
    exp = g["causal" if causal else "noncausal"]
    q, k, v = (np.array(inp[n]) for n in ("q", "k", "v"))
    o, lse = attention_forward(q, k, v, inp["scale"], causal=causal)
    np.testing.assert_allclose(o[0, 0], exp["o"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse[0, 0], exp["lse"], rtol=0, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_probabilities_rows_sum_to_one_and_respect_mask(causal):
    rng = np.random.default_rng(1)
    n, d = 37, 8
    q, k = _rand(rng, n, d), _rand(rng, n, d)
    p, _ = attention_probs(q, k, 0.3, causal=causal)
    assert np.all(p >= 0)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    vis = visibility(np.arange(n), np.arange(n), causal)
    assert np.all(p[~vis] == 0)


def test_against_scipy_softmax_and_logsumexp():
    rng = np.random.default_rng(2)
    n, d = 50, 16
    q, k, v = _rand(rng, n, d), _rand(rng, n, d), _rand(rng, n, d)
    scale = 1 / np.sqrt(d)
    o, lse = attention_forward(q, k, v, scale)
    s = scale * q @ k.T
    np.testing.assert_allclose(lse[0, 0], scipy.special.logsumexp(s, axis=1), rtol=0, atol=1e-13)
    np.testing.assert_allclose(o[0, 0], scipy.special.softmax(s, axis=1) @ v, rtol=0, atol=1e-13)


def test_zero_queries_noncausal_gives_mean_of_values():
    rng = np.random.default_rng(3)
    n, d = 33, 5
    v = _rand(rng, n, d)
    o, lse = attention_forward(np.zeros((n, d)), _rand(rng, n, d), v, 0.125)
    np.testing.assert_allclose(o[0, 0], np.broadcast_to(v.mean(axis=0), (n, d)), atol=1e-14)
    np.testing.assert_allclose(lse[0, 0], np.log(n), atol=1e-14)


def test_zero_queries_causal_gives_prefix_mean():
    rng = np.random.default_rng(4)
    n, d = 40, 4
    v = _rand(rng, n, d)
    o, lse = attention_forward(np.zeros((n, d)), _rand(rng, n, d), v, 0.125, causal=True)
    prefix = np.cumsum(v, axis=0) / np.arange(1, n + 1)[:, None]
    np.testing.assert_allclose(o[0, 0], prefix, atol=1e-13)
    np.testing.assert_allclose(lse[0, 0], np.log(np.arange(1, n + 1)), atol=1e-14)


def test_zero_queries_block_mask_counts():
    rng = np.random.default_rng(5)
    mb, nb, d = 4, 16, 3
    n = mb * nb
    bm = _butterfly(nb)
    bm[2, 3] = 0  # drop one block so counts differ between rows
    v = _rand(rng, n, d)
    o, lse = attention_forward(np.zeros((n, d)), _rand(rng, n, d), v, 0.5,
                               block_mask=bm, mask_block=mb)
    for i in range(n):
        cols = [j for j in range(n) if bm[i // mb, j // mb]]
        np.testing.assert_allclose(o[0, 0, i], v[cols].mean(axis=0), atol=1e-14)
        np.testing.assert_allclose(lse[0, 0, i], np.log(len(cols)), atol=1e-14)


def test_single_token_output_is_value():
    rng = np.random.default_rng(6)
    q, k, v = _rand(rng, 1, 64), _rand(rng, 1, 64), _rand(rng, 1, 64)
    for causal in (False, True):
        o, lse = attention_forward(q, k, v, 0.125, causal=causal)
        np.testing.assert_array_equal(o[0, 0], v)
        np.testing.assert_allclose(lse[0, 0, 0], 0.125 * float(q[0] @ k[0]), atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_adding_constant_to_values_shifts_output(causal):
    rng = np.random.default_rng(7)
    n, d = 29, 6
    q, k, v = _rand(rng, n, d), _rand(rng, n, d), _rand(rng, n, d)
    c = _rand(rng, d)
    o1, l1 = attention_forward(q, k, v, 0.4, causal=causal)
    o2, l2 = attention_forward(q, k, v + c, 0.4, causal=causal)
    np.testing.assert_allclose(o2, o1 + c, atol=1e-13)
    np.testing.assert_array_equal(l1, l2)


def test_key_value_permutation_invariance_noncausal():
    rng = np.random.default_rng(8)
    n, d = 31, 7
    q, k, v = _rand(rng, n, d), _rand(rng, n, d), _rand(rng, n, d)
    perm = rng.permutation(n)
    o1, l1 = attention_forward(q, k, v, 0.3)
    o2, l2 = attention_forward(q, k[perm], v[perm], 0.3)
    np.testing.assert_allclose(o1, o2, atol=1e-13)
    np.testing.assert_allclose(l1, l2, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_shift_invariance_of_row_scores(causal):
    """Adding the same vector c to every key adds scale*q_i.c to every score of
    row i: P and O are unchanged, LSE_i moves by exactly that amount."""
    rng = np.random.default_rng(9)
    n, d = 23, 5
    q, k, v = _rand(rng, n, d), _rand(rng, n, d), _rand(rng, n, d)
    c = 3.0 * _rand(rng, d)
    o1, l1 = attention_forward(q, k, v, 0.5, causal=causal)
    o2, l2 = attention_forward(q, k + c, v, 0.5, causal=causal)
    np.testing.assert_allclose(o1, o2, atol=1e-12)
    np.testing.assert_allclose(l2[0, 0] - l1[0, 0], 0.5 * q @ c, atol=1e-12)


def test_causal_rows_ignore_future_keys():
    rng = np.random.default_rng(10)
    n, d = 30, 4
    q, k, v = _rand(rng, n, d), _rand(rng, n, d), _rand(rng, n, d)
    o1, l1 = attention_forward(q, k, v, 0.5, causal=True)
    k2, v2 = k.copy(), v.copy()
    k2[20:] += 100.0
    v2[20:] -= 7.0
    o2, l2 = attention_forward(q, k2, v2, 0.5, causal=True)
    np.testing.assert_array_equal(o1[0, 0, :20], o2[0, 0, :20])
    np.testing.assert_array_equal(l1[0, 0, :20], l2[0, 0, :20])
    assert np.abs(o1[0, 0, 20:] - o2[0, 0, 20:]).max() > 1e-3


def test_fully_masked_row_is_zero_with_minus_inf_lse():
    rng = np.random.default_rng(11)
    mb, nb, d = 2, 4, 3
    n = mb * nb
    bm = np.ones((nb, nb), np.uint8)
    bm[1, :] = 0
    q, k, v = _rand(rng, n, d), _rand(rng, n, d), _rand(rng, n, d)
    o, lse = attention_forward(q, k, v, 1.0, block_mask=bm, mask_block=mb)
    assert np.all(o[0, 0, 2:4] == 0)
    assert np.all(np.isneginf(lse[0, 0, 2:4]))
    assert np.all(np.isfinite(lse[0, 0, :2])) and np.all(np.isfinite(lse[0, 0, 4:]))


@pytest.mark.parametrize("causal,masked", [(False, False), (True, False), (False, True), (True, True)])
@pytest.mark.parametrize("br,bc", [(1, 1), (3, 5), (5, 3), (7, 7), (40, 40), (40, 1), (1, 40)])
def test_block_recurrence_both_orders_equal_one_shot(causal, masked, br, bc):
    """The pages' online-softmax recurrence, in both loop orders and for tile
    sizes that do and do not divide N (B_c = 1 is the serial online softmax),
    reproduces the one-shot definition."""
    rng = np.random.default_rng(100 + br * 7 + bc)
    n, d = 40, 6
    q, k, v = 2 * _rand(rng, n, d), 2 * _rand(rng, n, d), _rand(rng, n, d)
    bm = None
    mb = 4
    if masked:
        bm = _butterfly(n // mb)
    o_ref, l_ref = attention_forward(q, k, v, 0.7, causal=causal, block_mask=bm, mask_block=mb)
    for fn in (tiled_forward_kv_outer, tiled_forward_q_outer):
        o, lse = fn(q, k, v, 0.7, br, bc, causal=causal, block_mask=bm, mask_block=mb)
        np.testing.assert_allclose(o, o_ref[0, 0], rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse, l_ref[0, 0], rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_row_chunked_equals_single_pass(causal):
    rng = np.random.default_rng(12)
    n, d = 45, 6
    q, k, v = _rand(rng, 2, 3, n, d), _rand(rng, 2, 3, n, d), _rand(rng, 2, 3, n, d)
    o1, l1 = attention_forward(q, k, v, 0.3, causal=causal, row_chunk=n)
    for chunk in (1, 4, 7):
        o2, l2 = attention_forward(q, k, v, 0.3, causal=causal, row_chunk=chunk)
        np.testing.assert_allclose(o1, o2, atol=1e-14)
        np.testing.assert_allclose(l1, l2, atol=1e-14)


def test_block_sparse_column_gather_equals_dense_masking():
    """The gathered evaluation (only kept key blocks are touched) matches a
    dense evaluation over all N columns with the mask applied as -inf."""
    rng = np.random.default_rng(13)
    mb, nb, d = 4, 16, 5
    n = mb * nb
    bm = _butterfly(nb)
    q, k, v = _rand(rng, n, d), _rand(rng, n, d), _rand(rng, n, d)
    o, lse = attention_forward(q, k, v, 0.6, block_mask=bm, mask_block=mb)
    s = 0.6 * q @ k.T
    keep = np.kron(bm, np.ones((mb, mb))) != 0
    s = np.where(keep, s, -np.inf)
    np.testing.assert_allclose(lse[0, 0], scipy.special.logsumexp(s, axis=1), atol=1e-13)
    np.testing.assert_allclose(o[0, 0], scipy.special.softmax(s, axis=1) @ v, atol=1e-13)


def test_heads_selection_matches_full():
    rng = np.random.default_rng(14)
    q, k, v = _rand(rng, 2, 3, 16, 4), _rand(rng, 2, 3, 16, 4), _rand(rng, 2, 3, 16, 4)
    o, lse = attention_forward(q, k, v, 0.5, causal=True)
    sel = [(1, 2), (0, 1)]
    o2, l2 = attention_forward(q, k, v, 0.5, causal=True, heads=sel)
    for t, (b, h) in enumerate(sel):
        np.testing.assert_array_equal(o2[t], o[b, h])
        np.testing.assert_array_equal(l2[t], lse[b, h])
