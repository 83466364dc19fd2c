"""Pins of the oracle for queries at an offset in the key sequence (the
decode shape: a few queries against many keys).  CPU only.

Each pin is fixed by something other than the oracle's own code: the Q = 0
closed forms (mean of the visible values, log of their count), scipy's
softmax for a single query, and the statement that decoding the last rows
equals those rows of the square problem (whose oracle is pinned by the
closed forms and finite differences of test_oracle_forward/backward).
"""

import numpy as np
import pytest
from scipy.special import logsumexp, softmax

from oracle import attention_forward


def _rand(*shape, seed=0):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("causal,window", [(True, 0), (False, 0), (True, 5), (False, 7)])
@pytest.mark.parametrize("nk,nq", [(37, 1), (37, 4), (9, 9), (64, 3)])
def test_zero_queries_average_visible_values(causal, window, nk, nq):
    """Q = 0 makes every visible score 0: O_i is the mean of the visible V rows
    and LSE_i = ln(#visible), with visibility taken at position nk - nq + i."""
    d = 8
    q = np.zeros((nq, d))
    k, v = _rand(nk, d, seed=1), _rand(nk, d, seed=2)
    o, lse = attention_forward(q, k, v, 0.3, causal=causal, window=window, q_offset=nk - nq)
    for i in range(nq):
        pos = nk - nq + i
        lo = max(0, pos - window + 1) if window else 0
        hi = pos if causal else (min(nk - 1, pos + window - 1) if window else nk - 1)
        np.testing.assert_allclose(o[0, 0, i], v[lo:hi + 1].mean(axis=0), rtol=0, atol=1e-14)
        assert abs(lse[0, 0, i] - np.log(hi - lo + 1)) < 1e-14


@pytest.mark.parametrize("causal", [True, False])
def test_single_query_is_a_softmax_over_all_keys(causal):
    """The last position sees every key, causal or not: O = softmax(s q K^T) V."""
    nk, d, scale = 50, 16, 0.25
    q, k, v = _rand(1, d, seed=3), _rand(nk, d, seed=4), _rand(nk, d, seed=5)
    o, lse = attention_forward(q, k, v, scale, causal=causal, q_offset=nk - 1)
    s = scale * (q @ k.T)[0]
    np.testing.assert_allclose(o[0, 0, 0], softmax(s) @ v, rtol=1e-13, atol=1e-14)
    assert abs(lse[0, 0, 0] - logsumexp(s)) < 1e-13


@pytest.mark.parametrize("causal,window", [(True, 0), (True, 6), (False, 4)])
def test_last_rows_of_the_square_problem(causal, window):
    """Decoding the last nq positions = the last nq rows of the square case,
    also with grouped K/V heads."""
    nk, nq, d, scale = 40, 5, 8, 0.35
    qf = _rand(2, 4, nk, d, seed=6)
    k, v = _rand(2, 2, nk, d, seed=7), _rand(2, 2, nk, d, seed=8)
    o_full, lse_full = attention_forward(qf, k, v, scale, causal=causal, window=window)
    o, lse = attention_forward(qf[:, :, -nq:], k, v, scale, causal=causal, window=window,
                               q_offset=nk - nq)
    np.testing.assert_allclose(o, o_full[:, :, -nq:], rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, lse_full[:, :, -nq:], rtol=0, atol=1e-13)


def test_offset_moves_the_causal_boundary():
    """A planted mistake of ignoring the offset would let query 0 (position
    nk - nq) see only key 0; it must see keys 0 .. nk - nq."""
    nk, nq, d = 12, 3, 4
    q = np.zeros((nq, d))
    k = _rand(nk, d, seed=9)
    v = np.arange(nk, dtype=np.float64)[:, None] * np.ones((1, d))
    o, lse = attention_forward(q, k, v, 1.0, causal=True, q_offset=nk - nq)
    assert abs(o[0, 0, 0, 0] - (nk - nq) / 2.0) < 1e-14
    assert abs(lse[0, 0, 0] - np.log(nk - nq + 1)) < 1e-14


def test_negative_offset_rejected():
    with pytest.raises(ValueError):
        attention_forward(np.zeros((2, 4)), np.zeros((3, 4)), np.zeros((3, 4)), 1.0, q_offset=-1)
