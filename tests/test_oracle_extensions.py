"""Pins for the oracle's sliding window, grouped K/V heads and dropout (CPU only).

Each check ties the oracle to something other than itself: published
known-answer vectors of the generator, closed forms, a different route to the
same value (a sliced sequence, repeated K/V heads), binomial bounds on the
keep rate, and central finite differences of the gradient.
"""

import json
import os

import numpy as np
import pytest

from oracle import attention_backward, attention_forward
from oracle.online import tiled_forward_kv_outer, tiled_forward_q_outer
from oracle.philox import dropout_keep, philox4x32_10

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(rng, *shape):
    return rng.standard_normal(shape)


# ---------------------------------------------------------------- generator


def test_philox_known_answer_vectors():
    kat = json.load(open(os.path.join(GOLDEN, "philox4x32_10_kat.json")))
    for case in kat["cases"]:
        c = [int(x, 16) for x in case["ctr"]]
        k = [int(x, 16) for x in case["key"]]
        out = philox4x32_10(*c, *k)
        assert [int(x) for x in out] == [int(x, 16) for x in case["out"]]


def test_philox_vectorised_equals_scalar_calls():
    rng = np.random.default_rng(5)
    c = rng.integers(0, 2**32, size=(4, 50), dtype=np.uint64)
    k = rng.integers(0, 2**32, size=2, dtype=np.uint64)
    vec = philox4x32_10(*c, *k)
    for t in range(50):
        one = philox4x32_10(*(int(x[t]) for x in c), int(k[0]), int(k[1]))
        assert [int(w[t]) for w in vec] == [int(w) for w in one]


@pytest.mark.parametrize("p", [0.0, 0.1, 0.25, 0.5, 0.9])
def test_keep_rate_within_binomial_bound(p):
    n = 1024
    keep, mult = dropout_keep(np.arange(n), np.arange(n), 3, 0x1234_5678_9ABC, 7, p)
    t8 = int(np.floor(p * 256))
    q = 1.0 - t8 / 256.0
    assert mult == pytest.approx(1.0 / q)
    frac = keep.mean()
    sigma = np.sqrt(q * (1 - q) / keep.size)
    assert abs(frac - q) <= 6 * sigma + 1e-12
    if p == 0.0:
        assert keep.all()


def test_keep_mask_depends_on_every_counter_field():
    base = dropout_keep(np.arange(64), np.arange(64), 2, 99, 5, 0.5)[0]
    for args in ((3, 99, 5), (2, 100, 5), (2, 99, 6), (2, 99 + (1 << 32), 5)):
        other = dropout_keep(np.arange(64), np.arange(64), args[0], args[1], args[2], 0.5)[0]
        assert (other != base).mean() > 0.3
    sub = dropout_keep(np.arange(8, 24), np.arange(40, 60), 2, 99, 5, 0.5)[0]
    assert np.array_equal(sub, base[8:24, 40:60])


def test_keep_bytes_of_a_block_are_one_generator_output():
    """The 16 (query, key) pairs of an aligned 4 x 4 block take the 16 bytes of
    one generator call, each once: with threshold t every byte value >= t is
    kept, so sweeping t over 0..255 recovers the multiset of bytes."""
    rows, cols = np.arange(8, 12), np.arange(20, 24)
    words = philox4x32_10(20 >> 2, 8 >> 2, 4, 9, 77, 0)
    want = sorted((int(w) >> (8 * b)) & 0xFF for w in words for b in range(4))
    kept_count = [int(dropout_keep(rows, cols, 4, 77, 9, t / 256.0)[0].sum())
                  for t in range(257) if t < 256]
    got = sorted(t for t in range(256) for _ in range(kept_count[t] - (kept_count[t + 1]
                                                                       if t < 255 else 0)))
    assert got == want


# ------------------------------------------------------------------ window


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("w", [1, 3, 8])
def test_window_zero_queries_counts(causal, w):
    """Q = 0 makes every visible score equal, so LSE_i = log(#visible keys)
    and O_i is the mean of the visible values."""
    n, d = 21, 3
    rng = np.random.default_rng(w)
    v = _rand(rng, n, d)
    o, lse = attention_forward(np.zeros((n, d)), _rand(rng, n, d), v, 0.5, causal=causal,
                               window=w)
    for i in range(n):
        lo = max(0, i - w + 1)
        hi = i + 1 if causal else min(n, i + w)
        assert lse[0, 0, i] == pytest.approx(np.log(hi - lo), abs=1e-14)
        np.testing.assert_allclose(o[0, 0, i], v[lo:hi].mean(axis=0), rtol=0, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_window_equals_attention_over_the_slice(causal):
    """Row i under a window W sees exactly keys max(0, i-W+1) .. i (causal) or
    .. i+W-1 (not causal): unmasked attention restricted to that slice."""
    rng = np.random.default_rng(33)
    n, d, w = 30, 5, 6
    q, k, v = _rand(rng, n, d), _rand(rng, n, d), _rand(rng, n, d)
    o, lse = attention_forward(q, k, v, 0.6, causal=causal, window=w)
    for i in range(n):
        lo = max(0, i - w + 1)
        hi = i + 1 if causal else min(n, i + w)
        s = 0.6 * k[lo:hi] @ q[i]
        e = np.exp(s - s.max())
        np.testing.assert_allclose(o[0, 0, i], e @ v[lo:hi] / e.sum(), rtol=0, atol=1e-13)
        assert lse[0, 0, i] == pytest.approx(s.max() + np.log(e.sum()), abs=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_window_wider_than_sequence_is_no_window(causal):
    rng = np.random.default_rng(2)
    q, k, v = (_rand(rng, 1, 2, 17, 4) for _ in range(3))
    a = attention_forward(q, k, v, 0.4, causal=causal, window=17)
    b = attention_forward(q, k, v, 0.4, causal=causal)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("br,bc", [(4, 4), (5, 3), (7, 11)])
def test_window_block_recurrence_equals_one_shot(causal, br, bc):
    rng = np.random.default_rng(br * 13 + bc)
    n, d, w = 37, 4, 9
    q, k, v = 2 * _rand(rng, n, d), 2 * _rand(rng, n, d), _rand(rng, n, d)
    o_ref, l_ref = attention_forward(q, k, v, 0.7, causal=causal, window=w, row_chunk=5)
    for fn in (tiled_forward_kv_outer, tiled_forward_q_outer):
        o, lse = fn(q, k, v, 0.7, br, bc, causal=causal, window=w)
        np.testing.assert_allclose(o, o_ref[0, 0], rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse, l_ref[0, 0], rtol=0, atol=1e-13)


# -------------------------------------------------------------- grouped K/V


@pytest.mark.parametrize("hkv", [1, 2, 6])
def test_grouped_heads_equal_repeated_kv(hkv):
    rng = np.random.default_rng(hkv)
    b, h, n, d = 2, 6, 19, 4
    q, do = _rand(rng, b, h, n, d), _rand(rng, b, h, n, d)
    k, v = _rand(rng, b, hkv, n, d), _rand(rng, b, hkv, n, d)
    g = h // hkv
    kr, vr = np.repeat(k, g, axis=1), np.repeat(v, g, axis=1)
    o, lse = attention_forward(q, k, v, 0.5, causal=True)
    o2, lse2 = attention_forward(q, kr, vr, 0.5, causal=True)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, lse2)
    dq, dk, dv = attention_backward(q, k, v, do, 0.5, causal=True)
    dq2, dk2, dv2 = attention_backward(q, kr, vr, do, 0.5, causal=True)
    np.testing.assert_array_equal(dq, dq2)
    assert dk.shape == k.shape and dv.shape == v.shape
    for got, full in ((dk, dk2), (dv, dv2)):
        want = np.stack([full[:, j * g:(j + 1) * g].sum(axis=1) for j in range(hkv)], axis=1)
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-13)


def test_grouped_heads_selection_gives_per_head_contribution():
    rng = np.random.default_rng(8)
    q, do = _rand(rng, 1, 4, 9, 3), _rand(rng, 1, 4, 9, 3)
    k, v = _rand(rng, 1, 2, 9, 3), _rand(rng, 1, 2, 9, 3)
    dq, dk, dv = attention_backward(q, k, v, do, 0.5)
    sel = attention_backward(q, k, v, do, 0.5, heads=[(0, 2), (0, 3)])
    np.testing.assert_array_equal(sel[0], dq[0, 2:4])
    np.testing.assert_allclose(sel[1].sum(axis=0), dk[0, 1], rtol=0, atol=1e-14)
    np.testing.assert_allclose(sel[2].sum(axis=0), dv[0, 1], rtol=0, atol=1e-14)


def test_grouped_heads_reject_non_divisor():
    x = np.zeros((1, 3, 4, 2))
    with pytest.raises(ValueError):
        attention_forward(x, np.zeros((1, 2, 4, 2)), np.zeros((1, 2, 4, 2)), 1.0)


# ----------------------------------------------------------------- dropout


def test_dropout_zero_is_plain_attention():
    rng = np.random.default_rng(1)
    q, k, v, do = (_rand(rng, 1, 2, 13, 4) for _ in range(4))
    a = attention_forward(q, k, v, 0.5, causal=True, dropout_p=0.0, seed=5)
    b = attention_forward(q, k, v, 0.5, causal=True)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
    ga = attention_backward(q, k, v, do, 0.5, causal=True, dropout_p=0.0, seed=5)
    gb = attention_backward(q, k, v, do, 0.5, causal=True)
    for x, y in zip(ga, gb):
        np.testing.assert_array_equal(x, y)


def test_dropout_leaves_lse_and_is_unbiased():
    """LSE does not see dropout; averaged over seeds the output approaches the
    undropped output (the 1/(1-p) scaling makes it unbiased)."""
    rng = np.random.default_rng(4)
    n, d = 16, 4
    q, k, v = _rand(rng, n, d), _rand(rng, n, d), _rand(rng, n, d)
    o0, l0 = attention_forward(q, k, v, 0.5)
    acc = np.zeros_like(o0)
    seeds = 400
    for s in range(seeds):
        o, lse = attention_forward(q, k, v, 0.5, dropout_p=0.25, seed=s)
        np.testing.assert_array_equal(lse, l0)
        acc += o
    mean = acc / seeds
    # Per element the dropped output has variance <= (p/(1-p)) sum_j P_ij^2 v_j^2.
    p, _ = np.exp(0.5 * q @ k.T - l0[0, 0][:, None]), None
    bound = np.sqrt((0.25 / 0.75) * (p ** 2) @ (v ** 2) / seeds)
    assert np.all(np.abs(mean[0, 0] - o0[0, 0]) <= 6 * bound + 1e-12)


def test_dropout_output_uses_the_keep_mask():
    rng = np.random.default_rng(6)
    n, d = 12, 3
    q, k, v = _rand(rng, n, d), _rand(rng, n, d), _rand(rng, n, d)
    o, _ = attention_forward(q, k, v, 0.5, causal=True, dropout_p=0.5, seed=11, offset=3)
    keep, mult = dropout_keep(np.arange(n), np.arange(n), 0, 11, 3, 0.5)
    s = 0.5 * q @ k.T
    s[np.triu_indices(n, 1)] = -np.inf
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    np.testing.assert_allclose(o[0, 0], (p * keep * mult) @ v, rtol=0, atol=1e-14)


@pytest.mark.parametrize("case", ["dropout", "dropout_causal_window", "gqa_dropout"])
def test_central_finite_differences(case):
    rng = np.random.default_rng({"dropout": 1, "dropout_causal_window": 2, "gqa_dropout": 3}[case])
    n, d = 10, 3
    hq, hkv = (2, 1) if case == "gqa_dropout" else (1, 1)
    kw = dict(dropout_p=0.3, seed=21, offset=4)
    if case == "dropout_causal_window":
        kw.update(causal=True, window=4)
    q, do = _rand(rng, 1, hq, n, d), _rand(rng, 1, hq, n, d)
    k, v = _rand(rng, 1, hkv, n, d), _rand(rng, 1, hkv, n, d)
    scale = 0.45
    dq, dk, dv, dd, ddot = attention_backward(q, k, v, do, scale, return_d=True, **kw)
    np.testing.assert_allclose(dd, ddot, rtol=0, atol=1e-13)

    def f(args):
        o, _ = attention_forward(args["q"], args["k"], args["v"], scale, **kw)
        return float((o * do).sum())

    h = 1e-6
    for name, g in (("q", dq), ("k", dk), ("v", dv)):
        args = {"q": q, "k": k, "v": v}
        x = args[name]
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            num[idx] = (f({**args, name: xp}) - f({**args, name: xm})) / (2 * h)
        err = np.linalg.norm(num - g) / max(np.linalg.norm(num), 1e-300)
        assert err < 1e-6, (name, err)


@pytest.mark.parametrize("causal", [False, True])
def test_window_finite_differences(causal):
    rng = np.random.default_rng(9)
    n, d, w = 11, 3, 3
    q, k, v, do = (_rand(rng, n, d) for _ in range(4))
    dq, dk, dv = attention_backward(q, k, v, do, 0.6, causal=causal, window=w)
    h = 1e-6
    base = {"q": q, "k": k, "v": v}
    for name, g in (("q", dq), ("k", dk), ("v", dv)):
        x = base[name]
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            fp = (attention_forward(**{**base, name: xp}, scale=0.6, causal=causal,
                                    window=w)[0][0, 0] * do).sum()
            fm = (attention_forward(**{**base, name: xm}, scale=0.6, causal=causal,
                                    window=w)[0][0, 0] * do).sum()
            num[idx] = (fp - fm) / (2 * h)
        err = np.linalg.norm(num - g[0, 0]) / np.linalg.norm(num)
        assert err < 1e-6, (name, err)
