"""Pins for the oracle's backward pass (CPU only): hand-derived fixture,
central finite differences of f = <O, dO>, the D identity, and special cases."""

import json
import os

import numpy as np
import pytest

from oracle import attention_backward, attention_forward

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _f(q, k, v, do, scale, causal, bm, mb):
    o, _ = attention_forward(q, k, v, scale, causal=causal, block_mask=bm, mask_block=mb)
    return float((o[0, 0] * do).sum())


@pytest.mark.parametrize("causal", [False, True])
def test_two_token_fixture(causal):
    g = json.load(open(os.path.join(GOLDEN, "two_token_closed_form.json")))
    inp = g["inputs"]
    exp = g["causal" if causal else "noncausal"]
    q, k, v, do = (np.array(inp[n]) for n in ("q", "k", "v", "do"))
    dq, dk, dv = attention_backward(q, k, v, do, inp["scale"], causal=causal)
    for got, name in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        np.testing.assert_allclose(got[0, 0], exp[name], rtol=0, atol=1e-14)


@pytest.mark.parametrize("case", ["dense", "causal", "masked", "causal_masked"])
def test_central_finite_differences(case):
    rng = np.random.default_rng({"dense": 1, "causal": 2, "masked": 3, "causal_masked": 4}[case])
    n, d, mb = 12, 4, 3
    causal = "causal" in case
    bm = None
    if "masked" in case:
        bm = np.array([[1, 0, 1, 0], [1, 1, 0, 0], [0, 1, 1, 0], [1, 0, 0, 1]], np.uint8)
    q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
    scale = 0.45
    dq, dk, dv = attention_backward(q, k, v, do, scale, causal=causal, block_mask=bm, mask_block=mb)
    h = 1e-6
    for name, x, g in (("q", q, dq[0, 0]), ("k", k, dk[0, 0]), ("v", v, dv[0, 0])):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            fp = _f(args["q"], args["k"], args["v"], do, scale, causal, bm, mb)
            args[name] = xm
            fm = _f(args["q"], args["k"], args["v"], do, scale, causal, bm, mb)
            num[idx] = (fp - fm) / (2 * h)
        err = np.linalg.norm(num - g) / max(np.linalg.norm(num), 1e-300)
        assert err < 1e-6, (name, err)


@pytest.mark.parametrize("causal", [False, True])
def test_d_identity(causal):
    rng = np.random.default_rng(20)
    q, k, v, do = (rng.standard_normal((2, 2, 33, 8)) for _ in range(4))
    _, _, _, dd, ddot = attention_backward(q, k, v, do, 0.35, causal=causal, return_d=True)
    np.testing.assert_allclose(dd, ddot, rtol=0, atol=1e-12)


def test_single_token_gradients():
    rng = np.random.default_rng(21)
    q, k, v, do = (rng.standard_normal((1, 64)) for _ in range(4))
    dq, dk, dv = attention_backward(q, k, v, do, 0.125)
    assert np.all(dq == 0) and np.all(dk == 0)
    np.testing.assert_array_equal(dv[0, 0], do)


def test_unseen_key_block_gets_zero_gradient():
    rng = np.random.default_rng(22)
    mb = 4
    bm = np.ones((3, 3), np.uint8)
    bm[:, 1] = 0  # no query sees keys 4..7
    q, k, v, do = (rng.standard_normal((12, 5)) for _ in range(4))
    dq, dk, dv = attention_backward(q, k, v, do, 0.5, block_mask=bm, mask_block=mb)
    assert np.all(dk[0, 0, 4:8] == 0) and np.all(dv[0, 0, 4:8] == 0)
    assert np.abs(dk[0, 0, :4]).max() > 0


@pytest.mark.parametrize("causal", [False, True])
def test_row_chunked_backward_equals_single_pass(causal):
    rng = np.random.default_rng(23)
    q, k, v, do = (rng.standard_normal((1, 2, 37, 6)) for _ in range(4))
    ref = attention_backward(q, k, v, do, 0.4, causal=causal, row_chunk=37)
    for chunk in (1, 5, 16):
        got = attention_backward(q, k, v, do, 0.4, causal=causal, row_chunk=chunk)
        for a, b in zip(ref, got):
            np.testing.assert_allclose(a, b, atol=1e-13)


def test_fully_masked_row_has_zero_query_gradient():
    rng = np.random.default_rng(24)
    bm = np.ones((4, 4), np.uint8)
    bm[2, :] = 0
    q, k, v, do = (rng.standard_normal((8, 3)) for _ in range(4))
    dq, dk, dv = attention_backward(q, k, v, do, 1.0, block_mask=bm, mask_block=2)
    assert np.all(dq[0, 0, 4:6] == 0)
    # rows 4, 5 contribute nothing: removing their dO leaves dK, dV unchanged
    do2 = do.copy()
    do2[4:6] = 123.0
    dq2, dk2, dv2 = attention_backward(q, k, v, do2, 1.0, block_mask=bm, mask_block=2)
    np.testing.assert_array_equal(dk, dk2)
    np.testing.assert_array_equal(dv, dv2)
