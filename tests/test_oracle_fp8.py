"""Pins of the FP8 oracle (oracle/fp8.py).  CPU only.

Fixed by things other than the oracle itself: the E4M3 format definition
(bias 7, 3 mantissa bits, subnormals m * 2^-9, largest finite 448, NaN at
0x7F), the Sylvester Hadamard matrix written out by recursion, orthogonality,
the exactness of power-of-two scaling, the reduction to exact attention when
nothing is quantised, and the pages' statement that block scales plus the
rotation lower the FP8 error against per-tensor FP8 on inputs with outliers."""

import numpy as np
import pytest

from oracle import attention_forward
from oracle.fp8 import (E4M3_MAX, block_dequantize, block_quantize, e4m3_decode, e4m3_encode,
                        fp8_attention_forward, hadamard_matrix, rotate_rows_f32, rotation_matrix)


def test_e4m3_code_table():
    codes = np.arange(256, dtype=np.uint8)
    v = e4m3_decode(codes)
    assert v[0x00] == 0.0 and v[0x01] == 2.0 ** -9 and v[0x07] == 7 * 2.0 ** -9
    assert v[0x08] == 2.0 ** -6 and v[0x38] == 1.0 and v[0x39] == 1.125
    assert v[0x7E] == 448.0 and np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert v[0x80] == 0.0 and v[0xB8] == -1.0 and v[0xFE] == -448.0
    finite = ~np.isnan(v)
    assert np.nanmax(v) == E4M3_MAX
    # every finite code round-trips (negative zero encodes to 0x80)
    assert np.array_equal(e4m3_encode(v[finite]), codes[finite])


def test_e4m3_rounding_is_nearest_even():
    # halfway cases go to the even mantissa
    assert e4m3_decode(e4m3_encode([1.0625, 1.1875, 3 * 2.0 ** -10, 464.0]))[:4].tolist() == \
        [1.0, 1.25, 2.0 ** -8, 448.0]
    # non-halfway: nearest
    x = np.random.default_rng(0).uniform(-400, 400, 5000)
    q = e4m3_decode(e4m3_encode(x))
    grid = np.unique(np.abs(e4m3_decode(np.arange(0, 127, dtype=np.uint8))))
    for xi, qi in zip(x[:200], q[:200]):
        nearest = grid[np.argmin(np.abs(grid - abs(xi)))]
        assert abs(abs(qi) - abs(xi)) <= abs(nearest - abs(xi)) + 1e-12
    assert e4m3_decode(e4m3_encode([1000.0, -1e6]))[:2].tolist() == [448.0, -448.0]


def test_hadamard_is_sylvester_and_rotation_orthogonal():
    h2 = np.array([[1, 1], [1, -1]])
    assert np.array_equal(hadamard_matrix(4), np.kron(h2, h2))
    for d in (64, 128):
        h = hadamard_matrix(d)
        assert np.array_equal(h @ h.T, d * np.eye(d))
        s = np.where(np.random.default_rng(d).random(d) < 0.5, -1.0, 1.0)
        m = rotation_matrix(s)
        assert np.allclose(m @ m.T, np.eye(d), atol=1e-14)


@pytest.mark.parametrize("d", [64, 128])
def test_float32_butterflies_equal_the_matrix_product(d):
    rng = np.random.default_rng(1)
    s = np.where(rng.random(d) < 0.5, -1.0, 1.0)
    x = rng.standard_normal((37, d)).astype(np.float32)
    y = rotate_rows_f32(x, s)
    assert y.dtype == np.float32
    ref = x.astype(np.float64) @ rotation_matrix(s)
    assert np.abs(y - ref).max() <= 1e-5 * np.abs(ref).max()
    # unit vectors map to rows of M exactly (one nonzero input: no rounding)
    e = np.eye(d, dtype=np.float32)
    assert np.array_equal(rotate_rows_f32(e, s).astype(np.float64),
                          (rotation_matrix(s) * np.sqrt(d)).astype(np.float32) * np.float32(1 / np.sqrt(d)))


def test_block_exponent_stays_in_the_e8m0_range():
    """A block whose largest magnitude is below 448 * 2^-128 keeps e = -127
    (the smallest E8M0 scale); just above it the tight rule applies."""
    y = np.zeros((128, 64), dtype=np.float32)
    y[0, 0] = np.float32(2.0 ** -125)       # tight e would be -125 - 8 = -133
    y[5, 3] = np.float32(-3.0 * 2.0 ** -130)
    y[64, 0] = np.float32(448.0 * 2.0 ** -127)  # tight e = -127 exactly
    codes, e = block_quantize(y)
    assert list(e) == [-127, -127]
    # 2^-125 / 2^-127 = 4 = 1.0 * 2^2: exponent field 9, mantissa 0 -> 0x48;
    # -3 * 2^-130 / 2^-127 = -3/8 = -1.5 * 2^-2: field 5, mantissa 4 -> 0x80 | 0x2C
    assert codes[0, 0] == 0x48 and codes[5, 3] == 0xAC and codes[64, 0] == 0x7E
    assert np.all(block_dequantize(codes, e, 128)[[0, 5, 64], [0, 3, 0]]
                  == [2.0 ** -125, -3.0 * 2.0 ** -130, 448.0 * 2.0 ** -127])
    _, e2 = block_quantize(np.full((64, 64), 1.75 * 2.0 ** -119, dtype=np.float32))
    assert e2[0] == -127                     # 1.75 * 2^-119 = 448 * 2^-127
    _, e3 = block_quantize(np.full((64, 64), 2.0 ** -118, dtype=np.float32))
    assert e3[0] == -126


def test_block_scales_are_tight_powers_of_two():
    rng = np.random.default_rng(2)
    y = (rng.standard_normal((2, 200, 64)) * rng.uniform(1e-3, 1e3, (2, 1, 1))).astype(np.float32)
    y[1, 64:128] = 0.0                                  # an all-zero block
    codes, e = block_quantize(y)
    assert codes.shape == (2, 256, 64) and e.shape == (2, 4)
    blocks = np.concatenate([y, np.zeros((2, 56, 64), np.float32)], axis=1).reshape(2, 4, 64, 64)
    amax = np.abs(blocks).max(axis=(2, 3))
    live = amax > 0
    assert np.all(amax[live] <= E4M3_MAX * 2.0 ** e[live])
    assert np.all(amax[live] > E4M3_MAX * 2.0 ** (e[live] - 1))
    assert np.all(codes[1, 64:128] == 0) and e[1, 1] == 0
    # dequantisation: each value within half an E4M3 step of its scaled original
    back = block_dequantize(codes, e, 200)
    step = np.maximum(np.exp2(np.floor(np.log2(np.maximum(np.abs(y), 1e-30)))) / 8.0,
                      2.0 ** -9 * np.exp2(np.repeat(e, 64, axis=1)[:, :200])[..., None])
    assert np.all(np.abs(back - y) <= step / 2 + 1e-30)


@pytest.mark.parametrize("causal", [True, False])
def test_without_quantisation_it_is_exact_attention(causal):
    rng = np.random.default_rng(3)
    B, H, Hkv, N, d = 1, 4, 2, 70, 64
    q = rng.standard_normal((B, H, N, d)).astype(np.float32)
    k = rng.standard_normal((B, Hkv, N, d)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, N, d)).astype(np.float32)
    s = np.where(rng.random(d) < 0.5, -1.0, 1.0)
    o, lse, _ = fp8_attention_forward(q, k, v, 0.125, s, causal, quantize=False)
    o_ref, lse_ref = attention_forward(q, k, v, 0.125, causal)
    assert np.abs(o - o_ref).max() < 2e-6 and np.abs(lse - lse_ref).max() < 2e-6


def test_block_scales_and_rotation_beat_per_tensor_fp8_on_outliers():
    """The pages report block quantisation + incoherent processing lowering the
    FP8 error of attention 2.6x against per-tensor FP8.  On inputs whose rows
    carry a few large outlier coordinates the method must at least beat the
    per-tensor baseline clearly."""
    rng = np.random.default_rng(4)
    B, H, N, d = 1, 2, 256, 64
    q, k, v = (rng.standard_normal((B, H, N, d)).astype(np.float32) for _ in range(3))
    for x in (q, k):
        x[..., 3] *= 30.0
        x[..., 17] *= 20.0
    s = np.where(rng.random(d) < 0.5, -1.0, 1.0)
    scale = 1.0 / 8.0
    o_ref, _ = attention_forward(q, k, v, scale, True)
    o_fp8, _, _ = fp8_attention_forward(q, k, v, scale, s, True)

    def per_tensor(x):
        sc = np.abs(x).max() / E4M3_MAX
        return e4m3_decode(e4m3_encode(x / sc)) * sc

    o_pt, _ = attention_forward(per_tensor(q), per_tensor(k), per_tensor(v), scale, True)
    err_method = np.linalg.norm(o_fp8 - o_ref)
    err_tensor = np.linalg.norm(o_pt - o_ref)
    assert err_method * 1.5 < err_tensor, (err_method, err_tensor)
