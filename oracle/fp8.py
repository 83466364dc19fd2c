"""FP8 forward with block scales and a random Hadamard rotation (oracle).

TEST INFRASTRUCTURE ONLY -- see ``oracle/__init__.py``.  Nothing in the
product path may import this module.

What the pages describe ([ldl] section 10 on FlashAttention-3; [mm] "FA3"):
Q, K and V are quantised to FP8 with one scale factor per tile (block
quantisation) after a randomised Hadamard-style orthogonal rotation that
spreads outlier coordinates over the whole vector (incoherent processing);
the rotation is undone after the matmul, so the attention is exact up to the
FP8 rounding.  Readings taken where the pages leave the details open:

* FP8 format: E4M3 (4 exponent bits, bias 7, 3 mantissa bits, subnormals
  m * 2^-9, largest finite value 448), round to nearest even.
* Rotation: M = diag(s) H / sqrt(d) with H the d x d Sylvester Hadamard
  matrix (entries +-1) and s a vector of random signs supplied by the caller;
  M is orthogonal, so (Q M)(K M)^T = Q K^T and O = ((P (V M)) M^T).  Rows are
  rotated in float32 with the fast Walsh-Hadamard butterflies in a fixed
  order (pair distances 1, 2, 4, ..., d/2; (a, b) -> (a + b, a - b)), then
  multiplied by float32(1 / sqrt(d)) -- the same float32 operations the GPU
  performs, so both sides reach identical quantised codes.
* Block: 64 consecutive rows of one head (the kernels' tile height); scale
  2^e with e the smallest integer such that max |y| <= 448 * 2^e (an exact
  power of two, so dequantisation is exact); codes = E4M3(y / 2^e).  The
  scale is carried as an 8-bit power-of-two exponent (E8M0, 2^-127 ..
  2^127), so e is raised to -127 for a block whose largest magnitude is below
  448 * 2^-128 (values near the float32 underflow threshold); e = 0 for an
  all-zero block.
* Attention: the plain definition (``oracle.attention``) applied to the
  dequantised rotated tensors in float64, then O multiplied by M^T.  The
  kernel additionally rounds the probabilities to E4M3 before the P V
  product; the oracle does not model that rounding (nor float32 accumulation
  order); the tolerances of the GPU parity tests absorb it.
"""

from __future__ import annotations

import numpy as np

from .attention import attention_forward

__all__ = [
    "E4M3_MAX",
    "e4m3_encode",
    "e4m3_decode",
    "hadamard_matrix",
    "rotation_matrix",
    "rotate_rows_f32",
    "block_quantize",
    "fp8_attention_forward",
]

E4M3_MAX = 448.0
BLOCK_ROWS = 64


def e4m3_decode(codes):
    """Values (float64) of E4M3 codes; 0x7F / 0xFF (NaN) decode to nan."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    ex = (c >> 3) & 15
    m = c & 7
    val = np.where(ex == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(ex.astype(np.float64) - 7))
    val = np.where((c & 0x7F) == 0x7F, np.nan, val)
    return sign * val


def e4m3_encode(x):
    """Round float values to E4M3 codes (nearest, ties to even), saturating at
    +-448 (the method never produces larger magnitudes)."""
    x = np.asarray(x, dtype=np.float64)
    sign = np.where(np.signbit(x), 0x80, 0).astype(np.int64)
    a = np.abs(x)
    _, e2 = np.frexp(np.where(a > 0, a, 1.0))   # a = f * 2^e2, f in [0.5, 1)
    e = np.maximum(e2 - 1, -6)                    # binade exponent; subnormals use -6
    q = a / np.exp2(e - 3)                        # in units of the last mantissa bit
    r = np.rint(q)                                # ties to even
    carry = r >= 16
    e = np.where(carry, e + 1, e)
    r = np.where(carry, r / 2, r)
    over = (e > 8) | ((e == 8) & (r > 14))
    sub = r < 8
    code = np.where(sub, r, ((e + 7) << 3) + (r - 8)).astype(np.int64)
    code = np.where(over, 0x7E, code)
    code = np.where(a == 0, 0, code)
    return (sign | code).astype(np.uint8)


def hadamard_matrix(d):
    """Sylvester Hadamard matrix H_d (d a power of two), entries +-1."""
    h = np.ones((1, 1))
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    if h.shape[0] != d:
        raise ValueError("d must be a power of two")
    return h


def rotation_matrix(signs):
    """M = diag(s) H / sqrt(d) (float64, orthogonal)."""
    s = np.asarray(signs, dtype=np.float64)
    d = s.size
    return (s[:, None] * hadamard_matrix(d)) / np.sqrt(d)


def rotate_rows_f32(x, signs):
    """Rows of x times M, computed in float32 in the fixed butterfly order
    described in the module docstring (returns float32)."""
    y = np.asarray(x, dtype=np.float32) * np.asarray(signs, dtype=np.float32)
    d = y.shape[-1]
    h = 1
    while h < d:
        y = y.reshape(*y.shape[:-1], d // (2 * h), 2, h)
        a, b = y[..., 0, :], y[..., 1, :]
        y = np.stack([a + b, a - b], axis=-2).reshape(*y.shape[:-3], d)
        h *= 2
    return (y * np.float32(1.0 / np.sqrt(d))).astype(np.float32)


E8M0_MIN_EXP = -127


def _block_exponent(amax):
    """Smallest integer e >= -127 with amax <= 448 * 2^e (0 for an all-zero
    block)."""
    amax = np.asarray(amax, dtype=np.float64)
    f, e2 = np.frexp(np.where(amax > 0, amax, 1.0))  # amax = f * 2^e2, f in [0.5, 1)
    mant = 2.0 * f                                     # amax = mant * 2^(e2 - 1)
    e = (e2 - 1) - 8 + (mant > 1.75).astype(np.int64)
    e = np.maximum(e, E8M0_MIN_EXP)
    return np.where(amax > 0, e, 0).astype(np.int64)


def block_quantize(y, rows=BLOCK_ROWS):
    """Quantise float32 y (..., N, d) in blocks of ``rows`` rows along N (the
    last block padded with zeros): returns (codes uint8 (..., N_pad, d),
    exponents int64 (..., N_pad / rows))."""
    y = np.asarray(y, dtype=np.float32)
    n, d = y.shape[-2:]
    npad = -(-n // rows) * rows
    pad = np.zeros((*y.shape[:-2], npad - n, d), dtype=np.float32)
    yp = np.concatenate([y, pad], axis=-2)
    blocks = yp.reshape(*y.shape[:-2], npad // rows, rows, d)
    amax = np.abs(blocks).max(axis=(-2, -1))
    e = _block_exponent(amax)
    scaled = blocks * np.exp2(-e.astype(np.float64))[..., None, None]  # exact: power of two
    codes = e4m3_encode(scaled).reshape(*y.shape[:-2], npad, d)
    return codes, e


def block_dequantize(codes, e, n, rows=BLOCK_ROWS):
    """float64 values of (codes, exponents), first n rows."""
    d = codes.shape[-1]
    v = e4m3_decode(codes).reshape(*codes.shape[:-2], -1, rows, d)
    v = v * np.exp2(e.astype(np.float64))[..., None, None]
    return v.reshape(*codes.shape[:-2], -1, d)[..., :n, :]


def fp8_attention_forward(q, k, v, scale, signs, causal=False, window=0, heads=None,
                          quantize=True):
    """O (float64), LSE (float64) and the quantised tensors of the FP8 method.

    q: (B, H, N, d), k, v: (B, H_kv, N, d) in any float dtype (upcast exactly).
    signs: d values +-1.  With quantize=False the rotated tensors are used
    without quantisation (then O equals exact attention up to rounding).
    Returns (o, lse, quant) with quant = {name: (codes, exponents)} for
    name in ("q", "k", "v") (codes row-major, exponents per 64-row block)."""
    q, k, v = (np.asarray(x, dtype=np.float32) for x in (q, k, v))
    n = q.shape[-2]
    m = rotation_matrix(signs)
    quant = {}
    deq = {}
    for name, x in (("q", q), ("k", k), ("v", v)):
        y = rotate_rows_f32(x, signs)
        if quantize:
            codes, e = block_quantize(y)
            quant[name] = (codes, e)
            deq[name] = block_dequantize(codes, e, n)
        else:
            deq[name] = y.astype(np.float64)
    o_rot, lse = attention_forward(deq["q"], deq["k"], deq["v"], scale, causal, window=window,
                                   heads=heads)
    o = o_rot @ m.T
    return o, lse, quant
