"""GPU parity of the decode-shaped forward (fa_fwd_decode; MI355X only).

The last n_q positions of a sequence against its N keys: fp64 oracle with the
query offset N - n_q on the same seeded inputs, covering one and several
queries, grouped heads (rows of several query heads per workgroup, more than
one 128-row block), causal and windowed visibility, ragged key counts, a
single key, the split path and the direct (one split) path, the decode
workload at full size, and 60 seeded random problems over the same features.
Q = 0 makes LSE an exact count of the visible keys."""

import numpy as np
import pytest
import torch

from io_aware_exact_fwd_amd import fa_fwd, fa_fwd_decode
from io_aware_exact_fwd_amd.workloads import WORKLOADS, make_decode_inputs
from oracle import attention_forward

from gpu_util import LSE_TOL, O_TOL, say, to_np

pytestmark = pytest.mark.gpu


def _decode_case(name, B, H, hkv, N, nq, d, dtype, causal, window=0, scale=None, q_zero=False):
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    say(f"[case] {name}: B={B} H={H} H_kv={hkv} N={N} n_q={nq} d={d} {dtype} causal={causal} "
        f"window={window}")
    q, k, v = make_decode_inputs(B, H, N, d, nq, dtype, hkv=hkv)
    if q_zero:
        q = torch.zeros_like(q)
    dev = torch.device("cuda:0")
    o, lse = fa_fwd_decode(q.to(dev), k.to(dev), v.to(dev), causal=causal, scale=scale,
                           window=window)
    torch.cuda.synchronize()
    o_ref, lse_ref = attention_forward(*(x.float().numpy() for x in (q, k, v)), scale, causal,
                                       window=window, q_offset=N - nq)
    o_g, lse_g = to_np(o), to_np(lse)
    assert np.all(np.isfinite(o_g)) and np.all(np.isfinite(lse_g)), name
    err = {"o": float(np.abs(o_g - o_ref).max()), "lse": float(np.abs(lse_g - lse_ref).max())}
    say(f"[case] {name}: errors {err}")
    assert err["o"] <= O_TOL[dtype], (name, err)
    assert err["lse"] <= LSE_TOL, (name, err)
    return o_g, lse_g, lse_ref


CASES = [
    # dtype, d, B, H, hkv, N, nq, causal, window
    ("f16", 64, 1, 2, 2, 1, 1, True, 0),         # a single key
    ("f16", 64, 2, 4, 1, 100, 1, True, 0),       # multi-query, one tile, ragged
    ("bf16", 128, 2, 8, 2, 4097, 1, True, 0),    # many splits, ragged last tile
    ("f16", 64, 1, 8, 8, 4096, 4, True, 0),      # several queries, causal inside the last tile
    ("f16", 128, 2, 4, 2, 2000, 16, False, 0),   # non-causal
    ("bf16", 64, 1, 6, 3, 3000, 3, True, 500),   # causal window
    ("f16", 64, 2, 4, 2, 300, 5, False, 64),     # two-sided window
    ("f16", 64, 1, 8, 1, 1024, 40, True, 0),     # 320 rows per K/V head: three row blocks
    ("bf16", 128, 1, 2, 1, 777, 777, True, 0),   # n_q = N: the square problem
    ("f16", 64, 64, 16, 16, 64, 1, True, 0),     # one tile: the direct path, no merge
]


@pytest.mark.parametrize("dtype,d,B,H,hkv,N,nq,causal,window", CASES)
def test_decode_small(dtype, d, B, H, hkv, N, nq, causal, window):
    _decode_case(f"decode-{dtype}-d{d}-B{B}-H{H}-kv{hkv}-N{N}-q{nq}-c{int(causal)}-w{window}",
                 B, H, hkv, N, nq, d, dtype, causal, window)


@pytest.mark.parametrize("N,nq,causal,window", [(8192, 1, True, 0), (5000, 7, True, 0),
                                                (4100, 3, True, 1000), (3000, 2, False, 700)])
def test_decode_zero_queries_lse_counts_visible_keys(N, nq, causal, window):
    """Q = 0: LSE_i = ln(#keys visible from position N - nq + i), exact to
    rounding, so an off-by-one in split bounds, tile skipping or masks shows."""
    _, lse_g, lse_ref = _decode_case(f"decode-q0-N{N}-q{nq}", 1, 4, 2, N, nq, 64, "f16", causal,
                                     window, q_zero=True)
    for i in range(nq):
        pos = N - nq + i
        lo = max(0, pos - window + 1) if window else 0
        hi = pos if causal else (min(N - 1, pos + window - 1) if window else N - 1)
        assert np.allclose(lse_g[..., i], np.log(hi - lo + 1), rtol=0, atol=1e-5), (i, pos)
    assert np.allclose(lse_g, lse_ref, rtol=0, atol=1e-5)


def test_decode_square_equals_forward_kernel():
    """n_q = N through the decode path agrees with fa_fwd on the same inputs,
    to the stated O and LSE tolerances (the two paths tile the keys differently,
    32 vs 64, so their running reference maxima -- and with them the fp16
    rounding of the weights that the row sum adds up -- differ)."""
    B, H, N, d = 1, 4, 1000, 64
    q, k, v = make_decode_inputs(B, H, N, d, N, "f16", hkv=2)
    dev = torch.device("cuda:0")
    qd, kd, vd = (x.to(dev) for x in (q, k, v))
    o1, l1 = fa_fwd_decode(qd, kd, vd, causal=True)
    o2, l2 = fa_fwd(qd, kd, vd, causal=True)
    torch.cuda.synchronize()
    assert float((o1.float() - o2.float()).abs().max()) <= O_TOL["f16"]
    assert float((l1 - l2).abs().max()) <= LSE_TOL


def test_workload_decode_gqa_full_size():
    w = WORKLOADS["decode_gqa"]
    _decode_case("decode_gqa", w.B, w.H, w.H_kv, w.N, w.nq, w.d, w.dtype, w.causal,
                 scale=w.scale)


def test_decode_repeatable():
    """The split and merge order is fixed by the problem, so two calls give
    the same bits."""
    q, k, v = make_decode_inputs(2, 16, 5000, 128, 2, "bf16", hkv=4)
    dev = torch.device("cuda:0")
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    o1, l1 = fa_fwd_decode(qd, kd, vd, causal=True)
    o2, l2 = fa_fwd_decode(qd, kd, vd, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def _draw_decode(i):
    """Seeded random decode problems: either dtype and head dim, grouped heads,
    ragged key counts (a single key included), one or several queries,
    causal or not, with or without a window."""
    rng = np.random.default_rng(70000 + i)
    d = int(rng.choice([64, 128]))
    dtype = str(rng.choice(["f16", "bf16"]))
    hkv = int(rng.choice([1, 2, 4]))
    H = hkv * int(rng.choice([1, 2, 4, 8]))
    B = int(rng.choice([1, 2]))
    N = int(rng.integers(1, 6000))
    nq = int(min(N, rng.choice([1, 1, 2, 3, int(rng.integers(1, 65))])))
    causal = bool(rng.random() < 0.7)
    window = int(rng.choice([0, 0, int(rng.integers(1, 1500))]))
    return dtype, d, B, H, hkv, N, nq, causal, window


@pytest.mark.parametrize("i", list(range(60)))
def test_decode_random(i):
    dtype, d, B, H, hkv, N, nq, causal, window = _draw_decode(i)
    _decode_case(f"decode-random{i}", B, H, hkv, N, nq, d, dtype, causal, window)
