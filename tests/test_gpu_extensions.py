"""GPU parity of the sliding window and of grouped K/V heads (MI355X only).

Same bar as the dense cases: fp64 oracle on the same seeded inputs, small
shapes spanning several tiles with ragged ends, the full-size workloads on
every head (whole tensors), and Q = 0 cases whose LSE is an exact count of
visible keys."""

import numpy as np
import pytest
import torch

from io_aware_exact_fwd_amd import fa_bwd, fa_fwd
from io_aware_exact_fwd_amd.workloads import WORKLOADS, butterfly_block_mask, make_inputs

from gpu_util import check_case, say

pytestmark = pytest.mark.gpu

WINDOW = []
for dtype, d in (("f16", 64), ("bf16", 128)):
    for N, causal, w in ((129, True, 1), (300, True, 37), (300, False, 64), (1000, True, 128),
                         (1000, False, 200), (777, False, 1000)):
        WINDOW.append((dtype, d, N, causal, w))


@pytest.mark.parametrize("dtype,d,N,causal,w", WINDOW)
def test_small_window(dtype, d, N, causal, w):
    check_case(f"window-{dtype}-d{d}-N{N}-c{int(causal)}-w{w}", 1, 2, N, d, dtype, causal,
               window=w)


@pytest.mark.parametrize("causal,w", [(True, 50), (False, 33)])
def test_window_f32(causal, w):
    err = check_case(f"window-f32-c{int(causal)}-w{w}", 1, 2, 257, 64, "f32", causal, window=w)
    assert err["o"] < 1e-5


@pytest.mark.parametrize("causal", [False, True])
def test_window_with_block_mask(causal):
    N, mb = 1024, 128
    check_case(f"window-blocks-c{int(causal)}", 1, 2, N, 64, "f16", causal,
               block_mask=butterfly_block_mask(N // mb), mask_block=mb, window=300)


GQA = [("f16", 64, 300, True, 6, 2), ("f16", 64, 1024, False, 8, 1), ("bf16", 128, 513, True, 4, 2),
       ("bf16", 64, 200, False, 6, 3), ("f32", 64, 130, True, 4, 1), ("f32", 128, 100, False, 4, 2)]


@pytest.mark.parametrize("dtype,d,N,causal,H,hkv", GQA)
def test_small_grouped_heads(dtype, d, N, causal, H, hkv):
    check_case(f"gqa-{dtype}-d{d}-N{N}-c{int(causal)}-H{H}-kv{hkv}", 2, H, N, d, dtype, causal,
               hkv=hkv)


def test_grouped_heads_window_block_mask():
    N, mb = 1024, 256
    check_case("gqa-window-blocks", 1, 4, N, 64, "bf16", True,
               block_mask=butterfly_block_mask(N // mb), mask_block=mb, window=400, hkv=2)


def test_workload_long_window_full_size():
    w = WORKLOADS["long_window"]
    err = check_case(w.name, w.B, w.H, w.N, w.d, w.dtype, w.causal, w.scale, window=w.window)
    assert err["heads"] == w.B * w.H


def test_workload_gqa_full_size():
    w = WORKLOADS["gqa_h64_kv8"]
    err = check_case(w.name, w.B, w.H, w.N, w.d, w.dtype, w.causal, w.scale, hkv=w.H_kv)
    assert err["heads"] == w.B * w.H


def _window_counts(N, causal, w):
    i = np.arange(N)
    lo = np.maximum(0, i - w + 1)
    hi = i if causal else np.minimum(N - 1, i + w - 1)
    return hi - lo + 1


@pytest.mark.parametrize("N,causal,w,d", [(4096, True, 300, 64), (4096, False, 1000, 128),
                                          (8192, True, 512, 128), (1000, False, 1, 64)])
def test_zero_queries_lse_counts_window(N, causal, w, d):
    """Q = 0: LSE_i = ln(#keys in row i's window) exactly."""
    dev = torch.device("cuda:0")
    say(f"[case] zero-q window N={N} causal={causal} w={w} d={d}")
    _, k, v, _ = make_inputs(1, 2, N, d, "f16", hkv=1)
    q = torch.zeros((1, 2, N, d), dtype=torch.float16)
    o, lse = fa_fwd(q.to(dev), k.to(dev), v.to(dev), causal=causal, scale=0.125, window=w)
    want = np.log(_window_counts(N, causal, w))
    got = lse.cpu().numpy().astype(np.float64)
    for h in range(2):
        assert np.abs(got[0, h] - want).max() <= 1e-5


# ------------------------------------------------------------------ dropout

DROPOUT = [("f16", 64, 300, True, 0.5, 0, 0), ("bf16", 128, 513, False, 0.2, 0, 0),
           ("f16", 64, 1000, True, 0.1, 200, 0), ("bf16", 64, 257, False, 0.75, 0, 0),
           ("f16", 128, 130, True, 0.3, 0, 0), ("f32", 64, 100, True, 0.5, 0, 0),
           ("f32", 128, 70, False, 0.25, 20, 0)]


@pytest.mark.parametrize("dtype,d,N,causal,p,w,_", DROPOUT)
def test_small_dropout(dtype, d, N, causal, p, w, _):
    check_case(f"dropout-{dtype}-d{d}-N{N}-c{int(causal)}-p{p}-w{w}", 2, 2, N, d, dtype, causal,
               window=w, dropout=(p, 0x1234_5678_9ABC_DEF0 + N, 7))


def test_dropout_grouped_heads_block_mask():
    N, mb = 1024, 256
    check_case("dropout-gqa-blocks", 1, 4, N, 64, "f16", True,
               block_mask=butterfly_block_mask(N // mb), mask_block=mb, hkv=2,
               dropout=(0.5, 99, 3))


def test_workload_dropout_full_size():
    w = WORKLOADS["gpt2_medium_dropout"]
    err = check_case(w.name, w.B, w.H, w.N, w.d, w.dtype, w.causal, w.scale,
                     dropout=(w.dropout, 2024, 1))
    assert err["heads"] == w.B * w.H


@pytest.mark.parametrize("causal,p,d", [(False, 0.5, 64), (True, 0.25, 64), (False, 0.1, 128)])
def test_dropout_keep_mask_bit_exact(causal, p, d):
    """Q = 0 makes every visible weight 1/count; with V[j, c] = [j mod d == c]
    the output times count / mult is the number of kept keys j = c (mod d) of
    row i, an exact integer to compare with the oracle's keep mask."""
    from oracle.philox import dropout_keep

    dev = torch.device("cuda:0")
    N, H, seed, offset = 384, 2, 0xDEADBEEF12345, 11
    say(f"[case] dropout keep mask causal={causal} p={p} d={d}")
    q = torch.zeros((1, H, N, d), dtype=torch.float16)
    _, k, _, _ = make_inputs(1, H, N, d, "f16")
    v = torch.zeros((1, H, N, d), dtype=torch.float16)
    v[:, :, torch.arange(N), torch.arange(N) % d] = 1
    o, _ = fa_fwd(q.to(dev), k.to(dev), v.to(dev), causal=causal, scale=0.125, dropout_p=p,
                  seed=seed, offset=offset)
    got = o.float().cpu().numpy().astype(np.float64)
    count = (np.arange(N) + 1 if causal else np.full(N, N)).astype(np.float64)
    for h in range(H):
        keep, mult = dropout_keep(np.arange(N), np.arange(N), h, seed, offset, p)
        if causal:
            keep &= np.tril(np.ones((N, N), bool))
        want = np.stack([keep[:, c::d].sum(axis=1) for c in range(d)], axis=1)
        kept = np.rint(got[0, h] * count[:, None] / mult)
        assert np.array_equal(kept, want), h


# A window at least as wide as the sequence hides nothing.  Causal work with a
# window runs one workgroup per tile in head order; without one, the persistent
# grid over tile pairs or, when every tile fits on the GPU at once and the heads
# split evenly over the 8 XCDs, one workgroup per tile in the spread order: the
# schedules must give bitwise the same outputs (every tile is computed the same
# way, only their assignment to workgroups differs).  B=8 H=32 takes the tile
# pairs; the other shapes take the spread order wherever their heads split
# evenly over the XCDs, the 8 x 65 tiles of N = 8300 in all three kernels, with
# rounds in both directions and a partial last round.  The dropout case has
# whole query tiles: in a ragged last tile the rows past N see a band that does
# depend on the window, and as a wave moves the reference of all its rows
# together, the rows before N can then differ in rounding (not beyond).
@pytest.mark.parametrize("dtype,d,B,H,hkv,N,p", [("f16", 64, 8, 32, None, 1024, 0.0),
                                              ("bf16", 128, 1, 8, 2, 2000, 0.0),
                                              ("f16", 64, 2, 4, None, 768, 0.1),
                                              ("f16", 64, 1, 8, None, 8300, 0.0)])
def test_persistent_grid_equals_one_workgroup_per_tile(dtype, d, B, H, hkv, N, p):
    say(f"[case] persistent vs per-tile grid: B={B} H={H} hkv={hkv} N={N} d={d} {dtype} p={p}")
    q, k, v, do = (t.to("cuda") for t in make_inputs(B, H, N, d, dtype, hkv=hkv))
    outs = []
    for window in (0, N + 5):
        kw = dict(causal=True, scale=1.0 / np.sqrt(d), window=window, dropout_p=p, seed=7)
        o, lse = fa_fwd(q, k, v, **kw)
        outs.append((o, lse) + tuple(fa_bwd(q, k, v, o, do, lse, **kw)))
    torch.cuda.synchronize()
    for name, a, b in zip(("O", "LSE", "dQ", "dK", "dV"), *outs):
        assert torch.equal(a, b), name
