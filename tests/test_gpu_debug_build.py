"""The debug library (include/fa_debug.h; MI355X only).

1. NaN-filled LDS: every tiled kernel of the debug build fills its LDS with NaN
   before first use.  Its outputs must equal the production library's bit for
   bit (and be finite), on ragged shapes, masks, windows, grouped heads,
   dropout, the decode shape, the FP8 path and the float32 path: no kernel
   reads LDS it has not written.  The float32 kernels of the debug build also
   run on a grid of at most 3 row blocks per head, each workgroup looping over
   many, so the same equality covers that loop (which the production library
   reaches only past N = 524,280).
2. Tile visits: the forward, dQ and dK/dV kernels of the debug build count the
   tiles they load.  A tile must be loaded exactly when some row of the
   workgroup sees some key of it under the visibility definition (the
   oracle's ``visibility``: causal, window, block mask) -- so only kept blocks
   of a block-sparse mask are touched (block-sparse paragraph of the
   agihunt.info summary of the paper), and no key tile entirely in the future
   of a causal query tile (causal-mask section of the marketmaker.cc
   article)."""

import numpy as np
import pytest
import torch

from io_aware_exact_fwd_amd import binding, fa_bwd, fa_fwd, fa_fwd_decode, fa_fwd_fp8
from io_aware_exact_fwd_amd.build import LIB_DEBUG
from io_aware_exact_fwd_amd.workloads import (butterfly_block_mask, make_decode_inputs, make_inputs,
                                              make_signs)
from oracle import visibility

from gpu_util import say

pytestmark = pytest.mark.gpu


def _holes(nb):
    bm = butterfly_block_mask(nb)
    bm[:, 1] = 0
    bm[2, :] = 0
    return bm


CASES = [
    # name, B, H, hkv, N, d, dtype, causal, window, mask, dropout
    ("dense-f16-d64-ragged-causal", 2, 2, 2, 1000, 64, "f16", True, 0, None, 0.0),
    # 8 heads, every tile resident: the three kernels in the spread order
    ("spread-bf16-d64-causal", 2, 4, 4, 1500, 64, "bf16", True, 0, None, 0.0),
    ("dense-bf16-d128-ragged", 1, 3, 3, 777, 128, "bf16", False, 0, None, 0.0),
    ("window-f16-d64", 1, 2, 2, 1500, 64, "f16", True, 300, None, 0.0),
    ("window-bf16-d128-twosided", 1, 2, 2, 1300, 128, "bf16", False, 200, None, 0.0),
    ("blocks-f16-d64", 1, 4, 2, 1024, 64, "f16", False, 0, "holes", 0.0),
    ("blocks-bf16-d128-causal", 1, 2, 2, 1024, 128, "bf16", True, 0, "holes", 0.0),
    ("dropout-f16-d64", 1, 2, 2, 640, 64, "f16", True, 0, None, 0.25),
    ("dropout-bf16-d128", 1, 2, 1, 513, 128, "bf16", False, 0, None, 0.25),
]


def _run(case, lib_path=None, visits=None):
    name, B, H, hkv, N, d, dtype, causal, window, mask, p = case
    dev = torch.device("cuda:0")
    q, k, v, do = (t.to(dev) for t in make_inputs(B, H, N, d, dtype, hkv=hkv))
    bm = None if mask is None else _holes(N // 128)
    bmd = None if bm is None else torch.as_tensor(bm, device=dev)
    kw = dict(causal=causal, scale=1.0 / np.sqrt(d), block_mask=bmd, mask_block=128,
              window=window, dropout_p=p, seed=77, offset=3)
    o, lse = fa_fwd(q, k, v, **kw)
    g = fa_bwd(q, k, v, o, do, lse, **kw)
    torch.cuda.synchronize()
    return (o, lse, *g), bm


F32_CASES = [
    ("f32-d64-ragged-causal", 1, 2, 2, 1000, 64, "f32", True, 0, None, 0.0),
    ("f32-d128-window-gqa", 1, 4, 2, 700, 128, "f32", False, 150, None, 0.0),
    ("f32-d64-blocks-dropout", 1, 2, 1, 1024, 64, "f32", True, 0, "holes", 0.25),
]


@pytest.mark.parametrize("case", CASES + F32_CASES, ids=[c[0] for c in CASES + F32_CASES])
def test_nan_filled_lds_changes_nothing(case):
    say(f"[case] NaN LDS {case[0]}")
    prod, _ = _run(case)
    with binding.use_library(LIB_DEBUG):
        dbg, _ = _run(case)
    for a, b in zip(prod, dbg):
        assert torch.equal(a, b), case[0]
        assert not torch.isnan(b.float()).any(), case[0]


def test_nan_filled_lds_decode_and_fp8():
    say("[case] NaN LDS decode, FP8")
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in make_decode_inputs(2, 8, 3000, 128, 3, "bf16", hkv=2))
    x, y, z, _ = (t.to(dev) for t in make_inputs(1, 2, 1000, 64, "f16"))
    s = make_signs(64).to(dev)
    outs = []
    for path in (None, LIB_DEBUG):
        ctx = binding.use_library(path) if path else torch.no_grad()
        with ctx:
            od, ld = fa_fwd_decode(q, k, v, causal=True)
            o8, l8 = fa_fwd_fp8(x, y, z, s, True)
            torch.cuda.synchronize()
            outs.append((od, ld, o8, l8))
    for a, b in zip(*outs):
        assert torch.equal(a, b) and not torch.isnan(b.float()).any()


def _key_tile(d, dtype, dropout):
    return 64 if d == 64 or dropout > 0 else 32


def _expected_visits(case, bm):
    """Tile visits the definition needs, in the layout of fa_debug.h."""
    name, B, H, hkv, N, d, dtype, causal, window, mask, p = case
    nb = (N + 127) // 128
    want = np.zeros((3, nb, nb), np.int64)  # the same for every head
    # forward key tiles: 64 keys (32 at head dim 128 without dropout); dQ: 64
    for kern, kt in ((0, _key_tile(d, dtype, p)), (1, 64)):
        for qt in range(nb):
            rows = np.arange(qt * 128, min(N, qt * 128 + 128))
            for k0 in range(0, N, kt):
                keys = np.arange(k0, min(N, k0 + kt))
                if visibility(rows, keys, causal, bm, 128, window).any():
                    want[kern, qt, k0 // 128] += kt
    for t in range(nb):  # dK/dV: 128-key tile t, 64-query steps
        keys = np.arange(t * 128, min(N, t * 128 + 128))
        for qs in range(0, N, 64):
            rows = np.arange(qs, min(N, qs + 64))
            if visibility(rows, keys, causal, bm, 128, window).any():
                want[2, t, qs // 128] += 64
    return want


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_tiles_loaded_are_exactly_the_needed_ones(case):
    name, B, H, hkv, N, d, dtype, causal, window, mask, p = case
    say(f"[case] tile visits {name}")
    nb = (N + 127) // 128
    dev = torch.device("cuda:0")
    visits = torch.zeros(3 * B * H * nb * nb, dtype=torch.int32, device=dev)
    with binding.use_library(LIB_DEBUG):
        binding.fa_debug_set_tile_visits(visits)
        try:
            _, bm = _run(case)
        finally:
            binding.fa_debug_set_tile_visits(None)
    got = visits.cpu().numpy().reshape(3, B * H, nb, nb)
    want = _expected_visits(case, bm)
    for h in range(B * H):
        for kern, label in enumerate(("forward", "dQ", "dK/dV")):
            bad = np.argwhere(got[kern, h] != want[kern])
            assert bad.size == 0, (name, label, h, bad[:5].tolist(),
                                   got[kern, h][tuple(bad[0])], want[kern][tuple(bad[0])])
    say(f"[case] {name}: {int(got.sum())} keys/queries loaded, all needed")
