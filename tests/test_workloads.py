"""Host-side checks of the workload module (inputs, masks, work accounting)."""

import numpy as np
import torch

from io_aware_exact_fwd_amd import workloads as wl


def test_butterfly_mask_properties():
    bm = wl.butterfly_block_mask(512)
    assert bm.dtype == np.uint8 and bm.shape == (512, 512)
    assert np.all(bm.sum(axis=1) == 10)  # diagonal + 9 single-bit neighbours
    assert bm.sum() == 5120
    assert np.array_equal(bm, bm.T)
    # brute-force the rule on a sample of rows
    for i in (0, 1, 77, 300, 511):
        for j in range(512):
            want = i == j or bin(i ^ j).count("1") == 1
            assert bool(bm[i, j]) == want


def test_kept_pairs():
    assert wl.kept_pairs_per_head(1024, True) == 1024 * 1025 // 2
    assert wl.kept_pairs_per_head(256, False) == 65536
    bm = wl.butterfly_block_mask(512)
    assert wl.kept_pairs_per_head(65536, False, bm, 128) == 10 * 512 * 128 * 128
    small = wl.butterfly_block_mask(8)
    dense = np.kron(small, np.ones((4, 4))) != 0
    causal_dense = dense & np.tril(np.ones((32, 32), bool))
    assert wl.kept_pairs_per_head(32, True, small, 4) == causal_dense.sum()


def test_headline_flops():
    w = wl.WORKLOADS["gpt2_medium"]
    assert abs(wl.fwd_flops(w) / 1e9 - 137.57) < 0.01
    assert abs((wl.fwd_flops(w) + wl.bwd_flops(w)) / 1e9 - 481.51) < 0.01
    assert abs(wl.fwd_compulsory_bytes(w) / 1e6 - 541.1) < 0.1


def test_inputs_seeded_and_rounded():
    q, k, v, do = wl.make_inputs(1, 2, 16, 8, "bf16")
    q2, *_ = wl.make_inputs(1, 2, 16, 8, "bf16")
    assert q.dtype == torch.bfloat16 and q.shape == (1, 2, 16, 8)
    assert torch.equal(q, q2)
    g = torch.Generator("cpu").manual_seed(1016)
    ref = torch.randn((1, 2, 16, 8), generator=g)
    assert torch.equal(q, ref.to(torch.bfloat16))
    assert not torch.equal(q, k)
