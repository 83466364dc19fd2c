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


def test_kept_pairs_with_window_match_the_oracle_visibility():
    from oracle import visibility

    for n, causal, w, bm, mb in ((40, True, 7, None, 4), (40, False, 7, None, 4),
                                 (32, True, 5, wl.butterfly_block_mask(8), 4),
                                 (32, False, 100, wl.butterfly_block_mask(8), 4),
                                 (33, False, 1, None, 4)):
        want = visibility(np.arange(n), np.arange(n), causal, bm, mb, w).sum()
        assert wl.kept_pairs_per_head(n, causal, bm, mb, w) == want
    # the pages' sliding-window example: N = 8192, W = 512, causal
    assert wl.kept_pairs_per_head(8192, True, window=512) == 512 * 513 // 2 + (8192 - 512) * 512


def test_grouped_inputs_share_the_stream():
    q, k, v, do = wl.make_inputs(2, 4, 16, 8, "f16", hkv=2)
    assert q.shape == (2, 4, 16, 8) and k.shape == (2, 2, 16, 8) and do.shape == q.shape
    q1, k1, *_ = wl.make_inputs(2, 4, 16, 8, "f16")
    assert torch.equal(q, q1) and not torch.equal(k, k1[:, :2])
    w = wl.WORKLOADS["gqa_h64_kv8"]
    x = w.N * w.d * 2
    assert wl.fwd_compulsory_bytes(w) == w.B * (w.H * (2 * x + 4 * w.N) + w.H_kv * 2 * x)


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


def test_bench_units_follow_window_and_grouped_heads():
    """bench.py's per-kernel units: the window's pairs (not the full causal
    triangle) and K/V tensors with H_kv heads; the headline is unchanged."""
    import bench

    lw, full = wl.WORKLOADS["long_window"], wl.WORKLOADS["long_wide"]
    u_lw, u_full = bench.kernel_work(lw), bench.kernel_work(full)
    pairs = wl.kept_pairs_per_head(lw.N, lw.causal, None, 128, lw.window) * lw.B * lw.H
    assert u_lw["fwd"]["flops"] == 4.0 * lw.d * pairs
    assert u_lw["fwd"]["flops"] < u_full["fwd"]["flops"] / 8  # W = 512 of N = 8192
    assert u_lw["dkdv"]["bytes"] == u_full["dkdv"]["bytes"]     # bytes do not depend on W

    g = wl.WORKLOADS["gqa_h64_kv8"]
    x = g.B * g.H * g.N * g.d * g.elem_bytes
    xkv = g.B * g.H_kv * g.N * g.d * g.elem_bytes
    n4 = g.B * g.H * g.N * 4
    u = bench.kernel_work(g)
    assert u["fwd"]["bytes"] == 2 * x + 2 * xkv + n4
    assert u["dkdv"]["bytes"] == 2 * x + 4 * xkv + 2 * n4

    h = wl.WORKLOADS["gpt2_medium"]
    assert bench.kernel_work(h)["fwd"]["bytes"] == 541_065_216  # Q, K, V, O and LSE once
