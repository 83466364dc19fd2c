"""GPU parity of the HIP path against the fp64 oracle (MI355X only).

Small shapes span several tiles and ragged sequence ends; the five workloads
run at full size in the same launch configuration the bench times, and every
head of every output is compared with the oracle: max |O - O_ref| and
max |LSE - LSE_ref| over the whole tensors, the relative Frobenius errors of
dQ, dK, dV over the whole (B, H, N, d) tensors."""

import numpy as np
import pytest
import torch

from io_aware_exact_fwd_amd import fa_bwd, fa_fwd, fa_mask_compile
from io_aware_exact_fwd_amd.workloads import WORKLOADS, butterfly_block_mask, make_inputs

from gpu_util import check_case, say

pytestmark = pytest.mark.gpu


def _mask_with_holes(nb):
    """Butterfly, plus one query block that sees nothing and one key block
    that nobody sees (rows with -inf LSE, keys with zero gradient)."""
    bm = butterfly_block_mask(nb)
    bm[1, :] = 0
    bm[:, nb - 1] = 0
    bm[nb - 1, nb - 1] = 1
    return bm


SMALL = []
for dtype in ("f16", "bf16"):
    for d in (64, 128):
        for N in (1, 17, 129, 300):
            for causal in (False, True):
                SMALL.append((dtype, d, N, causal))
for dtype in ("f16", "bf16"):
    SMALL.append((dtype, 64, 1024, True))
    SMALL.append((dtype, 128, 513, False))


@pytest.mark.parametrize("dtype,d,N,causal", SMALL)
def test_small_dense(dtype, d, N, causal):
    check_case(f"small-{dtype}-d{d}-N{N}-c{int(causal)}", 2, 2, N, d, dtype, causal)


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("f32", 128)])
@pytest.mark.parametrize("N,causal", [(1, False), (100, True), (256, False), (257, True)])
def test_small_f32(dtype, d, N, causal):
    err = check_case(f"small-{dtype}-d{d}-N{N}-c{int(causal)}", 1, 2, N, d, dtype, causal)
    assert err["o"] < 1e-5


@pytest.mark.parametrize("dtype,d", [("f16", 64), ("bf16", 128), ("f32", 64)])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("kind", ["butterfly", "holes"])
def test_small_block_sparse(dtype, d, causal, kind):
    N, mb = 1024, 128
    bm = butterfly_block_mask(N // mb) if kind == "butterfly" else _mask_with_holes(N // mb)
    check_case(f"blocks-{kind}-{dtype}-d{d}-c{int(causal)}", 1, 3, N, d, dtype, causal,
               block_mask=bm, mask_block=mb)


def test_block_sparse_larger_mask_block():
    N, mb = 1024, 256
    bm = _mask_with_holes(N // mb)
    check_case("blocks-mb256", 1, 2, N, 64, "f16", True, block_mask=bm, mask_block=mb)


@pytest.mark.parametrize("name", ["single_head", "gpt2_small", "gpt2_medium", "long_wide",
                                  "butterfly"])
def test_workload_full_size(name):
    """Whole tensors of the workload against the oracle (every head)."""
    w = WORKLOADS[name]
    err = check_case(name, w.B, w.H, w.N, w.d, w.dtype, w.causal, w.scale, w.block_mask(),
                     w.mask_block)
    assert err["heads"] == w.B * w.H


def _lse_counts(N, causal, bm, mb):
    rows = np.arange(N)
    if bm is None:
        cnt = rows + 1 if causal else np.full(N, N)
    else:
        kept = np.asarray(bm, bool)[rows // mb]          # [N, nb]
        cnt = kept.sum(axis=1) * mb
        if causal:
            cnt = np.array([sum(min(mb, i - kb * mb + 1) for kb in np.nonzero(kept[i])[0]
                                if kb * mb <= i) for i in rows])
    return cnt


@pytest.mark.parametrize("case", ["causal8192", "butterfly", "butterfly_holes_causal"])
def test_zero_queries_lse_counts_visible_keys(case):
    """With Q = 0 every visible score is 0, so LSE_i = ln(#visible keys of row i)
    exactly: a wrong tile, block or diagonal shows up as a different count."""
    dev = torch.device("cuda:0")
    if case == "causal8192":
        N, d, causal, bm, mb, H = 8192, 128, True, None, 128, 2
    elif case == "butterfly":
        N, d, causal, bm, mb, H = 65536, 64, False, butterfly_block_mask(512), 128, 2
    else:
        N, d, causal, bm, mb, H = 4096, 64, True, _mask_with_holes(32), 128, 2
    say(f"[case] zero-q {case}")
    _, k, v, _ = make_inputs(1, H, N, d, "f16")
    q = torch.zeros_like(k)
    bmd = None if bm is None else torch.as_tensor(bm, device=dev)
    o, lse = fa_fwd(q.to(dev), k.to(dev), v.to(dev), causal=causal, scale=0.125,
                    block_mask=bmd, mask_block=mb)
    cnt = _lse_counts(N, causal, bm, mb)
    want = np.where(cnt > 0, np.log(np.maximum(cnt, 1)), -np.inf)
    got = lse.cpu().numpy().astype(np.float64)
    for h in range(H):
        live = cnt > 0
        assert np.array_equal(np.isfinite(got[0, h]), live)
        assert np.abs(got[0, h][live] - want[live]).max() <= 1e-5


def _sparse_mask_with_empty_lines(nb, density, seed):
    bm = (np.random.default_rng(seed).random((nb, nb)) < density).astype(np.uint8)
    bm[[0, 5, nb - 1], :] = 0   # query blocks that keep nothing
    bm[:, [3, nb // 2]] = 0     # key blocks nobody keeps
    return bm


def test_mask_compile_lists_exact():
    """Row and column lists against numpy, bit for bit: sizes below and above
    one row or column per thread of the compile kernels (256), a size that
    leaves the last thread a partial chunk, empty rows and columns, a dense
    mask and the one-block masks."""
    dev = torch.device("cuda:0")
    for bm in (butterfly_block_mask(512), _mask_with_holes(16),
               (np.random.default_rng(0).random((37, 37)) < 0.3).astype(np.uint8),
               _sparse_mask_with_empty_lines(777, 0.05, 1), np.ones((300, 300), np.uint8),
               np.ones((1, 1), np.uint8), np.zeros((1, 1), np.uint8)):
        say(f"[case] mask compile nb={bm.shape[0]}")
        row_ptr, col_idx, col_ptr, row_idx = fa_mask_compile(torch.as_tensor(bm, device=dev))
        b = bm != 0
        rp = np.concatenate([[0], np.cumsum(b.sum(axis=1))])
        cp = np.concatenate([[0], np.cumsum(b.sum(axis=0))])
        assert np.array_equal(row_ptr.cpu().numpy(), rp)
        assert np.array_equal(col_ptr.cpu().numpy(), cp)
        assert np.array_equal(col_idx.cpu().numpy(), np.nonzero(b)[1])
        assert np.array_equal(row_idx.cpu().numpy(), np.nonzero(b.T)[1])


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_bitwise_repeatable(dtype):
    dev = torch.device("cuda:0")
    say(f"[case] repeatable {dtype}")
    q, k, v, do = (t.to(dev) for t in make_inputs(2, 4, 1000, 64, dtype))
    o1, l1 = fa_fwd(q, k, v, causal=True)
    o2, l2 = fa_fwd(q, k, v, causal=True)
    g1 = fa_bwd(q, k, v, o1, do, l1, causal=True)
    g2 = fa_bwd(q, k, v, o1, do, l1, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def test_autograd_wrapper_matches_entry_points():
    from io_aware_exact_fwd_amd import attention

    dev = torch.device("cuda:0")
    say("[case] autograd wrapper")
    q, k, v, do = (t.to(dev) for t in make_inputs(1, 2, 256, 64, "f16"))
    qr, kr, vr = (t.clone().requires_grad_(True) for t in (q, k, v))
    o = attention(qr, kr, vr, causal=True, scale=0.125)
    o.backward(do)
    o2, lse = fa_fwd(q, k, v, causal=True, scale=0.125)
    g = fa_bwd(q, k, v, o2, do, lse, causal=True, scale=0.125)
    assert torch.equal(o, o2)
    for a, b in zip((qr.grad, kr.grad, vr.grad), g):
        assert torch.equal(a, b)


def test_backward_stages_equal_fused_entry_point():
    from io_aware_exact_fwd_amd import bwd_workspace, fa_bwd_dkdv, fa_bwd_dq

    dev = torch.device("cuda:0")
    say("[case] backward stages")
    bm = torch.as_tensor(_mask_with_holes(8), device=dev)
    q, k, v, do = (t.to(dev) for t in make_inputs(1, 2, 1024, 64, "f16"))
    o, lse = fa_fwd(q, k, v, causal=True, scale=0.125, block_mask=bm, mask_block=128)
    g = fa_bwd(q, k, v, o, do, lse, causal=True, scale=0.125, block_mask=bm, mask_block=128)
    p, ws, ws_n, _ = bwd_workspace(q, True, 0.125, bm, 128)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    fa_bwd_dq(p, q, k, v, o, do, lse, dq, ws, ws_n)
    fa_bwd_dkdv(p, q, k, v, do, lse, dk, dv, ws, ws_n)
    torch.cuda.synchronize()
    for a, b in zip(g, (dq, dk, dv)):
        assert torch.equal(a, b)


def test_shared_workspace_reuses_block_lists():
    """A forward and a backward given one workspace: the backward called with
    FA_REUSE_LISTS (lists left by the forward) gives bitwise the results of
    separate calls that each compile the mask, also through the two stages."""
    from io_aware_exact_fwd_amd import bwd_workspace, fa_bwd_dkdv, fa_bwd_dq, fa_workspace_size
    from io_aware_exact_fwd_amd.binding import make_problem

    dev = torch.device("cuda:0")
    say("[case] shared workspace, block lists reused")
    bm = torch.as_tensor(_mask_with_holes(8), device=dev)
    q, k, v, do = (t.to(dev) for t in make_inputs(1, 4, 1024, 64, "f16", hkv=2))
    kw = dict(causal=True, scale=0.125, block_mask=bm, mask_block=128, window=500)
    o1, l1 = fa_fwd(q, k, v, **kw)
    g1 = fa_bwd(q, k, v, o1, do, l1, **kw)
    p = make_problem(q, True, 0.125, bm, 128, k, 500)
    ws = torch.empty(fa_workspace_size(p, 1), dtype=torch.uint8, device=dev)
    assert fa_workspace_size(p, 1) >= fa_workspace_size(p, 0) > 0
    o2, l2 = fa_fwd(q, k, v, workspace=ws, **kw)
    g2 = fa_bwd(q, k, v, o2, do, l2, workspace=ws, reuse_lists=True, **kw)
    p3, ws3, ws3_n, bm3 = bwd_workspace(q, k=k, reuse_lists=True, **kw)
    o3, l3 = fa_fwd(q, k, v, workspace=ws3, **kw)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    fa_bwd_dq(p3, q, k, v, o3, do, l3, dq, ws3, ws3_n)
    fa_bwd_dkdv(p3, q, k, v, do, l3, dk, dv, ws3, ws3_n)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2) and torch.equal(o1, o3)
    for a, b, c in zip(g1, g2, (dq, dk, dv)):
        assert torch.equal(a, b) and torch.equal(a, c)
