"""Skipped tiles are never used (MI355X only).

Block-sparse attention visits only the kept blocks (block-sparse paragraph of
the agihunt.info summary of the paper).  Here K and V hold NaN in every key
block that no query block keeps, and the kernels must never read those keys
into any product: O, LSE, dQ and the gradients of the kept keys stay finite
and match the oracle (which gives the unseen keys zero gradient without
reading them), and dK, dV of the poisoned keys are exactly zero.  A kernel that
loaded a skipped tile and treated any of its keys as visible would turn the
NaN into the outputs.  (With causal or windowed visibility every key is
visible to some row, so those tile skips are pinned instead by the Q = 0 tests,
whose LSE counts the visible keys of every row.)"""

import numpy as np
import pytest
import torch

from io_aware_exact_fwd_amd import fa_bwd, fa_fwd
from io_aware_exact_fwd_amd.workloads import butterfly_block_mask, make_inputs
from oracle import attention_backward, attention_forward

from gpu_util import GRAD_TOL, LSE_TOL, O_TOL, rel_fro, say, to_np

pytestmark = pytest.mark.gpu


def _poisoned_case(name, N, d, dtype, causal, bm, mb, hkv=None, window=0):
    B, H = 1, 4
    say(f"[case] {name}: N={N} d={d} {dtype} causal={causal} window={window}")
    q, k, v, do = make_inputs(B, H, N, d, dtype, hkv=hkv)
    keys = np.arange(N)
    if bm is not None:
        unseen = ~np.asarray(bm, bool).any(axis=0)          # key blocks nobody keeps
        dead = unseen[keys // mb]
    else:
        dead = np.zeros(N, bool)
    assert dead.any(), "the case must leave some keys unseen"
    kp, vp = k.clone(), v.clone()
    kp[:, :, torch.as_tensor(dead)] = float("nan")
    vp[:, :, torch.as_tensor(dead)] = float("nan")
    dev = torch.device("cuda:0")
    bmd = None if bm is None else torch.as_tensor(bm, device=dev)
    kw = dict(causal=causal, scale=1.0 / np.sqrt(d), block_mask=bmd, mask_block=mb, window=window)
    qd, kd, vd, dod = (t.to(dev) for t in (q, kp, vp, do))
    o, lse = fa_fwd(qd, kd, vd, **kw)
    dq, dk, dv = fa_bwd(qd, kd, vd, o, dod, lse, **kw)
    torch.cuda.synchronize()
    o_g, lse_g, dq_g, dk_g, dv_g = (to_np(t) for t in (o, lse, dq, dk, dv))
    assert np.all(np.isfinite(o_g)) and np.all(np.isfinite(dq_g)), name
    assert not np.isnan(lse_g).any(), name
    assert np.all(dk_g[:, :, dead] == 0) and np.all(dv_g[:, :, dead] == 0), name
    assert np.all(np.isfinite(dk_g)) and np.all(np.isfinite(dv_g)), name
    # the oracle on the clean inputs: the poisoned keys are never visible
    qn, kn, vn, don = (x.float().numpy() for x in (q, k, v, do))
    o_ref, lse_ref = attention_forward(qn, kn, vn, kw["scale"], causal, bm, mb, window=window)
    g_ref = attention_backward(qn, kn, vn, don, kw["scale"], causal, bm, mb, window=window)
    live = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(lse_g), live), name
    err_o = float(np.abs(o_g - o_ref).max())
    err_l = float(np.abs(lse_g[live] - lse_ref[live]).max())
    errs = [rel_fro(g, r) for g, r in zip((dq_g, dk_g, dv_g), g_ref)]
    say(f"[case] {name}: O {err_o:.2e} LSE {err_l:.2e} dQ,dK,dV {errs[0]:.2e},{errs[1]:.2e},"
        f"{errs[2]:.2e}; {int(dead.sum())} poisoned keys")
    assert err_o <= O_TOL[dtype] and err_l <= LSE_TOL and max(errs) <= GRAD_TOL, name


def _holes(nb):
    """Butterfly with two key blocks nobody keeps and one query block that
    keeps nothing."""
    bm = butterfly_block_mask(nb)
    bm[:, [1, nb - 2]] = 0
    bm[3, :] = 0
    return bm


@pytest.mark.parametrize("dtype,d", [("f16", 64), ("bf16", 64), ("f16", 128), ("bf16", 128)])
@pytest.mark.parametrize("causal", [False, True])
def test_unseen_key_blocks_never_read(dtype, d, causal):
    _poisoned_case(f"poison-{dtype}-d{d}-c{int(causal)}", 2048, d, dtype, causal, _holes(16), 128)


def test_unseen_key_blocks_never_read_grouped_window_mb256():
    N, mb = 2048, 256
    bm = butterfly_block_mask(N // mb)
    bm[:, 2] = 0
    _poisoned_case("poison-gqa-window-mb256", N, 64, "f16", True, bm, mb, hkv=2, window=700)
