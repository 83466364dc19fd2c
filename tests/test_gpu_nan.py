"""NaN inputs through the forward (MI355X only).

The pages do not define attention on NaN inputs; the reading taken is that a
NaN propagates to exactly the rows whose softmax includes it: a NaN in key j
makes O and LSE of every row that sees key j NaN and leaves every other row as
it is, and a NaN in query i makes row i NaN.  The forward's running maximum is
an IEEE maximum that propagates NaN, and masked scores are replaced by -inf
before any exponential, so a hidden NaN key contributes nothing.  Rows that do
not see the NaN are compared with the oracle on the clean inputs (the oracle's
masking drops hidden keys the same way)."""

import numpy as np
import pytest
import torch

from io_aware_exact_fwd_amd import fa_fwd
from io_aware_exact_fwd_amd.workloads import make_inputs
from oracle import attention_forward

from gpu_util import LSE_TOL, O_TOL, say, to_np

pytestmark = pytest.mark.gpu

CASES = [(N, d, dtype) for N in (300, 1024) for d in (64, 128) for dtype in ("f16", "bf16")]


@pytest.mark.parametrize("N,d,dtype", CASES)
def test_nan_key_reaches_only_rows_that_see_it(N, d, dtype):
    say(f"[case] NaN key: N={N} d={d} {dtype} causal")
    j0 = N // 2 + 3
    q, k, v, _ = make_inputs(1, 2, N, d, dtype)
    kp = k.clone()
    kp[:, :, j0] = float("nan")
    dev = torch.device("cuda:0")
    scale = 1.0 / np.sqrt(d)
    o, lse = fa_fwd(q.to(dev), kp.to(dev), v.to(dev), causal=True, scale=scale)
    torch.cuda.synchronize()
    o_g, lse_g = to_np(o), to_np(lse)
    sees = np.arange(N) >= j0
    assert np.isnan(lse_g[:, :, sees]).all() and np.isnan(o_g[:, :, sees]).all()
    assert np.isfinite(lse_g[:, :, ~sees]).all() and np.isfinite(o_g[:, :, ~sees]).all()
    o_ref, lse_ref = attention_forward(q.float().numpy(), k.float().numpy(), v.float().numpy(), scale, True)
    err_o = float(np.abs(o_g[:, :, ~sees] - o_ref[:, :, ~sees]).max())
    err_l = float(np.abs(lse_g[:, :, ~sees] - lse_ref[:, :, ~sees]).max())
    say(f"  rows before the NaN key: max|O - O_ref| {err_o:.2e}, max|LSE - LSE_ref| {err_l:.2e}")
    assert err_o <= O_TOL[dtype] and err_l <= LSE_TOL


@pytest.mark.parametrize("N,d,dtype", CASES)
def test_nan_query_reaches_only_its_row(N, d, dtype):
    say(f"[case] NaN query: N={N} d={d} {dtype} non-causal")
    i0 = N // 3
    q, k, v, _ = make_inputs(1, 2, N, d, dtype)
    qp = q.clone()
    qp[:, :, i0] = float("nan")
    dev = torch.device("cuda:0")
    scale = 1.0 / np.sqrt(d)
    o, lse = fa_fwd(qp.to(dev), k.to(dev), v.to(dev), causal=False, scale=scale)
    torch.cuda.synchronize()
    o_g, lse_g = to_np(o), to_np(lse)
    row = np.arange(N) == i0
    assert np.isnan(lse_g[:, :, row]).all() and np.isnan(o_g[:, :, row]).all()
    o_ref, lse_ref = attention_forward(q.float().numpy(), k.float().numpy(), v.float().numpy(), scale, False)
    err_o = float(np.abs(o_g[:, :, ~row] - o_ref[:, :, ~row]).max())
    err_l = float(np.abs(lse_g[:, :, ~row] - lse_ref[:, :, ~row]).max())
    say(f"  other rows: max|O - O_ref| {err_o:.2e}, max|LSE - LSE_ref| {err_l:.2e}")
    assert err_o <= O_TOL[dtype] and err_l <= LSE_TOL
