"""The no-allocation decode entry point (fa_fwd_decode_noalloc; MI355X only).

Called through the C ABI (the binding passes the caller's buffers, no
workspace) and compared with fa_fwd_decode, which runs the same kernels on a
workspace the caller allocates: O and LSE must be bitwise equal, and both
within the oracle's tolerances.  Two calls in a row on the shared static
scratch, the second with a smaller problem (fewer rows and splits, another
dtype and head dimension), so stale partials of the first call would show."""

import numpy as np
import pytest
import torch

from io_aware_exact_fwd_amd import fa_fwd_decode, fa_fwd_decode_noalloc
from io_aware_exact_fwd_amd.binding import NOALLOC_SCRATCH_BYTES, fa_decode_workspace_size, make_problem
from io_aware_exact_fwd_amd.workloads import make_decode_inputs
from oracle import attention_forward

from gpu_util import LSE_TOL, O_TOL, say, to_np

pytestmark = pytest.mark.gpu


def _run(B, H, hkv, N, nq, d, dtype, causal, window=0):
    say(f"[case] noalloc decode B={B} H={H} H_kv={hkv} N={N} n_q={nq} d={d} {dtype} "
        f"causal={causal} window={window}")
    q, k, v = make_decode_inputs(B, H, N, d, nq, dtype, hkv=hkv)
    dev = torch.device("cuda:0")
    qd, kd, vd = (x.to(dev) for x in (q, k, v))
    p = make_problem(kd, causal, None, None, 128, kd, window)
    p.H = H
    need = fa_decode_workspace_size(p, nq)
    assert 0 < need <= NOALLOC_SCRATCH_BYTES, need  # the split path, inside the scratch
    o_ref_gpu, lse_ref_gpu = fa_fwd_decode(qd, kd, vd, causal=causal, window=window)
    out = torch.empty_like(qd)
    lse = torch.empty((B, H, nq), dtype=torch.float32, device=dev)
    o, l = fa_fwd_decode_noalloc(qd, kd, vd, causal=causal, window=window, out=out, lse=lse)
    torch.cuda.synchronize()
    assert o.data_ptr() == out.data_ptr() and l.data_ptr() == lse.data_ptr()
    assert torch.equal(o, o_ref_gpu) and torch.equal(l, lse_ref_gpu)
    o_ref, lse_ref = attention_forward(*(x.float().numpy() for x in (q, k, v)),
                                       1.0 / np.sqrt(d), causal, window=window, q_offset=N - nq)
    err_o = float(np.abs(to_np(o) - o_ref).max())
    err_l = float(np.abs(to_np(l) - lse_ref).max())
    say(f"[case] noalloc decode: O {err_o:.2e} LSE {err_l:.2e}, scratch {need} bytes")
    assert err_o <= O_TOL[dtype] and err_l <= LSE_TOL
    return need


def test_noalloc_decode_matches_workspace_entry_two_calls():
    big = _run(8, 64, 8, 8192, 1, 128, "bf16", True)
    small = _run(2, 8, 2, 1000, 3, 64, "f16", True, window=300)
    assert small < big


def test_noalloc_decode_rejects_problem_beyond_scratch():
    from io_aware_exact_fwd_amd.binding import FaError

    dev = torch.device("cuda:0")
    q = torch.zeros((1, 8, 16, 128), dtype=torch.bfloat16, device=dev)
    k = torch.zeros((1, 1, 65536, 128), dtype=torch.bfloat16, device=dev)
    with pytest.raises(FaError, match="static scratch"):
        fa_fwd_decode_noalloc(q, k, k, causal=True)
