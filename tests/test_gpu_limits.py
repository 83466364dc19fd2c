"""GPU parity at the largest head the library accepts (MI355X only).

One head of Q, K or V may take up to 2^31 - 1 bytes (32-bit buffer offsets):
N = (2^31 - 1) // (d * 2) = 8,388,607 rows at d = 128 in bf16.  A sliding
window of 256 keys keeps the work small while every tile, row and copy offset
of the largest head is exercised, including the zero-filled rows past N whose
byte offsets pass 2^31.  Inputs come from torch's seeded generator on the
device (B = H = 1, N(0, 1) rounded to bf16); the oracle checks sampled rows
on square slices that hold every key those rows see (and, for a key, every
query that sees it), so each sampled O, LSE, dQ, dK and dV row is the exact
definition's value."""

import math

import numpy as np
import pytest
import torch

from io_aware_exact_fwd_amd import fa_bwd, fa_fwd
from oracle import attention_backward, attention_forward

from gpu_util import LSE_TOL, O_TOL, say, to_np

pytestmark = pytest.mark.gpu

D = 128
N_MAX = (2**31 - 1) // (D * 2)
W = 256


def _slice(t, a, b):
    return t[:, :, a:b].float().cpu().numpy().astype(np.float64)


def test_largest_head_windowed():
    N = N_MAX
    scale = 1.0 / math.sqrt(D)
    say(f"[case] largest head: N={N} d={D} bf16 causal window={W}")
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(4242)
    q, k, v, do = (torch.randn((1, 1, N, D), generator=g, device=dev).to(torch.bfloat16)
                   for _ in range(4))
    o, lse = fa_fwd(q, k, v, causal=True, scale=scale, window=W)
    dq, dk, dv = fa_bwd(q, k, v, o, do, lse, causal=True, scale=scale, window=W)
    torch.cuda.synchronize()

    rng = np.random.default_rng(7)
    rows = sorted(set([0, 1, W - 1, W, 2**22, 2**22 + 1, N // 2, N - W, N - 2, N - 1]
                      + [int(x) for x in rng.integers(0, N, 8)]))
    err_o = err_l = 0.0
    dq_num = dq_den = dk_num = dk_den = dv_num = dv_den = 0.0
    for i in rows:
        # query row i: keys i - W + 1 .. i, all inside the slice [a, i]
        a = max(0, i - W + 1)
        qs, ks, vs, dos = (_slice(t, a, i + 1) for t in (q, k, v, do))
        o_ref, lse_ref = attention_forward(qs, ks, vs, scale, True, window=W)
        dq_ref, _, _ = attention_backward(qs, ks, vs, dos, scale, True, window=W)
        o_g = to_np(o[0, 0, i])
        err_o = max(err_o, float(np.abs(o_g - o_ref[0, 0, -1]).max()))
        err_l = max(err_l, abs(float(lse[0, 0, i]) - float(lse_ref[0, 0, -1])))
        dq_num += float(np.sum((to_np(dq[0, 0, i]) - dq_ref[0, 0, -1]) ** 2))
        dq_den += float(np.sum(dq_ref[0, 0, -1] ** 2))
        # key j = i: queries j .. j + W - 1 see it, and they see keys from
        # j - W + 1 on: the slice [a, c) holds them all (earlier rows of the
        # slice do not see key j and add nothing to its gradient)
        c = min(N, i + W)
        qs, ks, vs, dos = (_slice(t, a, c) for t in (q, k, v, do))
        _, dk_ref, dv_ref = attention_backward(qs, ks, vs, dos, scale, True, window=W)
        dk_num += float(np.sum((to_np(dk[0, 0, i]) - dk_ref[0, 0, i - a]) ** 2))
        dk_den += float(np.sum(dk_ref[0, 0, i - a] ** 2))
        dv_num += float(np.sum((to_np(dv[0, 0, i]) - dv_ref[0, 0, i - a]) ** 2))
        dv_den += float(np.sum(dv_ref[0, 0, i - a] ** 2))
    rel = {n: math.sqrt(x / y) for n, x, y in (("dq", dq_num, dq_den), ("dk", dk_num, dk_den),
                                             ("dv", dv_num, dv_den))}
    say(f"[case] largest head: {len(rows)} rows, max|O| err {err_o:.2e}, max|LSE| err {err_l:.2e}, "
        f"rel grads {rel}")
    assert err_o <= O_TOL["bf16"] and err_l <= LSE_TOL
    assert all(x <= 1e-2 for x in rel.values()), rel
    assert torch.isfinite(o).all() and torch.isfinite(dq).all()


def test_largest_head_fp8_windowed():
    """FP8 path on the largest head: codes of the blocks around sampled rows
    bit-exact, and their O and LSE within the FP8 bounds, against the oracle
    on 64-row-aligned slices (quantisation blocks are absolute 64-row blocks,
    so an aligned slice of whole blocks quantises the same way)."""
    from io_aware_exact_fwd_amd import fa_fwd_fp8, fp8_quantize, fp8_workspace_views
    from io_aware_exact_fwd_amd.workloads import make_signs
    from oracle.fp8 import fp8_attention_forward

    from test_gpu_fp8 import _check_attention, _v_rowmajor

    N = N_MAX
    scale = 1.0 / math.sqrt(D)
    say(f"[case] largest head, FP8: N={N} d={D} bf16 causal window={W}")
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(777)
    q, k, v = (torch.randn((1, 1, N, D), generator=g, device=dev).to(torch.bfloat16)
               for _ in range(3))
    signs = make_signs(D)
    sd = signs.to(dev)
    _, ws = fp8_quantize(q, k, v, sd, True, scale, W)
    o, lse = fa_fwd_fp8(q, k, v, sd, True, scale, W, workspace=ws)
    torch.cuda.synchronize()
    views = fp8_workspace_views(ws, 1, 1, 1, N, D)
    for i in (0, W, 2**22 + 5, N // 2 + 77, N - 65, N - 1):
        a = (max(0, i - W + 1) // 64) * 64
        b = min(N, (i // 64 + 1) * 64)
        name = f"largest head FP8, row {i} (slice {a}..{b})"
        qs, ks, vs = (_slice(t, a, b).astype(np.float32) for t in (q, k, v))
        o_ref, lse_ref, quant = fp8_attention_forward(qs, ks, vs, scale, signs.numpy(), True, W)
        for nm, key in (("q", "qc"), ("k", "kc")):
            got = views[key][0, a:b].cpu().numpy()
            assert np.array_equal(got, quant[nm][0][0, 0, :b - a]), (name, nm)
            assert np.array_equal(views[key[0] + "e"][0, a // 64:(b + 63) // 64].cpu().numpy(),
                                  quant[nm][1][0, 0]), (name, nm, "exponents")
        vt = _v_rowmajor(views["vc"][:, a // 64:(b + 63) // 64].cpu().numpy())
        assert np.array_equal(vt[0, :b - a], quant["v"][0][0, 0, :b - a]), (name, "v")
        _check_attention(name, to_np(o[:, :, a:b]), to_np(lse[:, :, a:b]), o_ref, lse_ref, quant,
                         "bf16", scale, True, W, 1, b - a, [(0, 0)], rows=np.array([i - a]))


def test_largest_head_decode():
    """Decode shape on the largest head: the last 4 positions against all N
    keys, windowed, against the oracle on the keys they see."""
    from io_aware_exact_fwd_amd import fa_fwd_decode

    N, nq = N_MAX, 4
    scale = 1.0 / math.sqrt(D)
    say(f"[case] largest head, decode: N={N} n_q={nq} d={D} bf16 causal window={W}")
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(99)
    q = torch.randn((1, 2, nq, D), generator=g, device=dev).to(torch.bfloat16)
    k, v = (torch.randn((1, 1, N, D), generator=g, device=dev).to(torch.bfloat16)
            for _ in range(2))
    o, lse = fa_fwd_decode(q, k, v, causal=True, scale=scale, window=W)
    torch.cuda.synchronize()
    a = N - nq - W + 1
    ks, vs = _slice(k, a, N), _slice(v, a, N)
    o_ref, lse_ref = attention_forward(to_np(q), ks, vs, scale, True, window=W,
                                       q_offset=N - a - nq)
    err_o = float(np.abs(to_np(o) - o_ref).max())
    err_l = float(np.abs(to_np(lse) - lse_ref).max())
    say(f"[case] largest head, decode: max|O| err {err_o:.2e}, max|LSE| err {err_l:.2e}")
    assert err_o <= O_TOL["bf16"] and err_l <= LSE_TOL
