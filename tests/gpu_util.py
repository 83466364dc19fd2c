"""Shared helpers of the GPU parity tests: run the HIP path, run the oracle on
the same seeded inputs, compare with the stated tolerances."""

from __future__ import annotations

import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

from io_aware_exact_fwd_amd import fa_bwd, fa_fwd
from io_aware_exact_fwd_amd.workloads import make_inputs
from oracle import attention_backward, attention_forward

# Tolerances: fp16 max|O - O_ref| <= 2e-3, bf16 <= 1e-2; |LSE - LSE_ref| <= 1e-3;
# relative Frobenius error of dQ, dK, dV <= 1e-2.  float32 inputs are gated at
# the fp16 numbers (and are expected to land near 1e-6).
O_TOL = {"f16": 2e-3, "bf16": 1e-2, "f32": 2e-3}
LSE_TOL = 1e-3
GRAD_TOL = 1e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_fro(x, ref):
    den = np.linalg.norm(ref)
    num = np.linalg.norm(x - ref)
    return num / den if den > 0 else num


def run_gpu(q, k, v, do, causal, scale, block_mask, mask_block, backward=True, atomic_dq=False,
            **ext):
    dev = torch.device("cuda:0")
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    bm = None if block_mask is None else torch.as_tensor(block_mask, dtype=torch.uint8, device=dev)
    o, lse = fa_fwd(qd, kd, vd, causal=causal, scale=scale, block_mask=bm, mask_block=mask_block,
                    **ext)
    grads = None
    if backward:
        grads = fa_bwd(qd, kd, vd, o, dod, lse, causal=causal, scale=scale, block_mask=bm,
                       mask_block=mask_block, atomic_dq=atomic_dq, **ext)
    torch.cuda.synchronize()
    return o, lse, grads


def _workers():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _group_selection(sel, g):
    """Query heads of ``sel`` grouped by the K/V head they read, in order.
    Every K/V head touched must have all g of its query heads selected."""
    groups = {}
    for b, h in sel:
        groups.setdefault((b, h // g), []).append((b, h))
    for key, hs in groups.items():
        assert len(hs) == g, "select whole groups of query heads"
    return groups


def compare_heads(name, qn, kn, vn, don, outs, scale, causal, block_mask, mask_block, sel, g,
                  okw, backward, o_rel=0.0):
    """Oracle of every selected head against the GPU results ``outs`` =
    (o, lse, grads or None), host float32 arrays.  One K/V head (with its
    group of query heads) per task on a thread pool with single-threaded
    BLAS.  Returns the metrics over the whole selection: max |O - O_ref|,
    max |LSE - LSE_ref| over rows with a visible key, and the relative
    Frobenius error of dQ, dK, dV (sums of squares over every selected
    head before the ratio).  o_rel > 0 reports max(|O - O_ref| - o_rel |O_ref|)
    instead of max |O - O_ref| (an output rounding of o_rel relative taken
    off before the absolute gate)."""
    from threadpoolctl import threadpool_limits

    o, lse, grads = outs
    groups = _group_selection(sel, g)

    def one(key):
        b, j = key
        st = {"o": 0.0, "lse": 0.0}
        num = {"dq": 0.0, "dk": 0.0, "dv": 0.0}
        den = {"dq": 0.0, "dk": 0.0, "dv": 0.0}
        dk_sum = dv_sum = None
        for (bb, h) in groups[key]:
            o_ref, lse_ref = attention_forward(qn, kn, vn, scale, causal, block_mask, mask_block,
                                               heads=[(bb, h)], **okw)
            o_ref, lse_ref = o_ref[0], lse_ref[0]
            o_g = o[bb, h].astype(np.float64)
            lse_g = lse[bb, h].astype(np.float64)
            assert np.all(np.isfinite(o_g)), f"{name}: non-finite O in head {(bb, h)}"
            live = np.isfinite(lse_ref)
            assert np.array_equal(np.isfinite(lse_g), live), f"{name}: -inf LSE rows differ {(bb, h)}"
            assert np.all(o_g[~live] == 0), f"{name}: rows with no visible key must be 0 {(bb, h)}"
            st["o"] = max(st["o"], float((np.abs(o_g - o_ref) - o_rel * np.abs(o_ref)).max()))
            if live.any():
                st["lse"] = max(st["lse"], float(np.abs(lse_g[live] - lse_ref[live]).max()))
            if backward:
                dq_ref, dk_ref, dv_ref = attention_backward(qn, kn, vn, don, scale, causal,
                                                            block_mask, mask_block,
                                                            heads=[(bb, h)], **okw)
                dq_g = grads[0][bb, h].astype(np.float64)
                assert np.all(np.isfinite(dq_g)), f"{name}: non-finite dq {(bb, h)}"
                num["dq"] += float(np.sum((dq_g - dq_ref[0]) ** 2))
                den["dq"] += float(np.sum(dq_ref[0] ** 2))
                dk_sum = dk_ref[0] if dk_sum is None else dk_sum + dk_ref[0]
                dv_sum = dv_ref[0] if dv_sum is None else dv_sum + dv_ref[0]
        if backward:
            for nm, ref, gt in (("dk", dk_sum, grads[1]), ("dv", dv_sum, grads[2])):
                x = gt[b, j].astype(np.float64)
                assert np.all(np.isfinite(x)), f"{name}: non-finite {nm} {(b, j)}"
                num[nm] += float(np.sum((x - ref) ** 2))
                den[nm] += float(np.sum(ref ** 2))
        return st, num, den

    with threadpool_limits(1):
        with ThreadPoolExecutor(_workers()) as ex:
            parts = list(ex.map(one, list(groups)))
    err = {"o": max(p[0]["o"] for p in parts), "lse": max(p[0]["lse"] for p in parts)}
    if backward:
        for nm in ("dq", "dk", "dv"):
            n = sum(p[1][nm] for p in parts)
            d = sum(p[2][nm] for p in parts)
            err[nm] = float(np.sqrt(n / d)) if d > 0 else float(np.sqrt(n))
    err["heads"] = len(sel)
    return err


def _host32(t):
    return t.detach().float().cpu().numpy()


def check_case(name, B, H, N, d, dtype, causal, scale=None, block_mask=None, mask_block=128,
               heads=None, backward=True, seed=None, window=0, hkv=None, dropout=None,
               inputs=None, atomic_dq=False, o_rel=0.0):
    """Run one case on the GPU and compare the selected heads (default: every
    head, i.e. the whole tensors) with the oracle.

    hkv: K/V heads (grouped-query attention); dropout: (p, seed, offset);
    inputs: (q, k, v, dO) CPU tensors to use instead of ``make_inputs``;
    atomic_dq: run the single-pass backward (FA_BWD_ATOMIC_DQ); o_rel: see
    ``compare_heads`` (0: the plain absolute gate on O).
    Returns a dict of the observed errors."""
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    ext = {"window": window}
    okw = {"window": window}
    if dropout is not None:
        ext.update(dropout_p=dropout[0], seed=dropout[1], offset=dropout[2])
        okw.update(dropout_p=dropout[0], seed=dropout[1], offset=dropout[2])
    say(f"[case] {name}: B={B} H={H} H_kv={hkv or H} N={N} d={d} {dtype} causal={causal} "
        f"mask={'none' if block_mask is None else 'blocks'} window={window} "
        f"dropout={dropout} heads={'all' if heads is None else heads}"
        f"{' single-pass' if atomic_dq else ''}")
    q, k, v, do = make_inputs(B, H, N, d, dtype, seed, hkv=hkv) if inputs is None else inputs
    g = H // (hkv or H)
    o, lse, grads = run_gpu(q, k, v, do, causal, scale, block_mask, mask_block, backward,
                            atomic_dq, **ext)
    outs = (_host32(o), _host32(lse), None if grads is None else tuple(_host32(t) for t in grads))
    del o, lse, grads
    sel = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    qn, kn, vn, don = (x.float().numpy() for x in (q, k, v, do))
    err = compare_heads(name, qn, kn, vn, don, outs, scale, causal, block_mask, mask_block, sel,
                        g, okw, backward, o_rel)
    say(f"[case] {name}: errors {err}")
    assert err["o"] <= O_TOL[dtype], (name, "O", err)
    assert err["lse"] <= LSE_TOL, (name, "LSE", err)
    if backward:
        for nm in ("dq", "dk", "dv"):
            assert err[nm] <= GRAD_TOL, (name, nm, err)
    return err
