"""C ABI checks that need no GPU: the library loads, exports every function
that include/fa.h declares, and rejects invalid problems before any launch."""

import ctypes
import math
import os
import re

import pytest

from io_aware_exact_fwd_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

pytestmark = pytest.mark.skipif(not os.path.exists(B.LIB_PATH),
                                reason="libfa_mi355x.so not built (run __graft_entry__.build())")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_binding_exports():
    assert _declared_functions() == sorted(B.EXPORTS)


def test_every_declared_symbol_is_exported():
    L = ctypes.CDLL(B.LIB_PATH)
    for name in _declared_functions():
        assert hasattr(L, name), name


def test_version_and_status_strings():
    assert B.fa_version() == 10600
    assert B.fa_status_string(0) == "ok"
    assert "workspace" in B.fa_status_string(B.FA_ERR_WORKSPACE)
    assert B.fa_status_string(12345) == "unknown status"


def _problem(**kw):
    p = B.FaProblem()
    p.B, p.H, p.N, p.d = kw.get("B", 2), kw.get("H", 3), kw.get("N", 256), kw.get("d", 64)
    p.dtype = kw.get("dtype", B.FA_F16)
    p.causal = kw.get("causal", 0)
    p.scale = kw.get("scale", 0.125)
    p.block_mask = kw.get("block_mask", None)
    p.mask_block = kw.get("mask_block", 0)
    p.window = kw.get("window", 0)
    p.H_kv = kw.get("H_kv", 0)
    p.dropout_p = kw.get("dropout_p", 0.0)
    p.seed = kw.get("seed", 0)
    p.offset = kw.get("offset", 0)
    p.flags = kw.get("flags", 0)
    return p


def test_problem_struct_layout_matches_header():
    """Field offsets of the ctypes mirror follow the C layout of fa_problem
    (natural alignment: the pointer and the 64-bit seed on 8-byte boundaries)."""
    off = {name: getattr(B.FaProblem, name).offset for name, _ in B.FaProblem._fields_}
    assert off["scale"] == 24 and off["block_mask"] == 32 and off["mask_block"] == 40
    assert off["window"] == 44 and off["H_kv"] == 48 and off["dropout_p"] == 52
    assert off["seed"] == 56 and off["offset"] == 64 and off["flags"] == 68
    assert ctypes.sizeof(B.FaProblem) == 72


def test_workspace_sizes():
    p = _problem()
    assert B.fa_workspace_size(p, 0) == 0
    dvec = 2 * 3 * 256 * 4
    assert B.fa_workspace_size(p, 1) == (dvec + 255) // 256 * 256
    pm = _problem(N=512, block_mask=0x1000, mask_block=128)
    nb = 4
    lists = 2 * 256 + 2 * ((nb * nb * 4 + 255) // 256 * 256)
    assert B.fa_workspace_size(pm, 0) == lists
    assert B.fa_workspace_size(pm, 1) == (2 * 3 * 512 * 4 + 255) // 256 * 256 + lists
    # float32 reads the dense mask directly: no lists
    assert B.fa_workspace_size(_problem(N=512, dtype=B.FA_F32, block_mask=0x1000,
                                        mask_block=128), 0) == 0
    assert B.fa_workspace_size(_problem(d=96), 1) == 0  # invalid problem


FAKE = 0x10000  # an aligned non-null address; never dereferenced (errors come first)


def _fwd(p, ws=None, ws_n=0, ptrs=(FAKE,) * 5):
    L = B.lib()
    return L.fa_fwd(ctypes.byref(p), *ptrs, ws, ws_n, None)


@pytest.mark.parametrize("kw,status", [
    ({"d": 96}, B.FA_ERR_UNSUPPORTED),
    ({"d": 32}, B.FA_ERR_UNSUPPORTED),
    ({"dtype": 7}, B.FA_ERR_UNSUPPORTED),
    ({"N": 0}, B.FA_ERR_ARG),
    ({"B": -1}, B.FA_ERR_ARG),
    ({"scale": math.inf}, B.FA_ERR_ARG),
    ({"scale": math.nan}, B.FA_ERR_ARG),
    ({"causal": 2}, B.FA_ERR_ARG),
    ({"block_mask": FAKE, "mask_block": 64}, B.FA_ERR_UNSUPPORTED),
    ({"block_mask": FAKE, "mask_block": 128, "N": 200}, B.FA_ERR_UNSUPPORTED),
    ({"N": 1 << 24, "d": 128}, B.FA_ERR_UNSUPPORTED),
    ({"scale": 0.0}, B.FA_ERR_ARG),
    ({"scale": -0.125}, B.FA_ERR_ARG),
    ({"window": -1}, B.FA_ERR_ARG),
    ({"H_kv": 2}, B.FA_ERR_ARG),          # does not divide H = 3
    ({"H_kv": -3}, B.FA_ERR_ARG),
    ({"dropout_p": 1.0}, B.FA_ERR_ARG),
    ({"dropout_p": -0.1}, B.FA_ERR_ARG),
    ({"dropout_p": math.nan}, B.FA_ERR_ARG),
    ({"flags": 4}, B.FA_ERR_ARG),          # an unknown flag bit
    ({"flags": 0x80000001}, B.FA_ERR_ARG),
])
def test_invalid_problems_rejected(kw, status):
    assert _fwd(_problem(**kw)) == status


def test_single_pass_workspace_and_stage_checks():
    """FA_BWD_ATOMIC_DQ adds the float32 dQ accumulator (B*H*N*d) after D in the
    backward workspace (16-bit dtypes only), leaves the forward's size alone,
    and is refused by the two stages of the two-kernel backward and, for
    float32, by fa_bwd -- all before any GPU call."""
    L = B.lib()
    flag = B.FA_BWD_ATOMIC_DQ
    p, pa = _problem(), _problem(flags=flag)
    acc = 2 * 3 * 256 * 64 * 4
    assert B.fa_workspace_size(pa, 0) == B.fa_workspace_size(p, 0)
    assert B.fa_workspace_size(pa, 1) == B.fa_workspace_size(p, 1) + acc
    pm, pma = (_problem(N=512, block_mask=0x1000, mask_block=128, flags=f) for f in (0, flag))
    assert B.fa_workspace_size(pma, 1) == B.fa_workspace_size(pm, 1) + acc * 2
    pf = _problem(dtype=B.FA_F32, flags=flag)
    assert B.fa_workspace_size(pf, 1) == B.fa_workspace_size(_problem(dtype=B.FA_F32), 1)
    args = [FAKE] * 9
    n = B.fa_workspace_size(pa, 1)
    assert L.fa_bwd_dq(ctypes.byref(pa), *args[:7], FAKE, n, None) == B.FA_ERR_ARG
    assert L.fa_bwd_dkdv(ctypes.byref(pa), *args[:7], FAKE, n, None) == B.FA_ERR_ARG
    assert L.fa_bwd(ctypes.byref(pa), *args, FAKE, n - 256, None) == B.FA_ERR_WORKSPACE
    assert L.fa_bwd(ctypes.byref(pf), *args, FAKE, B.fa_workspace_size(pf, 1),
                    None) == B.FA_ERR_UNSUPPORTED


def test_null_and_misaligned_pointers_rejected():
    p = _problem()
    assert _fwd(p, ptrs=(FAKE, FAKE, None, FAKE, FAKE)) == B.FA_ERR_ARG
    assert _fwd(p, ptrs=(FAKE, FAKE + 2, FAKE, FAKE, FAKE)) == B.FA_ERR_ARG
    assert B.lib().fa_fwd(None, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None) == B.FA_ERR_ARG


def test_workspace_checked_before_launch():
    pm = _problem(N=512, block_mask=FAKE, mask_block=128)
    need = B.fa_workspace_size(pm, 0)
    assert _fwd(pm, ws=None, ws_n=0) == B.FA_ERR_WORKSPACE
    assert _fwd(pm, ws=FAKE, ws_n=need - 1) == B.FA_ERR_WORKSPACE
    p = _problem()
    L = B.lib()
    args = [FAKE] * 9
    assert L.fa_bwd(ctypes.byref(p), *args, None, 0, None) == B.FA_ERR_WORKSPACE
    assert L.fa_bwd(ctypes.byref(p), *args, FAKE, B.fa_workspace_size(p, 1) - 4,
                    None) == B.FA_ERR_WORKSPACE


def test_misaligned_workspace_same_status_everywhere():
    """A workspace that is not 16-byte aligned is FA_ERR_WORKSPACE from every
    entry point that takes one (the lists it holds are read with loads that
    ignore the low address bits)."""
    L = B.lib()
    pm = _problem(N=512, block_mask=FAKE, mask_block=128)
    assert _fwd(pm, ws=FAKE + 4, ws_n=1 << 20) == B.FA_ERR_WORKSPACE
    for p in (_problem(), pm):
        n = B.fa_workspace_size(p, 1)
        args = [FAKE] * 9
        assert L.fa_bwd(ctypes.byref(p), *args, FAKE + 8, n + 64, None) == B.FA_ERR_WORKSPACE
        assert L.fa_bwd_dq(ctypes.byref(p), *args[:7], FAKE + 8, n + 64,
                           None) == B.FA_ERR_WORKSPACE
        assert L.fa_bwd_dkdv(ctypes.byref(p), *args[:7], FAKE + 8, n + 64,
                             None) == B.FA_ERR_WORKSPACE
    pd = _problem(N=4096, H=8, H_kv=2)
    need = B.fa_decode_workspace_size(pd, 1)
    assert L.fa_fwd_decode(ctypes.byref(pd), 1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE + 4, need + 64,
                           None) == B.FA_ERR_WORKSPACE


def test_binding_checks_block_mask_shape():
    """The C ABI only sees a pointer to the mask; the binding rejects a mask
    whose shape is not (N / mask_block, N / mask_block)."""
    import numpy as np
    import torch

    q = torch.zeros((1, 1, 512, 64), dtype=torch.float16)
    ok = B._mask_arg(np.ones((4, 4), np.uint8), q, 128)
    assert ok.shape == (4, 4) and ok.dtype == torch.uint8
    for bad, mb in ((np.ones((2, 2), np.uint8), 128), (np.ones((4, 2), np.uint8), 128),
                    (np.ones(16, np.uint8), 128), (np.ones((4, 4), np.uint8), 256),
                    (np.ones((4, 4), np.uint8), 0), (np.ones((3, 3), np.uint8), 200)):
        with pytest.raises(ValueError):
            B._mask_arg(bad, q, mb)


def test_mask_compile_argument_checks():
    L = B.lib()
    assert L.fa_mask_compile(None, 4, FAKE, FAKE, FAKE, FAKE, None) == B.FA_ERR_ARG
    assert L.fa_mask_compile(FAKE, 0, FAKE, FAKE, FAKE, FAKE, None) == B.FA_ERR_ARG


def _decode_splits(B_, Hkv, N, n_q, group, window=0):
    """The split rule the library documents: >= 1024 workgroups of (K/V head,
    128-row block, key split), never more splits than 32-key tiles."""
    rows = group * n_q
    nrb = (rows + 127) // 128
    lo = max(0, N - n_q - window + 1) if window else 0
    ntiles = (N - 1) // 32 - lo // 32 + 1
    wgs = B_ * Hkv * nrb
    want = min(max(1, -(-1024 // wgs)), ntiles)
    tps = -(-ntiles // want)
    return -(-ntiles // tps)


@pytest.mark.parametrize("B_,H,Hkv,N,d,n_q,window", [
    (2, 8, 2, 4096, 64, 1, 0), (1, 64, 8, 8192, 128, 1, 0), (3, 4, 4, 1000, 64, 7, 0),
    (2, 8, 2, 4096, 128, 4, 300), (64, 16, 16, 64, 64, 1, 0)])
def test_decode_workspace_size(B_, H, Hkv, N, d, n_q, window):
    p = _problem(B=B_, H=H, H_kv=Hkv, N=N, d=d, causal=1, window=window)
    ns = _decode_splits(B_, Hkv, N, n_q, H // Hkv, window)
    rows = B_ * H * n_q
    want = 0 if ns == 1 else (-(-rows * ns * d * 4 // 256) * 256 + -(-rows * ns * 4 // 256) * 256)
    assert B.fa_decode_workspace_size(p, n_q) == want


@pytest.mark.parametrize("kw,n_q,status", [
    ({}, 0, B.FA_ERR_ARG), ({"N": 16}, 17, B.FA_ERR_ARG),
    ({"dtype": B.FA_F32}, 1, B.FA_ERR_UNSUPPORTED),
    ({"block_mask": FAKE, "mask_block": 128}, 1, B.FA_ERR_UNSUPPORTED),
    ({"dropout_p": 0.1}, 1, B.FA_ERR_UNSUPPORTED),
    ({"d": 96}, 1, B.FA_ERR_UNSUPPORTED), ({"H_kv": 2}, 1, B.FA_ERR_ARG)])
def test_decode_invalid_problems_rejected(kw, n_q, status):
    p = _problem(**kw)
    assert B.lib().fa_fwd_decode(ctypes.byref(p), n_q, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0,
                                 None) == status
    assert B.fa_decode_workspace_size(p, n_q) == 0


def test_decode_pointers_and_workspace_checked_before_launch():
    L = B.lib()
    p = _problem(N=4096, H=8, H_kv=2)
    need = B.fa_decode_workspace_size(p, 1)
    assert need > 0
    assert L.fa_fwd_decode(ctypes.byref(p), 1, FAKE, FAKE, None, FAKE, FAKE, FAKE, need,
                           None) == B.FA_ERR_ARG
    assert L.fa_fwd_decode(ctypes.byref(p), 1, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0,
                           None) == B.FA_ERR_WORKSPACE
    assert L.fa_fwd_decode(ctypes.byref(p), 1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need - 4,
                           None) == B.FA_ERR_WORKSPACE


def _fp8_size(B_, H, Hkv, N, d):
    """The FP8 workspace layout the header documents: Q, K, V codes, then the
    int8 block exponents of Q, K, V, each region 256-byte aligned."""
    n64 = -(-N // 64) * 64

    def al(x):
        return -(-x // 256) * 256

    hq, hk = B_ * H, B_ * Hkv
    return (al(hq * n64 * d) + 2 * al(hk * n64 * d) + al(hq * n64 // 64)
            + 2 * al(hk * n64 // 64))


@pytest.mark.parametrize("B_,H,Hkv,N,d", [(2, 3, 3, 256, 64), (1, 8, 2, 1000, 128),
                                          (4, 16, 16, 1, 64)])
def test_fp8_workspace_size(B_, H, Hkv, N, d):
    p = _problem(B=B_, H=H, H_kv=Hkv, N=N, d=d)
    assert B.fa_fp8_workspace_size(p) == _fp8_size(B_, H, Hkv, N, d)


@pytest.mark.parametrize("kw,status", [
    ({"dtype": B.FA_F32}, B.FA_ERR_UNSUPPORTED),
    ({"block_mask": FAKE, "mask_block": 128}, B.FA_ERR_UNSUPPORTED),
    ({"dropout_p": 0.1}, B.FA_ERR_UNSUPPORTED),
    ({"d": 96}, B.FA_ERR_UNSUPPORTED), ({"H_kv": 2}, B.FA_ERR_ARG), ({"N": 0}, B.FA_ERR_ARG)])
def test_fp8_invalid_problems_rejected(kw, status):
    p = _problem(**kw)
    L = B.lib()
    assert B.fa_fp8_workspace_size(p) == 0
    assert L.fa_fp8_quantize(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30,
                             None) == status
    assert L.fa_fwd_fp8(ctypes.byref(p), FAKE, FAKE, 1 << 30, FAKE, FAKE, None) == status


def test_fp8_pointers_and_workspace_checked_before_launch():
    L = B.lib()
    p = _problem()
    need = B.fa_fp8_workspace_size(p)
    assert need > 0
    q = ctypes.byref(p)
    assert L.fa_fp8_quantize(q, None, FAKE, FAKE, FAKE, FAKE, need, None) == B.FA_ERR_ARG
    assert L.fa_fp8_quantize(q, FAKE + 2, FAKE, FAKE, FAKE, FAKE, need, None) == B.FA_ERR_ARG
    assert L.fa_fp8_quantize(q, FAKE, FAKE, None, FAKE, FAKE, need, None) == B.FA_ERR_ARG
    assert L.fa_fp8_quantize(q, FAKE, FAKE, FAKE, FAKE + 8, FAKE, need, None) == B.FA_ERR_ARG
    assert L.fa_fp8_quantize(q, FAKE, FAKE, FAKE, FAKE, None, need, None) == B.FA_ERR_WORKSPACE
    assert L.fa_fp8_quantize(q, FAKE, FAKE, FAKE, FAKE, FAKE, need - 1,
                             None) == B.FA_ERR_WORKSPACE
    assert L.fa_fwd_fp8(q, FAKE, FAKE, need, None, FAKE, None) == B.FA_ERR_ARG
    assert L.fa_fwd_fp8(q, FAKE, FAKE, need, FAKE, FAKE + 2, None) == B.FA_ERR_ARG
    assert L.fa_fwd_fp8(q, FAKE, FAKE, need - 1, FAKE, FAKE, None) == B.FA_ERR_WORKSPACE
    assert L.fa_fwd_fp8(q, FAKE, FAKE + 8, need, FAKE, FAKE, None) == B.FA_ERR_WORKSPACE


@pytest.mark.parametrize("B_,H,Hkv,N,d", [(2, 3, 3, 256, 64), (1, 8, 2, 1000, 128), (1, 2, 1, 1, 64)])
def test_fp8_workspace_views_match_the_documented_layout(B_, H, Hkv, N, d):
    """The binding's views of an FP8 workspace (a CPU byte tensor here) tile
    exactly the size the library reports, in the header's order, each region
    on a 256-byte boundary and no two overlapping."""
    import torch

    need = B.fa_fp8_workspace_size(_problem(B=B_, H=H, H_kv=Hkv, N=N, d=d))
    ws = torch.zeros(need, dtype=torch.uint8)
    views = B.fp8_workspace_views(ws, B_, H, Hkv, N, d)
    n64 = -(-N // 64) * 64
    assert views["qc"].shape == (B_ * H, n64, d) and views["kc"].shape == (B_ * Hkv, n64, d)
    assert views["vc"].shape == (B_ * Hkv, n64 // 64, d, 64)
    assert views["qe"].shape == (B_ * H, n64 // 64) and views["ve"].dtype == torch.int8
    base = ws.data_ptr()
    spans = []
    for name in ("qc", "kc", "vc", "qe", "ke", "ve"):
        start = views[name].data_ptr() - base
        assert start % 256 == 0, name
        spans.append((start, start + views[name].numel()))
    assert all(a[1] <= b[0] for a, b in zip(spans, spans[1:]))
    assert spans[-1][1] <= need < spans[-1][1] + 256


def test_decode_noalloc_checks_before_any_gpu_call():
    """fa_fwd_decode_noalloc checks its arguments and the scratch limit before
    touching the GPU: invalid problems, null or misaligned pointers, and a
    problem whose partials exceed the 64 MiB static scratch."""
    L = B.lib()
    for kw, n_q, status in (({}, 0, B.FA_ERR_ARG), ({"dtype": B.FA_F32}, 1, B.FA_ERR_UNSUPPORTED),
                            ({"dropout_p": 0.1}, 1, B.FA_ERR_UNSUPPORTED),
                            ({"d": 96}, 1, B.FA_ERR_UNSUPPORTED)):
        p = _problem(**kw)
        assert L.fa_fwd_decode_noalloc(ctypes.byref(p), n_q, FAKE, FAKE, FAKE, FAKE, FAKE,
                                       None) == status
    p = _problem(N=4096, H=8, H_kv=2)
    assert L.fa_fwd_decode_noalloc(ctypes.byref(p), 1, FAKE, None, FAKE, FAKE, FAKE,
                                   None) == B.FA_ERR_ARG
    assert L.fa_fwd_decode_noalloc(ctypes.byref(p), 1, FAKE, FAKE, FAKE, FAKE + 4, FAKE,
                                   None) == B.FA_ERR_ARG
    # 128 rows of one K/V head, 1024 splits of 64 keys, d = 128: 67.6 MB of partials
    big = _problem(B=1, H=8, H_kv=1, N=65536, d=128, causal=1, dtype=B.FA_BF16)
    assert B.fa_decode_workspace_size(big, 16) > B.NOALLOC_SCRATCH_BYTES
    assert L.fa_fwd_decode_noalloc(ctypes.byref(big), 16, FAKE, FAKE, FAKE, FAKE, FAKE,
                                   None) == B.FA_ERR_SCRATCH
    assert "scratch" in B.fa_status_string(B.FA_ERR_SCRATCH)


def test_debug_header_entry_only_in_debug_library():
    """include/fa_debug.h declares what only the debug build exports."""
    from io_aware_exact_fwd_amd.build import LIB_DEBUG

    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "fa_debug.h")).read(),
                  flags=re.S)
    names = sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))
    assert names == ["fa_debug_set_tile_visits"]
    assert not hasattr(ctypes.CDLL(B.LIB_PATH), names[0])
    if os.path.exists(LIB_DEBUG):
        dbg = ctypes.CDLL(LIB_DEBUG)
        for n in names + _declared_functions():
            assert hasattr(dbg, n), n
