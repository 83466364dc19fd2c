"""ctypes binding of libfa_mi355x (include/fa.h).  Argument marshalling only.

Every step of the computation runs in the HIP library; PyTorch provides the
device memory (outputs and workspace) and the current stream.  If the library
is missing, or a tensor is not a contiguous GPU tensor of a supported type,
the call raises -- there is no CPU or PyTorch fallback.

Names follow the C ABI: ``fa_fwd``, ``fa_bwd``, ``fa_mask_compile``,
``fa_workspace_size``, ``fa_fwd_decode``, ``fa_fwd_decode_noalloc``,
``fa_decode_workspace_size``, ``fa_status_string``, ``fa_version``.
"""

from __future__ import annotations

import ctypes
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfa_mi355x.so")

FA_F32, FA_F16, FA_BF16 = 0, 1, 2
FA_OK, FA_ERR_ARG, FA_ERR_UNSUPPORTED, FA_ERR_WORKSPACE, FA_ERR_LAUNCH = 0, -1, -2, -3, -4
FA_ERR_SCRATCH = -5
FA_REUSE_LISTS = 1  # fa_problem.flags: the workspace already holds the compiled block lists
FA_BWD_ATOMIC_DQ = 2  # fa_problem.flags: single-pass backward, dQ by float32 atomics
NOALLOC_SCRATCH_BYTES = 64 << 20  # static scratch of fa_fwd_decode_noalloc, per GPU

EXPORTS = ("fa_workspace_size", "fa_fwd", "fa_bwd", "fa_bwd_dq", "fa_bwd_dkdv",
           "fa_mask_compile", "fa_decode_workspace_size", "fa_fwd_decode",
           "fa_fwd_decode_noalloc",
           "fa_fp8_workspace_size", "fa_fp8_quantize", "fa_fwd_fp8",
           "fa_status_string", "fa_version")


class FaProblem(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32),
        ("H", ctypes.c_int32),
        ("N", ctypes.c_int32),
        ("d", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("causal", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("block_mask", ctypes.c_void_p),
        ("mask_block", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("H_kv", ctypes.c_int32),
        ("dropout_p", ctypes.c_float),
        ("seed", ctypes.c_uint64),
        ("offset", ctypes.c_uint32),
        ("flags", ctypes.c_uint32),
    ]


class FaError(RuntimeError):
    def __init__(self, fn, status):
        super().__init__(f"{fn} failed: {fa_status_string(status)} ({status})")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load libfa_mi355x.so (built in-tree); raise if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is not built; run `python -m io_aware_exact_fwd_amd.build` "
            "(there is no fallback implementation)")
    L = ctypes.CDLL(LIB_PATH)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32
    pp = ctypes.POINTER(FaProblem)
    L.fa_workspace_size.argtypes = [pp, ctypes.c_int]
    L.fa_workspace_size.restype = sz
    L.fa_fwd.argtypes = [pp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.fa_fwd.restype = ctypes.c_int
    L.fa_bwd.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.fa_bwd.restype = ctypes.c_int
    L.fa_bwd_dq.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.fa_bwd_dq.restype = ctypes.c_int
    L.fa_bwd_dkdv.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.fa_bwd_dkdv.restype = ctypes.c_int
    L.fa_mask_compile.argtypes = [vp, i32, vp, vp, vp, vp, vp]
    L.fa_mask_compile.restype = ctypes.c_int
    L.fa_decode_workspace_size.argtypes = [pp, i32]
    L.fa_decode_workspace_size.restype = sz
    L.fa_fwd_decode.argtypes = [pp, i32, vp, vp, vp, vp, vp, vp, sz, vp]
    L.fa_fwd_decode.restype = ctypes.c_int
    L.fa_fwd_decode_noalloc.argtypes = [pp, i32, vp, vp, vp, vp, vp, vp]
    L.fa_fwd_decode_noalloc.restype = ctypes.c_int
    L.fa_fp8_workspace_size.argtypes = [pp]
    L.fa_fp8_workspace_size.restype = sz
    L.fa_fp8_quantize.argtypes = [pp, vp, vp, vp, vp, vp, sz, vp]
    L.fa_fp8_quantize.restype = ctypes.c_int
    L.fa_fwd_fp8.argtypes = [pp, vp, vp, sz, vp, vp, vp]
    L.fa_fwd_fp8.restype = ctypes.c_int
    L.fa_status_string.argtypes = [ctypes.c_int]
    L.fa_status_string.restype = ctypes.c_char_p
    L.fa_version.argtypes = []
    L.fa_version.restype = ctypes.c_int
    _lib = L
    return L


def use_library(path: str):
    """Context manager: route the calls of this module through the library at
    `path` (e.g. the debug build, ``build.LIB_DEBUG``) instead of the default
    one, then restore it.  Not thread-safe."""
    import contextlib

    @contextlib.contextmanager
    def _swap():
        global _lib, LIB_PATH
        saved = (_lib, LIB_PATH)
        _lib, LIB_PATH = None, path
        try:
            yield lib()
        finally:
            _lib, LIB_PATH = saved

    return _swap()


def fa_debug_set_tile_visits(visits) -> None:
    """Debug library only (include/fa_debug.h): later forward / backward calls
    add their tile visits to `visits` (int32 GPU tensor of 3 * B*H * nb * nb,
    nb = ceil(N / 128)); None clears."""
    L = lib()
    if not hasattr(L, "fa_debug_set_tile_visits"):
        raise RuntimeError("fa_debug_set_tile_visits: not the debug library")
    L.fa_debug_set_tile_visits.argtypes = [ctypes.c_void_p]
    L.fa_debug_set_tile_visits.restype = ctypes.c_int
    st = L.fa_debug_set_tile_visits(None if visits is None else visits.data_ptr())
    if st != FA_OK:
        raise FaError("fa_debug_set_tile_visits", st)


def fa_status_string(status: int) -> str:
    return lib().fa_status_string(int(status)).decode()


def fa_version() -> int:
    return int(lib().fa_version())


def _dtype_code(t):
    import torch

    codes = {torch.float32: FA_F32, torch.float16: FA_F16, torch.bfloat16: FA_BF16}
    if t.dtype not in codes:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return codes[t.dtype]


def make_problem(q, causal=False, scale=None, block_mask=None, mask_block=128, k=None,
                 window=0, dropout_p=0.0, seed=0, offset=0, flags=0) -> FaProblem:
    """Problem descriptor for (B, H, N, d) tensor q (and K/V tensor k, whose
    head count gives H_kv); scale defaults to 1/sqrt(d)."""
    if q.dim() != 4:
        raise ValueError("expected (B, H, N, d) tensors")
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    p = FaProblem()
    p.B, p.H, p.N, p.d = B, H, N, d
    p.dtype = _dtype_code(q)
    p.causal = 1 if causal else 0
    p.scale = float(scale)
    p.block_mask = block_mask.data_ptr() if block_mask is not None else None
    p.mask_block = int(mask_block) if block_mask is not None else 0
    p.window = int(window)
    p.H_kv = int(k.shape[1]) if k is not None else H
    p.dropout_p = float(dropout_p)
    p.seed = int(seed) & (2**64 - 1)
    p.offset = int(offset) & (2**32 - 1)
    p.flags = int(flags)
    return p


def fa_workspace_size(p: FaProblem, pass_: int) -> int:
    return int(lib().fa_workspace_size(ctypes.byref(p), int(pass_)))


def _check_tensors(ref, *ts):
    for t in ts:
        if not t.is_cuda:
            raise ValueError("tensors must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous (B, H, N, d)")
        if t.dtype != ref.dtype or t.shape != ref.shape:
            raise ValueError("tensors must share dtype and shape")


def _check_qkv(q, k, v):
    _check_tensors(q)
    _check_tensors(k, k, v)
    if k.dim() != 4 or k.shape[0] != q.shape[0] or k.shape[2:] != q.shape[2:]:
        raise ValueError("k, v must be (B, H_kv, N, d) with q's B, N and d")
    if k.shape[1] == 0 or q.shape[1] % k.shape[1]:
        raise ValueError("the K/V head count must divide the query head count")


def _mask_arg(block_mask, ref, mask_block):
    """The block mask as a contiguous uint8 tensor on ref's device.  The C ABI
    receives only a pointer, so its shape is checked here: 2-D, square, with
    side N / mask_block (N = ref.shape[2])."""
    import torch

    if block_mask is None:
        return None
    if not isinstance(block_mask, torch.Tensor):
        block_mask = torch.as_tensor(block_mask)
    N = ref.shape[2]
    if mask_block <= 0 or N % mask_block:
        raise ValueError(f"mask_block {mask_block} must be positive and divide N = {N}")
    nb = N // mask_block
    if block_mask.dim() != 2 or tuple(block_mask.shape) != (nb, nb):
        raise ValueError(f"block mask must be ({nb}, {nb}) for N = {N} and mask_block = "
                         f"{mask_block}, got {tuple(block_mask.shape)}")
    return block_mask.to(device=ref.device, dtype=torch.uint8).contiguous()


def _stream(t):
    import torch

    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _workspace(ws, need, dev):
    """A uint8 GPU workspace of at least `need` bytes: the caller's, or a new one."""
    import torch

    if ws is None:
        return torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    if ws.dtype != torch.uint8 or not ws.is_cuda or not ws.is_contiguous() or ws.numel() < need:
        raise ValueError(f"workspace must be a contiguous uint8 GPU tensor of >= {need} bytes")
    return ws


def fa_fwd(q, k, v, causal=False, scale=None, block_mask=None, mask_block=128, out=None,
           lse=None, window=0, dropout_p=0.0, seed=0, offset=0, workspace=None,
           reuse_lists=False):
    """Forward: returns (O, LSE); O like q, LSE float32 (B, H, N), natural log.
    k, v may have fewer heads than q (grouped / multi-query attention).
    workspace: optional uint8 GPU tensor (e.g. the backward's, which is at
    least as large); reuse_lists: it already holds this mask's block lists."""
    _check_qkv(q, k, v)
    bm = _mask_arg(block_mask, q, mask_block)
    p = make_problem(q, causal, scale, bm, mask_block, k, window, dropout_p, seed, offset,
                     FA_REUSE_LISTS if reuse_lists else 0)
    B, H, N, d = q.shape
    import torch

    o = torch.empty_like(q) if out is None else out
    lse_t = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None else lse
    _check_tensors(q, o)
    ws_n = fa_workspace_size(p, 0)
    ws = _workspace(workspace, ws_n, q.device)
    st = lib().fa_fwd(ctypes.byref(p), q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                      lse_t.data_ptr(), ws.data_ptr(), ws.numel(), _stream(q))
    if st != FA_OK:
        raise FaError("fa_fwd", st)
    return o, lse_t


def fa_decode_workspace_size(p: FaProblem, n_q: int) -> int:
    return int(lib().fa_decode_workspace_size(ctypes.byref(p), int(n_q)))


def _decode_args(q, k, v, causal, scale, window, out, lse):
    import torch

    _check_tensors(q)
    _check_tensors(k, k, v)
    if q.dim() != 4 or k.dim() != 4 or k.shape[0] != q.shape[0] or k.shape[3] != q.shape[3]:
        raise ValueError("q must be (B, H, n_q, d) and k, v (B, H_kv, N, d)")
    if k.shape[1] == 0 or q.shape[1] % k.shape[1]:
        raise ValueError("the K/V head count must divide the query head count")
    if k.dtype != q.dtype:
        raise ValueError("q, k, v must share a dtype")
    B, H, n_q, d = q.shape
    p = make_problem(k, causal, scale, None, 128, k, window)
    p.H = H  # query heads; N and H_kv come from k
    o = torch.empty_like(q) if out is None else out
    lse_t = torch.empty((B, H, n_q), dtype=torch.float32, device=q.device) if lse is None else lse
    _check_tensors(q, o)
    return p, n_q, o, lse_t


def fa_fwd_decode(q, k, v, causal=True, scale=None, window=0, out=None, lse=None):
    """Decode-shaped forward: q (B, H, n_q, d) holds the LAST n_q positions of
    a sequence whose N keys and values are k, v (B, H_kv, N, d).  Returns
    (O like q, LSE float32 (B, H, n_q), natural log).  The keys are split over
    workgroups and the partial results merged inside the library."""
    import torch

    p, n_q, o, lse_t = _decode_args(q, k, v, causal, scale, window, out, lse)
    ws_n = fa_decode_workspace_size(p, n_q)
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=q.device)
    st = lib().fa_fwd_decode(ctypes.byref(p), n_q, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                             o.data_ptr(), lse_t.data_ptr(), ws.data_ptr(), ws_n, _stream(q))
    if st != FA_OK:
        raise FaError("fa_fwd_decode", st)
    return o, lse_t


def fa_fwd_decode_noalloc(q, k, v, causal=True, scale=None, window=0, out=None, lse=None):
    """``fa_fwd_decode`` whose split partials live in the library's static
    per-GPU scratch (``NOALLOC_SCRATCH_BYTES``) instead of a workspace; for
    callers that cannot allocate.  Pass ``out`` and ``lse`` to allocate
    nothing at all.  Calls that overlap on one GPU share the scratch and must
    be ordered (one stream)."""
    import torch

    p, n_q, o, lse_t = _decode_args(q, k, v, causal, scale, window, out, lse)
    with torch.cuda.device(q.device):
        st = lib().fa_fwd_decode_noalloc(ctypes.byref(p), n_q, q.data_ptr(), k.data_ptr(),
                                         v.data_ptr(), o.data_ptr(), lse_t.data_ptr(),
                                         _stream(q))
    if st != FA_OK:
        raise FaError("fa_fwd_decode_noalloc", st)
    return o, lse_t


def fa_fp8_workspace_size(p: FaProblem) -> int:
    return int(lib().fa_fp8_workspace_size(ctypes.byref(p)))


def _check_signs(signs, q):
    import torch

    if (not isinstance(signs, torch.Tensor) or signs.dtype != torch.float32 or not signs.is_cuda
            or not signs.is_contiguous() or signs.shape != (q.shape[3],)):
        raise ValueError("signs must be a contiguous float32 GPU tensor of d values (+1 / -1)")


def fp8_quantize(q, k, v, signs, causal=False, scale=None, window=0, workspace=None):
    """Rotate and block-quantise q, k, v to E4M3 (``fa_fp8_quantize``).
    Returns (problem, workspace uint8 tensor); ``fp8_workspace_views`` names
    the regions of the workspace."""
    import torch

    _check_qkv(q, k, v)
    _check_signs(signs, q)
    p = make_problem(q, causal, scale, None, 128, k, window)
    ws_n = fa_fp8_workspace_size(p)
    if ws_n == 0:
        raise FaError("fa_fp8_workspace_size", FA_ERR_UNSUPPORTED)
    ws = torch.empty(ws_n, dtype=torch.uint8, device=q.device) if workspace is None else workspace
    if ws.dtype != torch.uint8 or not ws.is_cuda or not ws.is_contiguous() or ws.numel() < ws_n:
        raise ValueError(f"workspace must be a contiguous uint8 GPU tensor of >= {ws_n} bytes")
    st = lib().fa_fp8_quantize(ctypes.byref(p), signs.data_ptr(), q.data_ptr(), k.data_ptr(),
                               v.data_ptr(), ws.data_ptr(), ws.numel(), _stream(q))
    if st != FA_OK:
        raise FaError("fa_fp8_quantize", st)
    return p, ws


def fp8_workspace_views(ws, B, H, H_kv, N, d):
    """Views of the six regions of an FP8 workspace (layout of include/fa.h):
    q/k codes (heads, N64, d), v codes (H_kv heads, N64 / 64, d, 64), and the
    int8 block exponents (heads, N64 / 64)."""
    import torch

    n64 = (N + 63) // 64 * 64
    hq, hk = B * H, B * H_kv

    def al(x):
        return (x + 255) // 256 * 256

    sizes = [hq * n64 * d, hk * n64 * d, hk * n64 * d, hq * n64 // 64, hk * n64 // 64,
             hk * n64 // 64]
    offs, o = [], 0
    for sz in sizes:
        offs.append(o)
        o += al(sz)
    views = {
        "qc": ws[offs[0]:offs[0] + sizes[0]].view(hq, n64, d),
        "kc": ws[offs[1]:offs[1] + sizes[1]].view(hk, n64, d),
        "vc": ws[offs[2]:offs[2] + sizes[2]].view(hk, n64 // 64, d, 64),
    }
    for name, i, h in (("qe", 3, hq), ("ke", 4, hk), ("ve", 5, hk)):
        views[name] = ws[offs[i]:offs[i] + sizes[i]].view(torch.int8).view(h, n64 // 64)
    return views


def fa_fwd_fp8(q, k, v, signs, causal=False, scale=None, window=0, out=None, lse=None,
               workspace=None):
    """FP8 forward with block scales and the random Hadamard rotation given by
    ``signs`` (float32 (d,), +1 / -1): quantises q, k, v into the workspace,
    then runs attention on the codes.  Returns (O like q, LSE float32 (B, H, N))."""
    import torch

    p, ws = fp8_quantize(q, k, v, signs, causal, scale, window, workspace)
    B, H, N, d = q.shape
    o = torch.empty_like(q) if out is None else out
    lse_t = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None else lse
    _check_tensors(q, o)
    st = lib().fa_fwd_fp8(ctypes.byref(p), signs.data_ptr(), ws.data_ptr(), ws.numel(),
                          o.data_ptr(), lse_t.data_ptr(), _stream(q))
    if st != FA_OK:
        raise FaError("fa_fwd_fp8", st)
    return o, lse_t


def fa_bwd(q, k, v, o, dout, lse, causal=False, scale=None, block_mask=None, mask_block=128,
           window=0, dropout_p=0.0, seed=0, offset=0, workspace=None, reuse_lists=False,
           atomic_dq=False):
    """Backward of <O, dO>: returns (dQ, dK, dV); dQ like q, dK and dV like k.
    workspace / reuse_lists: as for ``fa_fwd`` (a forward given the same
    buffer leaves the block lists there for the backward).  atomic_dq: the
    single-pass backward (FA_BWD_ATOMIC_DQ; dQ summed with float32 atomics)."""
    import torch

    _check_qkv(q, k, v)
    _check_tensors(q, o, dout)
    if lse.dtype != torch.float32 or not lse.is_contiguous() or not lse.is_cuda:
        raise ValueError("lse must be a contiguous float32 GPU tensor")
    bm = _mask_arg(block_mask, q, mask_block)
    p = make_problem(q, causal, scale, bm, mask_block, k, window, dropout_p, seed, offset,
                     (FA_REUSE_LISTS if reuse_lists else 0) | (FA_BWD_ATOMIC_DQ if atomic_dq else 0))
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws_n = fa_workspace_size(p, 1)
    ws = _workspace(workspace, ws_n, q.device)
    st = lib().fa_bwd(ctypes.byref(p), q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                      dout.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                      dv.data_ptr(), ws.data_ptr(), ws.numel(), _stream(q))
    if st != FA_OK:
        raise FaError("fa_bwd", st)
    return dq, dk, dv


def bwd_workspace(q, causal=False, scale=None, block_mask=None, mask_block=128, k=None,
                  window=0, dropout_p=0.0, seed=0, offset=0, reuse_lists=False, atomic_dq=False):
    """(problem, workspace tensor, workspace bytes, mask) for the two backward
    stages (or, with atomic_dq, for ``fa_bwd_into`` running the single-pass
    backward); reuse_lists sets FA_REUSE_LISTS in the problem (for a workspace
    that a forward on the same buffer has filled)."""
    import torch

    bm = _mask_arg(block_mask, q, mask_block)
    p = make_problem(q, causal, scale, bm, mask_block, k, window, dropout_p, seed, offset,
                     (FA_REUSE_LISTS if reuse_lists else 0) | (FA_BWD_ATOMIC_DQ if atomic_dq else 0))
    ws_n = fa_workspace_size(p, 1)
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=q.device)
    return p, ws, ws_n, bm


def fa_bwd_into(p, q, k, v, o, dout, lse, dq, dk, dv, ws, ws_n):
    """The whole backward (fa_bwd) into given outputs, for a problem and
    workspace from ``bwd_workspace``."""
    st = lib().fa_bwd(ctypes.byref(p), q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                      dout.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                      dv.data_ptr(), ws.data_ptr(), ws_n, _stream(q))
    if st != FA_OK:
        raise FaError("fa_bwd", st)


def fa_bwd_dq(p, q, k, v, o, dout, lse, dq, ws, ws_n):
    """First backward stage (D and dQ) for a problem from ``bwd_workspace``."""
    st = lib().fa_bwd_dq(ctypes.byref(p), q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                         dout.data_ptr(), lse.data_ptr(), dq.data_ptr(), ws.data_ptr(), ws_n,
                         _stream(q))
    if st != FA_OK:
        raise FaError("fa_bwd_dq", st)


def fa_bwd_dkdv(p, q, k, v, dout, lse, dk, dv, ws, ws_n):
    """Second backward stage (dK, dV); same problem and workspace as fa_bwd_dq."""
    st = lib().fa_bwd_dkdv(ctypes.byref(p), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                           dout.data_ptr(), lse.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                           ws.data_ptr(), ws_n, _stream(q))
    if st != FA_OK:
        raise FaError("fa_bwd_dkdv", st)


def fa_mask_compile(block_mask):
    """Compile a uint8 [nb, nb] GPU block mask; returns (row_ptr, col_idx,
    col_ptr, row_idx) int32 GPU tensors, index lists trimmed to nnz."""
    import torch

    bm = block_mask.to(torch.uint8).contiguous()
    if not bm.is_cuda or bm.dim() != 2 or bm.shape[0] != bm.shape[1]:
        raise ValueError("block mask must be a square uint8 GPU tensor")
    nb = bm.shape[0]
    dev = bm.device
    row_ptr = torch.empty(nb + 1, dtype=torch.int32, device=dev)
    col_ptr = torch.empty(nb + 1, dtype=torch.int32, device=dev)
    col_idx = torch.empty(nb * nb, dtype=torch.int32, device=dev)
    row_idx = torch.empty(nb * nb, dtype=torch.int32, device=dev)
    st = lib().fa_mask_compile(bm.data_ptr(), nb, row_ptr.data_ptr(), col_idx.data_ptr(),
                               col_ptr.data_ptr(), row_idx.data_ptr(), _stream(bm))
    if st != FA_OK:
        raise FaError("fa_mask_compile", st)
    nnz = int(row_ptr[-1].item())
    return row_ptr, col_idx[:nnz], col_ptr, row_idx[:nnz]
