"""Seeded synthetic workloads and work accounting for tiled exact attention.

This module holds no attention arithmetic.  It is shared by the tests, the
bench and the smoke check: it draws the inputs (Q, K, V, dO), builds the
block mask that the block-sparse workload passes in, and counts algorithmic
FLOPs and bytes for the roofline figures.

Workloads (the pages measure on GPT-2 shaped attention and on long-sequence
tasks; these synthetic tensors stand in for them -- no dataset is used):

  single_head   B=1  H=1  N=256   d=64  fp32  non-causal   scale 1/8
  gpt2_small    B=8  H=12 N=1024  d=64  fp16  causal       scale 1/8
  gpt2_medium   B=64 H=16 N=1024  d=64  fp16  causal       scale 1/8
                (the shape of the headline GPT-2-medium measurement in the
                agihunt.info summary of the paper)
  long_wide     B=2  H=16 N=8192  d=128 bf16  causal       scale 1/sqrt(128)
  butterfly     B=1  H=8  N=65536 d=64  fp16  non-causal   scale 1/8,
                128x128 blocks, block (i, j) kept iff i == j or i XOR j is a
                power of two (block-sparse attention with a fixed butterfly
                pattern, agihunt.info summary, block-sparse paragraph)

Extensions of the method (sliding window, grouped K/V heads, dropout):

  long_window   long_wide with a sliding window of W=512 keys (the window
                and length of the lynx-cortex practice problem on sliding
                window attention)
  gqa_h64_kv8   B=1  H=64 H_kv=8 N=8192 d=128 bf16 causal: the head
                configuration the living-dl-book chapter gives for Llama-3
                70B (64 query heads sharing 8 K/V heads, head dim 128)
  gpt2_medium_dropout  gpt2_medium with attention dropout p = 0.1

Decode shape (a few new queries against a long key sequence, with grouped
K/V heads; forward only):

  decode_gqa    B=16 H=64 H_kv=8 N=8192 d=128 bf16, n_q=1 (the last position),
                causal: one token of a batch of 16 sequences with the
                grouped-head layout above and an 8K-token context

Input recipe: torch.Generator('cpu').manual_seed(1000 + N); Q (B, H, N, d),
K and V (B, H_kv, N, d), dO (B, H, N, d) drawn in that order as float32
N(0, 1), then rounded to the workload dtype with round-to-nearest-even.  Both
the GPU path and the oracle receive these same rounded values.  Decode
workloads draw Q (B, H, n_q, d), K, V (B, H_kv, N, d) in that order from the
same seed (``make_decode_inputs``).

FP8 path (block-quantised forward with the random rotation): the same shapes
in bf16 / fp16, and inputs with outlier channels (``make_outlier_inputs``:
the N(0, 1) draw of ``make_inputs`` with a few head-dim coordinates of Q and
K multiplied by large factors, the case the rotation exists for); the
rotation's signs are drawn by ``make_signs``.

Large logits (parity cases of the online softmax's rescaling): inputs with a
few outlier coordinates (``make_outlier_inputs``), and inputs whose logits
rise along the key sequence (``make_rising_inputs``: every query and key gets
a common component whose size grows with the key's position, so each row's
running maximum keeps growing by several units in base 2).

  long_wide_fp8 long_wide's shape (B=2 H=16 N=8192 d=128 causal) through the
                FP8 forward, bf16 in and out
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "make_inputs",
    "make_decode_inputs",
    "make_outlier_inputs",
    "make_rising_inputs",
    "make_signs",
    "butterfly_block_mask",
    "kept_pairs_per_head",
    "fwd_flops",
    "bwd_flops",
    "fwd_compulsory_bytes",
    "bwd_compulsory_bytes",
]


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str  # "f32" | "f16" | "bf16"
    causal: bool
    scale: float
    mask: str | None = None  # None | "butterfly"
    mask_block: int = 128
    window: int = 0          # 0: none; W > 0: |i - j| < W
    hkv: int = 0             # K/V heads; 0 means H
    dropout: float = 0.0
    nq: int = 0              # decode: queries per head (the last nq positions); 0: N
    fp8: bool = False        # forward through the FP8 path (block scales + rotation)

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def H_kv(self) -> int:
        return self.hkv or self.H

    def block_mask(self):
        if self.mask is None:
            return None
        if self.mask == "butterfly":
            return butterfly_block_mask(self.N // self.mask_block)
        raise ValueError(self.mask)


WORKLOADS = {
    "single_head": Workload("single_head", 1, 1, 256, 64, "f32", False, 1.0 / 8.0),
    "gpt2_small": Workload("gpt2_small", 8, 12, 1024, 64, "f16", True, 1.0 / 8.0),
    "gpt2_medium": Workload("gpt2_medium", 64, 16, 1024, 64, "f16", True, 1.0 / 8.0),
    "long_wide": Workload("long_wide", 2, 16, 8192, 128, "bf16", True, 1.0 / math.sqrt(128.0)),
    "butterfly": Workload("butterfly", 1, 8, 65536, 64, "f16", False, 1.0 / 8.0, "butterfly", 128),
    "long_window": Workload("long_window", 2, 16, 8192, 128, "bf16", True, 1.0 / math.sqrt(128.0),
                            window=512),
    "gqa_h64_kv8": Workload("gqa_h64_kv8", 1, 64, 8192, 128, "bf16", True,
                            1.0 / math.sqrt(128.0), hkv=8),
    "gpt2_medium_dropout": Workload("gpt2_medium_dropout", 64, 16, 1024, 64, "f16", True,
                                    1.0 / 8.0, dropout=0.1),
    "decode_gqa": Workload("decode_gqa", 16, 64, 8192, 128, "bf16", True, 1.0 / math.sqrt(128.0),
                           hkv=8, nq=1),
    "long_wide_fp8": Workload("long_wide_fp8", 2, 16, 8192, 128, "bf16", True,
                              1.0 / math.sqrt(128.0), fp8=True),
}


def _torch_dtype(name):
    import torch

    return {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[name]


def make_inputs(B, H, N, d, dtype="f16", seed=None, hkv=None):
    """Q, K, V, dO as CPU torch tensors in ``dtype``: Q and dO (B, H, N, d),
    K and V (B, hkv or H, N, d).

    Drawn as float32 N(0, 1) from torch.Generator('cpu').manual_seed(seed),
    seed defaulting to 1000 + N, in the order Q, K, V, dO; then rounded to
    the dtype (round-to-nearest-even).
    """
    import torch

    g = torch.Generator("cpu")
    g.manual_seed(1000 + N if seed is None else seed)
    out = []
    for heads in (H, hkv or H, hkv or H, H):
        x = torch.randn((B, heads, N, d), generator=g, dtype=torch.float32)
        out.append(x.to(_torch_dtype(dtype)).contiguous())
    return tuple(out)


def make_decode_inputs(B, H, N, d, nq, dtype="bf16", seed=None, hkv=None):
    """Decode-shaped inputs as CPU torch tensors in ``dtype``: Q (B, H, nq, d),
    K and V (B, hkv or H, N, d), drawn in that order as float32 N(0, 1) from
    torch.Generator('cpu').manual_seed(seed or 1000 + N), then rounded."""
    import torch

    g = torch.Generator("cpu")
    g.manual_seed(1000 + N if seed is None else seed)
    out = []
    for shape in ((B, H, nq, d), (B, hkv or H, N, d), (B, hkv or H, N, d)):
        x = torch.randn(shape, generator=g, dtype=torch.float32)
        out.append(x.to(_torch_dtype(dtype)).contiguous())
    return tuple(out)


def make_outlier_inputs(B, H, N, d, dtype="bf16", seed=None, hkv=None,
                        outliers=((3, 30.0), (17, 20.0))):
    """``make_inputs`` with the head-dim coordinates c of Q and K multiplied by
    f for each (c, f) in ``outliers`` (before the rounding to ``dtype``)."""
    import torch

    g = torch.Generator("cpu")
    g.manual_seed(1000 + N if seed is None else seed)
    out = []
    for i, heads in enumerate((H, hkv or H, hkv or H, H)):
        x = torch.randn((B, heads, N, d), generator=g, dtype=torch.float32)
        if i < 2:
            for c, f in outliers:
                x[..., c] *= f
        out.append(x.to(_torch_dtype(dtype)).contiguous())
    return tuple(out)


def make_rising_inputs(B, H, N, d, dtype="f16", seed=None, hkv=None, scale=None, step=64,
                       rise2=6.0, lift=4.0, nq=None):
    """``make_inputs`` (or, with ``nq``, ``make_decode_inputs``) with logits
    that rise along the key sequence: coordinate 0 of every query gets
    + ``lift`` and coordinate 0 of key j gets + inc * (j // step), with inc
    chosen so that the scaled score of a query grows by about ``rise2`` in
    base 2 (scale * log2(e) * lift * inc = rise2) from one block of ``step``
    keys to the next.  Each row's running maximum then keeps growing by more
    than a few units as the keys go by, which is the case the online
    softmax's rescaling step exists for.  Added before the rounding to
    ``dtype``; dO (if drawn) is unchanged.  scale defaults to 1/sqrt(d)."""
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    inc = rise2 / (scale * math.log2(math.e) * lift)
    if nq is None:
        q, k, v, do = make_inputs(B, H, N, d, "f32", seed, hkv)
    else:
        q, k, v = make_decode_inputs(B, H, N, d, nq, "f32", seed, hkv)
        do = None
    import torch

    q[..., 0] += lift
    k[..., 0] += inc * (torch.arange(N, dtype=torch.float32) // step)
    out = [x.to(_torch_dtype(dtype)).contiguous() for x in (q, k, v)]
    if do is not None:
        out.append(do.to(_torch_dtype(dtype)).contiguous())
    return tuple(out)


def make_signs(d, seed=7):
    """d random signs (+1 / -1) as a float32 CPU tensor, from
    torch.Generator('cpu').manual_seed(seed): sign = +1 where a uniform draw
    is below 1/2."""
    import torch

    g = torch.Generator("cpu")
    g.manual_seed(seed)
    u = torch.rand(d, generator=g, dtype=torch.float32)
    return torch.where(u < 0.5, 1.0, -1.0).to(torch.float32)


def butterfly_block_mask(nblocks: int) -> np.ndarray:
    """uint8 [nblocks, nblocks]: 1 iff i == j or i XOR j is a power of two."""
    i = np.arange(nblocks)[:, None]
    j = np.arange(nblocks)[None, :]
    x = i ^ j
    keep = (x == 0) | ((x & (x - 1)) == 0)
    return keep.astype(np.uint8)


def _band(N, causal, window):
    """Per query row i, the band [lo_i, hi_i] of keys that causal and window allow."""
    i = np.arange(N, dtype=np.int64)
    lo = np.maximum(0, i - window + 1) if window else np.zeros(N, np.int64)
    if causal:
        hi = i
    elif window:
        hi = np.minimum(N - 1, i + window - 1)
    else:
        hi = np.full(N, N - 1, np.int64)
    return lo, hi


def kept_pairs_per_head(N: int, causal: bool, block_mask=None, mask_block: int = 128,
                        window: int = 0) -> int:
    """Number of (query, key) pairs whose probability can be non-zero, per head."""
    lo, hi = _band(N, causal, window)
    if block_mask is None:
        return int((hi - lo + 1).sum())
    bm = np.asarray(block_mask) != 0
    total = 0
    for bi in range(bm.shape[0]):
        rl = lo[bi * mask_block:(bi + 1) * mask_block]
        rh = hi[bi * mask_block:(bi + 1) * mask_block]
        for bj in np.nonzero(bm[bi])[0]:
            a = np.maximum(rl, bj * mask_block)
            b = np.minimum(rh, (bj + 1) * mask_block - 1)
            total += int(np.maximum(0, b - a + 1).sum())
    return int(total)


def _pairs(w: Workload) -> int:
    return kept_pairs_per_head(w.N, w.causal, w.block_mask(), w.mask_block, w.window)


# FLOP convention: matrix-core work only, 2 FLOP per multiply-add, counted over
# kept pairs.  Forward: Q K^T and P V (4 d per pair).  Backward: the score
# recompute, dV, dP, dK and dQ products (10 d per pair).

def fwd_flops(w: Workload) -> float:
    return 4.0 * w.d * _pairs(w) * w.B * w.H


def bwd_flops(w: Workload) -> float:
    return 10.0 * w.d * _pairs(w) * w.B * w.H


def fwd_compulsory_bytes(w: Workload) -> float:
    """Read Q, K, V once; write O and the fp32 LSE once."""
    x = w.N * w.d * w.elem_bytes
    return float(w.B * (w.H * (2 * x + 4 * w.N) + w.H_kv * 2 * x))


def bwd_compulsory_bytes(w: Workload) -> float:
    """Pre-pass reads O, dO and writes D; main pass reads Q, K, V, dO, LSE, D
    and writes dQ, dK, dV."""
    x = w.N * w.d * w.elem_bytes
    return float(w.B * (w.H * (5 * x + 12 * w.N) + w.H_kv * 4 * x))
