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

Input recipe: torch.Generator('cpu').manual_seed(1000 + N); Q, K, V, dO drawn
in that order as float32 N(0, 1) of shape (B, H, N, d), then rounded to the
workload dtype with round-to-nearest-even.  Both the GPU path and the oracle
receive these same rounded values.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "make_inputs",
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

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

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
}


def _torch_dtype(name):
    import torch

    return {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[name]


def make_inputs(B, H, N, d, dtype="f16", seed=None):
    """Q, K, V, dO as CPU torch tensors (B, H, N, d) in ``dtype``.

    Drawn as float32 N(0, 1) from torch.Generator('cpu').manual_seed(seed),
    seed defaulting to 1000 + N, in the order Q, K, V, dO; then rounded to
    the dtype (round-to-nearest-even).
    """
    import torch

    g = torch.Generator("cpu")
    g.manual_seed(1000 + N if seed is None else seed)
    out = []
    for _ in range(4):
        x = torch.randn((B, H, N, d), generator=g, dtype=torch.float32)
        out.append(x.to(_torch_dtype(dtype)).contiguous())
    return tuple(out)


def butterfly_block_mask(nblocks: int) -> np.ndarray:
    """uint8 [nblocks, nblocks]: 1 iff i == j or i XOR j is a power of two."""
    i = np.arange(nblocks)[:, None]
    j = np.arange(nblocks)[None, :]
    x = i ^ j
    keep = (x == 0) | ((x & (x - 1)) == 0)
    return keep.astype(np.uint8)


def kept_pairs_per_head(N: int, causal: bool, block_mask=None, mask_block: int = 128) -> int:
    """Number of (query, key) pairs whose probability can be non-zero, per head."""
    if block_mask is None:
        return N * (N + 1) // 2 if causal else N * N
    bm = np.asarray(block_mask) != 0
    nb = bm.shape[0]
    total = 0
    for bi in range(nb):
        for bj in np.nonzero(bm[bi])[0]:
            if not causal or bj < bi:
                total += mask_block * mask_block
            elif bj == bi:
                total += mask_block * (mask_block + 1) // 2
    return int(total)


# FLOP convention: matrix-core work only, 2 FLOP per multiply-add, counted over
# kept pairs.  Forward: Q K^T and P V (4 d per pair).  Backward: the score
# recompute, dV, dP, dK and dQ products (10 d per pair).

def fwd_flops(w: Workload) -> float:
    return 4.0 * w.d * kept_pairs_per_head(w.N, w.causal, w.block_mask(), w.mask_block) * w.B * w.H


def bwd_flops(w: Workload) -> float:
    return 10.0 * w.d * kept_pairs_per_head(w.N, w.causal, w.block_mask(), w.mask_block) * w.B * w.H


def fwd_compulsory_bytes(w: Workload) -> float:
    """Read Q, K, V once; write O and the fp32 LSE once."""
    x = w.N * w.d * w.elem_bytes
    return float(w.B * w.H * (4 * x + 4 * w.N))


def bwd_compulsory_bytes(w: Workload) -> float:
    """Pre-pass reads O, dO and writes D; main pass reads Q, K, V, dO, LSE, D
    and writes dQ, dK, dV."""
    x = w.N * w.d * w.elem_bytes
    return float(w.B * w.H * (9 * x + 12 * w.N))
