"""MI355X-native tiled exact attention (FlashAttention forward and backward).

The compute path is the HIP library ``libfa_mi355x.so`` built from ``csrc/``
(``python -m io_aware_exact_fwd_amd.build``); this package only marshals
arguments to its C ABI (``include/fa.h``) and never computes on the CPU.

    o, lse = fa_fwd(q, k, v, causal=True, scale=0.125)
    dq, dk, dv = fa_bwd(q, k, v, o, do, lse, causal=True, scale=0.125)
    o = attention(q, k, v, causal=True)        # differentiable wrapper
    o, lse = fa_fwd_decode(q_last, k, v)       # last n_q positions vs N keys
    o, lse = fa_fwd_decode_noalloc(q_last, k, v, out=o, lse=lse)  # no allocation
    o, lse = fa_fwd_fp8(q, k, v, signs)        # FP8 with block scales + rotation
"""

from .binding import (  # noqa: F401
    FA_BF16,
    FA_F16,
    FA_F32,
    FaError,
    bwd_workspace,
    fa_bwd,
    fa_decode_workspace_size,
    fa_bwd_dkdv,
    fa_bwd_dq,
    fa_bwd_into,
    fa_fwd,
    fa_fwd_decode,
    fa_fwd_decode_noalloc,
    fa_fwd_fp8,
    fa_fp8_workspace_size,
    fp8_quantize,
    fp8_workspace_views,
    fa_mask_compile,
    fa_status_string,
    fa_version,
    fa_workspace_size,
    make_problem,
)


def attention(q, k, v, causal=False, scale=None, block_mask=None, mask_block=128, window=0,
              dropout_p=0.0, seed=0, offset=0):
    """softmax(scale * Q K^T, masked) V with a backward through ``fa_bwd``.

    k, v may carry fewer heads than q (grouped / multi-query attention); with
    dropout_p > 0 the same (seed, offset) regenerates the mask in the backward.
    """
    import torch

    opts = dict(causal=causal, scale=scale, block_mask=block_mask, mask_block=mask_block,
                window=window, dropout_p=dropout_p, seed=seed, offset=offset)

    class _Attention(torch.autograd.Function):
        @staticmethod
        def forward(ctx, q_, k_, v_):
            o, lse = fa_fwd(q_, k_, v_, **opts)
            ctx.save_for_backward(q_, k_, v_, o, lse)
            return o

        @staticmethod
        def backward(ctx, do):
            q_, k_, v_, o, lse = ctx.saved_tensors
            return fa_bwd(q_, k_, v_, o, do.contiguous(), lse, **opts)

    return _Attention.apply(q, k, v)
