"""torch.autograd integration of the forward and backward.

Follows the autograd glue of boostr 0.1.0, ``src/ops/autograd_attention.rs``
(``var_flash_attention`` and the ``FlashAttentionBackward`` grad function): the forward
returns the attention output and keeps q, k, v, the output and its lse; the backward takes
the incoming gradient of the output and returns the gradients of q, k and v.  The lse is
internal to the backward (it is returned only on request, as a non-differentiable tensor).
First-order only: the backward is not itself differentiable.

    out = flash_attention(q, k, v, causal=True)          # q, k, v with requires_grad
    out.backward(grad)                                    # fills q.grad, k.grad, v.grad
"""
from __future__ import annotations

import torch

from . import bwd, fwd

__all__ = ["FlashAttention", "flash_attention"]


class FlashAttention(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, causal: bool, scale, return_lse: bool, window_size: int):
        o, lse = fwd(q, k, v, causal=causal, scale=scale, window_size=window_size)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.causal = bool(causal)
        ctx.scale = scale
        ctx.window_size = int(window_size)
        if return_lse:
            ctx.mark_non_differentiable(lse)
            return o, lse
        return o

    @staticmethod
    @torch.autograd.function.once_differentiable
    def backward(ctx, do, *unused):
        q, k, v, o, lse = ctx.saved_tensors
        dq, dk, dv = bwd(do.contiguous(), q, k, v, o, lse, causal=ctx.causal, scale=ctx.scale,
                         window_size=ctx.window_size)
        return dq, dk, dv, None, None, None, None


def flash_attention(q, k, v, causal: bool = False, scale: float | None = None,
                    return_lse: bool = False, window_size: int = 0):
    """Attention output [B, H, Sq, D] (and its lse [B, H, Sq] if ``return_lse``), with
    gradients through the HIP backward.  Layouts, dtypes and ``window_size`` as for ``fwd``
    (the configuration autograd_attention.rs saves for the backward: causal and window)."""
    return FlashAttention.apply(q, k, v, causal, scale, return_lse, window_size)
