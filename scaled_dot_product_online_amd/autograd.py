"""torch.autograd wrapper over the C ABI.

    attention(q, k, v, scale=None, is_causal=False, attn_mask=None, sinks=None) -> o

Both directions run in libsdpa_mi355x.so: the forward is sdpa_fwd and the backward is
sdpa_bwd, which takes the forward's logsumexp. Following the pages' call sites (the
MPS SDPA pull request, "Unused second output"; mps-flash-sdpa, "Usage"), the
logsumexp is computed and kept only when an input requires a gradient, and a call is
checked for eligibility before anything runs. Where those pages fall back to the
unfused math path, an ineligible call here raises ValueError instead: every step of
the computation is meant to run in the library's kernels. Masks and sinks, which those
pages hand to the unfused path (mps-flash-sdpa, "When MFA Dispatches vs. Falls Back";
MLX pull request, "Limitations"), run in the library too: a boolean mask keeps the keys
where it is True, a mask of the operand dtype is added to the scaled scores, and the
sinks (float32, one logit per query head) get a gradient; the mask gets none.
"""

from __future__ import annotations

import math

import torch

from . import _lib

# The eligibility rules live with the binding, which applies them on every call.
check_eligible = _lib.check_eligible


class _Attention(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, scale, is_causal, attn_mask, sinks):
        need_grad = any(ctx.needs_input_grad[:3]) or ctx.needs_input_grad[6]
        o, lse = _lib.sdpa_fwd(q, k, v, scale=scale, is_causal=is_causal, need_lse=need_grad, attn_mask=attn_mask,
                               sinks=sinks)
        if need_grad:
            ctx.save_for_backward(q, k, v, o, lse, attn_mask, sinks)
        ctx.scale, ctx.is_causal = scale, is_causal
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse, attn_mask, sinks = ctx.saved_tensors
        grads = _lib.sdpa_bwd(q, k, v, o, lse, do.to(q.dtype).contiguous(), scale=ctx.scale, is_causal=ctx.is_causal,
                              attn_mask=attn_mask, sinks=sinks)
        dsinks = grads[3] if sinks is not None else None
        return grads[0], grads[1], grads[2], None, None, None, dsinks


def attention(q, k, v, scale=None, is_causal=False, attn_mask=None, sinks=None):
    """softmax(q k^T * scale [+ causal or attn_mask], with sinks) v for [B, H, L, D] tensors, differentiable.

    ``scale`` defaults to 1/sqrt(D), rounded to float32 as the library receives it.
    K and V may have fewer heads than Q (grouped-query attention). ``attn_mask``
    (bool, or q's dtype) broadcasts to [B, Hq, Lq, Lkv]; ``sinks`` is float32 [Hq]."""
    check_eligible(q, k, v, is_causal, attn_mask, sinks)
    if scale is None:
        scale = float(torch.tensor(1.0 / math.sqrt(q.shape[-1]), dtype=torch.float32))
    return _Attention.apply(q.contiguous(), k.contiguous(), v.contiguous(), float(scale), bool(is_causal), attn_mask,
                            None if sinks is None else sinks.contiguous())
