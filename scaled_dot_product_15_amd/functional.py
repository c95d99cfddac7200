"""Differentiable attention: the library's forward and backward as one
torch.autograd.Function.

The forward calls attn_fwd (or attn_fwd_bias) and keeps Q, K, V, O and the
row LSE; the backward calls attn_bwd with the same mask, softmax, dropout
state and bias, and returns the gradients of the inputs that require them
(Q, K, V, the learnable sink logits, the bias).  This mirrors the pages'
framework modules, which wrap the fused forward and backward calls as one
operation with a custom gradient (PR #2225's sequence diagrams: the forward
returns the output and the softmax statistics, the backward takes dO and
returns grad_q, grad_k, grad_v, grad_softmax_offset; TE's single-GPU page
passes a bias and a dropout rate to the same module).  Argument marshalling
only: every step runs in the library's kernels.
"""
from __future__ import annotations

from . import binding


def _autograd_function():
    import torch

    class _Attention(torch.autograd.Function):
        @staticmethod
        def forward(ctx, q, k, v, softmax_offset, bias, opts):
            o, lse = binding.attn_fwd(q, k, v, softmax_offset=softmax_offset, bias=bias, **opts)
            ctx.save_for_backward(q, k, v, o, lse, softmax_offset, bias)
            ctx.opts = opts
            return o

        @staticmethod
        def backward(ctx, d_o):
            q, k, v, o, lse, softmax_offset, bias = ctx.saved_tensors
            want_offset = softmax_offset is not None and ctx.needs_input_grad[3]
            want_bias = bias is not None and ctx.needs_input_grad[4]
            res = binding.attn_bwd(q, k, v, o, lse, d_o.contiguous(), softmax_offset=softmax_offset, bias=bias,
                                   want_d_bias=want_bias, **ctx.opts)
            dq, dk, dv, doff = res[:4]
            d_offset = doff.reshape(softmax_offset.shape).to(softmax_offset.dtype) if want_offset else None
            d_bias = res[4] if want_bias else None
            return dq, dk, dv, d_offset, d_bias, None

    return _Attention


_FN = None


def attention(q, k, v, *, num_gqa_groups=None, attn_mask_type="causal", window_size=(-1, -1),
              scale_factor=None, softmax_type="vanilla", softmax_offset=None, seqlens=None, seq_offsets=None,
              max_seqlen=None, dropout_p=0.0, rng_state=(0, 0), bias=None):
    """Attention output O (layouts as binding.attn_fwd) with autograd support.

    softmax_offset: the learnable sink logits [Hq] (softmax_type
    "learnable"); a tensor that requires grad receives d(loss)/d(offset).
    bias: an additive post-scale bias [1 or B, 1 or Hq, S, S]; it receives
    its gradient when it requires grad.  dropout_p / rng_state: attention
    dropout; the backward regenerates the same keep mask from rng_state.
    """
    global _FN
    if _FN is None:
        _FN = _autograd_function()
    opts = dict(num_gqa_groups=num_gqa_groups, attn_mask_type=attn_mask_type, window_size=window_size,
                scale_factor=scale_factor, softmax_type=softmax_type, seqlens=seqlens, seq_offsets=seq_offsets,
                max_seqlen=max_seqlen, dropout_p=dropout_p, rng_state=rng_state)
    return _FN.apply(q, k, v, softmax_offset, bias, opts)
