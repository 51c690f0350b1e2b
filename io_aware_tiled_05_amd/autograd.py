"""Differentiable exact attention on the HIP kernels.

``attention`` and ``scaled_dot_product_attention`` wrap ``fa_fwd`` /
``fa_bwd`` (and their block-sparse forms) in a ``torch.autograd.Function``:
the forward saves q, k, v, O and the per-row log-sum-exp, and the backward
recomputes the probabilities from them on the GPU ([ODP] "FlashAttention:
Fast and Memory-Efficient Exact Attention with IO-Awareness", section "The
key idea"; [DEC] "FlashAttention, Decoded", "The Hardware Picture: Why
Tiling Wins").  Nothing of size N x N is stored between the two passes.

Like the rest of the binding this only marshals tensors: every step of the
computation runs in ``libfa.so``; there is no PyTorch fallback.  The
kernels take contiguous ``[B, H, N, d]`` tensors; the ``[B, N, H, d]``
layout (``layout="bnhd"``) is accepted and copied to it on the way in (and
the gradients back).
"""

from __future__ import annotations

import torch

from . import fa_bwd, fa_bwd_blocksparse, fa_fwd, fa_fwd_blocksparse

__all__ = ["FlashAttention", "attention", "scaled_dot_product_attention"]


class FlashAttention(torch.autograd.Function):
    """O = softmax(q k^T * scale + mask) v with the mask given by ``causal``,
    ``key_len`` (keys j >= key_len[b] hidden) or a 128x128 ``block_mask``.
    q, k, v: contiguous [B, H, N, d] fp32, fp16 or bf16 (block_mask: fp16 or
    bf16)."""

    @staticmethod
    def forward(ctx, q, k, v, scale, causal, key_len, block_mask):
        q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
        if block_mask is not None:
            o, lse = fa_fwd_blocksparse(q, k, v, block_mask, scale=scale)
        else:
            o, lse = fa_fwd(q, k, v, scale=scale, causal=causal, key_len=key_len)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.scale, ctx.causal, ctx.key_len, ctx.block_mask = scale, causal, key_len, block_mask
        return o

    @staticmethod
    def backward(ctx, dO):
        q, k, v, o, lse = ctx.saved_tensors
        dO = dO.contiguous()
        if ctx.block_mask is not None:
            dq, dk, dv = fa_bwd_blocksparse(q, k, v, o, lse, dO, ctx.block_mask, scale=ctx.scale)
        else:
            dq, dk, dv = fa_bwd(q, k, v, o, lse, dO, scale=ctx.scale, causal=ctx.causal,
                                key_len=ctx.key_len)
        return dq, dk, dv, None, None, None, None


def attention(q, k, v, *, causal=False, scale=None, key_len=None, block_mask=None,
              layout="bhnd"):
    """Differentiable exact attention.

    layout "bhnd": q, k, v are [B, H, N, d]; "bnhd": [B, N, H, d] (the
    result has the same layout).  scale defaults to 1/sqrt(d).  key_len:
    int32 [B] on the GPU; block_mask: uint8 [ceil(N/128)]^2 on the GPU
    (not combined with causal or key_len).
    """
    if layout not in ("bhnd", "bnhd"):
        raise ValueError("layout must be 'bhnd' or 'bnhd'")
    if block_mask is not None and (causal or key_len is not None):
        raise ValueError("block_mask is not combined with causal or key_len")
    if layout == "bnhd":
        q, k, v = (t.transpose(1, 2) for t in (q, k, v))
    o = FlashAttention.apply(q, k, v, scale, bool(causal), key_len, block_mask)
    return o.transpose(1, 2) if layout == "bnhd" else o


def scaled_dot_product_attention(query, key, value, attn_mask=None, dropout_p=0.0,
                                 is_causal=False, scale=None):
    """The argument list of ``torch.nn.functional.scaled_dot_product_attention``
    for [B, H, N, d] inputs of one sequence length.  Dropout is not part of
    this path (dropout_p must be 0) and masks are given as ``is_causal``;
    use ``attention`` for key-padding lengths or a block mask."""
    if attn_mask is not None:
        raise ValueError("attn_mask is not supported: use is_causal, or attention(key_len=..., "
                         "block_mask=...)")
    if dropout_p != 0.0:
        raise ValueError("dropout is not supported (dropout_p must be 0)")
    return attention(query, key, value, causal=is_causal, scale=scale)
