"""Differentiable exact attention on the HIP kernels.

``attention`` and ``scaled_dot_product_attention`` wrap ``fa_fwd_strided``
/ ``fa_bwd_strided`` (every mask and dropout option of the library) in a
``torch.autograd.Function``:
the forward saves q, k, v, O and the per-row log-sum-exp, and the backward
recomputes the probabilities from them on the GPU ([ODP] "FlashAttention:
Fast and Memory-Efficient Exact Attention with IO-Awareness", section "The
key idea"; [DEC] "FlashAttention, Decoded", "The Hardware Picture: Why
Tiling Wins").  Nothing of size N x N is stored between the two passes.

Dropout (``dropout_p``) runs in the kernels too: the backward regenerates
the forward's mask from its seed instead of storing it.

Like the rest of the binding this only marshals tensors: every step of the
computation runs in ``libfa.so``; there is no PyTorch fallback.  The
kernels read and write strided views in place (``fa_fwd_strided``,
``fa_bwd_strided``), so the ``[B, N, H, d]`` layout (``layout="bnhd"``) and
non-contiguous SDPA inputs reach them without transposing copies; the
output and the gradients keep the inputs' memory order.
"""

from __future__ import annotations

import torch

from . import fa_bwd_strided, fa_fwd_strided

__all__ = ["FlashAttention", "attention", "scaled_dot_product_attention"]


class FlashAttention(torch.autograd.Function):
    """O = softmax(q k^T * scale + mask) v with the mask given by ``causal``,
    ``key_len`` (keys j >= key_len[b] hidden) or a 128x128 ``block_mask``,
    and optionally dropout on the probabilities (``dropout`` = (p, seed,
    offset); the backward regenerates the same mask from them).
    q, k, v: [B, H, N, d] views of any strides with a contiguous d, fp32,
    fp16 or bf16 (block_mask and dropout: fp16 or bf16)."""

    @staticmethod
    def forward(ctx, q, k, v, scale, causal, key_len, block_mask, dropout):
        p, seed, offset = dropout if dropout is not None else (0.0, 0, 0)
        o, lse = fa_fwd_strided(q, k, v, scale=scale, causal=causal, key_len=key_len,
                                block_mask=block_mask, dropout_p=p, seed=seed, offset=offset)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.scale, ctx.causal, ctx.key_len, ctx.block_mask = scale, causal, key_len, block_mask
        ctx.dropout = (p, seed, offset)
        return o

    @staticmethod
    def backward(ctx, dO):
        q, k, v, o, lse = ctx.saved_tensors
        p, seed, offset = ctx.dropout
        dq, dk, dv = fa_bwd_strided(q, k, v, o, lse, dO, scale=ctx.scale, causal=ctx.causal,
                                    key_len=ctx.key_len, block_mask=ctx.block_mask,
                                    dropout_p=p, seed=seed, offset=offset)
        return dq, dk, dv, None, None, None, None, None


def attention(q, k, v, *, causal=False, scale=None, key_len=None, block_mask=None,
              dropout_p=0.0, seed=None, offset=0, layout="bhnd"):
    """Differentiable exact attention.

    layout "bhnd": q, k, v are [B, H, N, d]; "bnhd": [B, N, H, d] (the
    result has the same layout).  scale defaults to 1/sqrt(d).  key_len:
    int32 [B] on the GPU; block_mask: uint8 [ceil(N/128)]^2 on the GPU
    (not combined with causal, key_len or dropout).  dropout_p > 0 drops
    probabilities with that rate; the mask is a function of (seed, offset)
    and the element's indices (seed defaults to a draw from torch's CPU
    generator, so torch.manual_seed makes it reproducible).
    """
    if layout not in ("bhnd", "bnhd"):
        raise ValueError("layout must be 'bhnd' or 'bnhd'")
    if block_mask is not None and (causal or key_len is not None):
        raise ValueError("block_mask is not combined with causal or key_len")
    if not 0.0 <= float(dropout_p) < 1.0:
        raise ValueError("dropout_p must be in [0, 1)")
    dropout = None
    if dropout_p > 0.0:
        if block_mask is not None:
            raise ValueError("block_mask is not combined with dropout")
        if seed is None:
            seed = int(torch.randint(0, 1 << 62, (1,)).item())
        dropout = (float(dropout_p), int(seed), int(offset))
    if layout == "bnhd":
        q, k, v = (t.transpose(1, 2) for t in (q, k, v))
    o = FlashAttention.apply(q, k, v, scale, bool(causal), key_len, block_mask, dropout)
    return o.transpose(1, 2) if layout == "bnhd" else o


def scaled_dot_product_attention(query, key, value, attn_mask=None, dropout_p=0.0,
                                 is_causal=False, scale=None):
    """The argument list of ``torch.nn.functional.scaled_dot_product_attention``
    for [B, H, N, d] inputs of one sequence length.  Masks are given as
    ``is_causal``; use ``attention`` for key-padding lengths or a block
    mask.  dropout_p > 0 applies dropout with a seed drawn from torch's CPU
    generator."""
    if attn_mask is not None:
        raise ValueError("attn_mask is not supported: use is_causal, or attention(key_len=..., "
                         "block_mask=...)")
    return attention(query, key, value, causal=is_causal, scale=scale, dropout_p=dropout_p)
