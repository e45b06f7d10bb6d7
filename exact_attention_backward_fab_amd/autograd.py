"""torch.autograd binding: attention whose backward is libfab's fused backward.

The forward saves O and the row LSE (fab_forward_lse); the backward hands them
to fab_backward, which writes dQ, dK and dV into one packed f32 blob, and the
gradients returned to autograd are views of that blob at its padded offsets
(the ggmlR test "autodiff views address their own slice of the packed buffer"
checks the same property of ggml's graph).  Argument marshalling only: all the
arithmetic runs in the library's kernels.

    O = attention(q, k, v, mask=None, scale=None, mode="f32", causal=False, alibi=None)

q (B,H,N,DK), k (B,Hkv,M,DK), v (B,Hkv,M,DV) float32 CUDA tensors, mask (N,M)
f16 bit patterns or None, alibi (H,) float32 per-head slopes or None, O (B,N,H,DV).
No gradient flows to the mask or the slopes.
"""
from __future__ import annotations

import math

import torch

from . import backward as _backward
from . import forward_lse as _forward_lse
from . import shape_of, unpack


class FabAttention(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, mask, scale, mode, causal, alibi):
        q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
        O, lse = _forward_lse(q, k, v, scale, mask=mask, mode=mode, causal=causal, alibi=alibi)
        ctx.save_for_backward(q, k, v, O, lse)
        ctx.mask, ctx.scale, ctx.mode, ctx.causal, ctx.alibi = mask, scale, mode, causal, alibi
        return O

    @staticmethod
    def backward(ctx, dO):
        q, k, v, O, lse = ctx.saved_tensors
        blob = _backward(q, k, v, dO.contiguous(), ctx.scale, mask=ctx.mask, mode=ctx.mode, O=O, lse=lse,
                         causal=ctx.causal, alibi=ctx.alibi)
        dq, dk, dv = unpack(blob, shape_of(q, k, v))
        return dq, dk, dv, None, None, None, None, None


def attention(q, k, v, mask=None, scale=None, mode="f32", causal=False, alibi=None):
    """softmax(scale * q.k^T + alibi_h (m - n) + mask) v with the fused backward; scale
    defaults to 1/sqrt(DK); causal=True applies the causal rule (key m seen by query n iff
    m <= n) without a mask; alibi: per-head slopes (H,) float32 or None."""
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    return FabAttention.apply(q, k, v, mask, float(scale), mode, bool(causal), alibi)
