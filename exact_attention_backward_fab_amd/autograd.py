"""torch.autograd binding: attention whose backward is libfab's fused backward.

The forward saves O and the row LSE (fab_forward_lse); the backward hands them
to fab_backward, which writes dQ, dK and dV into one packed f32 blob, and the
gradients returned to autograd are views of that blob at its padded offsets
(the ggmlR test "autodiff views address their own slice of the packed buffer"
checks the same property of ggml's graph).  Argument marshalling only: all the
arithmetic runs in the library's kernels.

    O = attention(q, k, v, mask=None, scale=None, mode="f32", causal=False, alibi=None)

q (B,H,N,DK), k (B,Hkv,M,DK), v (B,Hkv,M,DV) CUDA tensors, mask (N,M) f16 bit
patterns or None, alibi (H,) float32 per-head slopes or None, O (B,N,H,DV).
No gradient flows to the mask or the slopes.

float32 inputs give a float32 O and float32 gradients (any mode).  bfloat16 inputs
(mode "bf16") stay bfloat16 end to end: O is stored as bf16 (FAB_BF16_O, the f32
output rounded to nearest even), so the upstream gradient arrives as bf16 and is
read as such (FAB_BF16_INPUTS), and the gradients are bf16 views of one bf16 blob
(FAB_BF16_BLOB: the f32 gradients rounded once).  float16 inputs are refused: the
library stores O as f32 or bf16 only, so their upstream gradient would not be f16.
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
        if q.dtype == torch.float16:
            raise TypeError("attention(): float16 inputs are not supported (O is stored as f32 or bf16, so the "
                            "upstream gradient would not be f16); call fab.backward with f16 q, k, v, d directly")
        O, lse = _forward_lse(q, k, v, scale, mask=mask, mode=mode, causal=causal, alibi=alibi,
                              o_bf16=q.dtype == torch.bfloat16)
        ctx.save_for_backward(q, k, v, O, lse)
        ctx.mask, ctx.scale, ctx.mode, ctx.causal, ctx.alibi = mask, scale, mode, causal, alibi
        return O

    @staticmethod
    def backward(ctx, dO):
        q, k, v, O, lse = ctx.saved_tensors
        # bf16 inputs: dO (the gradient of a bf16 O) is bf16 too, and so is the blob
        blob = _backward(q, k, v, dO.to(q.dtype).contiguous(), ctx.scale, mask=ctx.mask, mode=ctx.mode, O=O,
                         lse=lse, causal=ctx.causal, alibi=ctx.alibi, blob_dtype=q.dtype)
        dq, dk, dv = unpack(blob, shape_of(q, k, v))
        return dq, dk, dv, None, None, None, None, None


def attention(q, k, v, mask=None, scale=None, mode="f32", causal=False, alibi=None):
    """softmax(scale * q.k^T + alibi_h (m - n) + mask) v with the fused backward; scale
    defaults to 1/sqrt(DK); causal=True applies the causal rule (key m seen by query n iff
    m <= n) without a mask; alibi: per-head slopes (H,) float32 or None."""
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    return FabAttention.apply(q, k, v, mask, float(scale), mode, bool(causal), alibi)
