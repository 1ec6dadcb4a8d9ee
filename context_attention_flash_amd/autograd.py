"""PyTorch autograd wrapper over the rank-share entry points.

The call surface follows the ring-attention function the pages show
("How to Implement Ring Attention for Long Sequences in Nanotron", "Calling the
Ring Attention Function Directly"): q, k, v, optional cu_seqlens and
max_seqlen, dropout, softmax scale (None -> 1/sqrt(head_dim)), causal,
window_size, alibi_slopes, deterministic, return_attn_probs and the process
group.  On one GPU the process group becomes the integers (world, rank), and
k / v hold every KV block the rank meets, block-major: [nb, B, Skv, Hkv, d]
(the varlen form also takes the packed [nb, Skv, Hkv, d] without the batch
axis).  Forward calls ``ring_attn_fwd``; backward calls ``ring_attn_bwd`` with
the saved out and lse.  The gradient of k / v is this rank's contribution to
every block, so summing it over the ranks gives the full dK / dV.

Only argument marshalling happens here: shapes into a descriptor, views that
add or drop the batch axis of the packed form, contiguity of the incoming
gradient, and the cast of the fp32 gradients to the inputs' dtype.
"""
from __future__ import annotations

from typing import Optional, Sequence

import torch

from . import (BASIC, LLAMA3, RA_MERGE_FUSED, VARLEN_RING, make_desc, ring_attn_bwd,
               ring_attn_fwd)
from .synth import VARLEN_LAYOUTS


def _check_unsupported(dropout_p, alibi_slopes, window_size):
    if dropout_p != 0.0:
        raise NotImplementedError("dropout_p must be 0: attention dropout is not implemented")
    if alibi_slopes is not None:
        raise NotImplementedError("alibi_slopes are not implemented")
    if len(window_size) != 2 or min(window_size) < -1:
        raise ValueError(f"window_size must be (left, right) with each side >= -1, got {window_size}")


class _RingFlashAttn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, desc_kw, cu_seqlens):
        desc = make_desc(**desc_kw)
        out, lse = ring_attn_fwd(desc, q, k, v, cu_seqlens)
        ctx.save_for_backward(q, k, v, out, lse)
        ctx.desc_kw = desc_kw
        ctx.cu_seqlens = cu_seqlens
        ctx.mark_non_differentiable(lse)
        return out, lse

    @staticmethod
    def backward(ctx, dout, _dlse):
        q, k, v, out, lse = ctx.saved_tensors
        desc = make_desc(**ctx.desc_kw)
        dq, dk, dv = ring_attn_bwd(desc, dout.contiguous(), q, k, v, out, lse, ctx.cu_seqlens)
        return dq.to(q.dtype), dk.to(k.dtype), dv.to(v.dtype), None, None


def _desc_kw(q, k, world, rank, layout, causal, softmax_scale, window_size, cu_seqlens):
    if q.dim() != 4 or k.dim() != 5:
        raise ValueError("q must be [B, S, Hq, d] and k, v [nb, B, Skv, Hkv, d]")
    if q.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError(f"q dtype {q.dtype}: bfloat16 or float32 expected")
    B, S, Hq, d = q.shape
    nb, Bk, Skv, Hkv, dk = k.shape
    if Bk != B or dk != d:
        raise ValueError(f"k shape {tuple(k.shape)} does not match q shape {tuple(q.shape)}")
    seqlen = Skv if layout == LLAMA3 else S * world
    return dict(batch=B, heads_q=Hq, heads_kv=Hkv, head_dim=d, seqlen=seqlen, world=world,
                rank=rank, causal=bool(causal), layout=layout,
                dtype="bf16" if q.dtype == torch.bfloat16 else "f32",
                softmax_scale=0.0 if softmax_scale is None else float(softmax_scale),
                cu_seqlens=cu_seqlens, merge_mode=RA_MERGE_FUSED,
                window=(int(window_size[0]), int(window_size[1])))


def ring_flash_attn_func(q, k, v, dropout_p: float = 0.0, softmax_scale: Optional[float] = None,
                         causal: bool = False, window_size=(-1, -1), alibi_slopes=None,
                         deterministic: bool = False, return_attn_probs: bool = False, *,
                         world: int = 1, rank: int = 0, layout: int = BASIC):
    """Batch form.  q [B, S, Hq, d] (the rank's rows in local order), k and v
    [nb, B, Skv, Hkv, d] block-major, bf16 or fp32 (backward: bf16 only).
    ``layout`` is BASIC, ZIGZAG or STRIPE.  Returns out [B, S, Hq, d], or
    (out, lse [B, Hq, S] fp32, None) with ``return_attn_probs``.  The kernels
    use no atomics, so results are deterministic whatever ``deterministic``
    says."""
    _check_unsupported(dropout_p, alibi_slopes, window_size)
    if layout in VARLEN_LAYOUTS:
        raise ValueError("packed layouts go through ring_flash_attn_varlen_func")
    kw = _desc_kw(q, k, world, rank, layout, causal, softmax_scale, window_size, None)
    out, lse = _RingFlashAttn.apply(q, k, v, kw, None)
    return (out, lse, None) if return_attn_probs else out


def ring_flash_attn_varlen_func(q, k, v, cu_seqlens: Sequence[int], max_seqlen=None,
                                dropout_p: float = 0.0, softmax_scale: Optional[float] = None,
                                causal: bool = False, window_size=(-1, -1), alibi_slopes=None,
                                deterministic: bool = False, return_attn_probs: bool = False, *,
                                world: int = 1, rank: int = 0, layout: int = VARLEN_RING):
    """Packed (varlen) form.  q [S, Hq, d] (or [1, S, Hq, d]): the rank's rows
    of the packed stream in local order; k, v [nb, Skv, Hkv, d] (or
    [nb, 1, Skv, Hkv, d]); ``cu_seqlens`` (host sequence of ints) in global
    packed coordinates.  ``layout`` is VARLEN_RING, VARLEN_ZIGZAG,
    VARLEN_STRIPE or LLAMA3.  ``max_seqlen`` is accepted for call
    compatibility and not needed: the kernels take per-row key intervals.
    Returns out shaped like q, or (out, lse [Hq, S] or [1, Hq, S], None)."""
    _check_unsupported(dropout_p, alibi_slopes, window_size)
    if layout not in VARLEN_LAYOUTS:
        raise ValueError("batch layouts go through ring_flash_attn_func")
    packed = q.dim() == 3
    if packed:
        if k.dim() != 4 or v.dim() != 4:
            raise ValueError("packed q [S, Hq, d] needs k, v [nb, Skv, Hkv, d]")
        q, k, v = q.unsqueeze(0), k.unsqueeze(1), v.unsqueeze(1)
    cu = [int(c) for c in cu_seqlens]
    kw = _desc_kw(q, k, world, rank, layout, causal, softmax_scale, window_size, cu)
    if layout != LLAMA3 and kw["seqlen"] != cu[-1]:
        raise ValueError(f"cu_seqlens ends at {cu[-1]}, but world * local rows = {kw['seqlen']}")
    out, lse = _RingFlashAttn.apply(q, k, v, kw, cu)
    if packed:
        out, lse = out.squeeze(0), lse.squeeze(0)
    return (out, lse, None) if return_attn_probs else out
