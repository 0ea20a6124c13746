"""Autograd-facing forms of the virtual ring, mirroring the reference API's
function family ("Ring Flash Attention" README, function list: ring /
zigzag ring / stripe functions, each with plain, kv-packed and qkv-packed
forms, and a varlen form taking one cu_seqlens).

Every function here computes on ONE GPU: the global sequence is laid out
into the N ranks' local chunks by the library's layout positions, every
rank's share runs through ra_ring_fwd / ra_ring_bwd (the virtual ring), and
the per-rank results are scattered back to global token order.  Packed
inputs are accepted as strided views: the ring forms gather them into
rank-major K/V rings (one copy, as a real ring's send buffers would be), and
the block step (`gathered_share_attn`, `api.block_attn_fwd`) reads strided
views in place.  Gradients are exact softmax-attention gradients (the
backward recomputes P from the saved lse).

The llama3-style context-parallel share (SourcePulse summary of the
reference, "How It Works" / "Highlighted Details": gather all K/V, then a
rank attends its local queries against them; recommended there for varlen)
is `gathered_share_attn` for one rank and `gathered_attn_func` /
`llama3_attn_varlen_func` for every rank of a virtual context-parallel group:
one block step per rank over the whole gathered K/V (ra_gathered_fwd /
ra_gathered_bwd), differentiable.

Low-precision results (the bf16 output of a bf16 call, and the bf16 gradients)
come from the library as well: the forward kernel writes the bf16 copy of the
output with the last ring step, and the gradients are cast by
ra_cast_f32_to_bf16 (round to nearest, ties to even).
"""
from __future__ import annotations

from typing import Optional, Sequence

from . import api


def _torch():
    import torch
    return torch


def _lowp(x32, dtype):
    """``x32`` (fp32) in ``dtype``: itself for fp32, the library's RNE copy for bf16."""
    torch = _torch()
    if dtype == torch.float32:
        return x32
    if dtype == torch.bfloat16:
        return api.cast_f32_to_bf16(x32.contiguous())
    raise TypeError(f"unsupported dtype {dtype} (bf16 or fp32)")


def _cu_once(cu_seqlens, device):
    """Host and device copies of cu_seqlens made once for all the calls of one
    forward and backward (None stays None)."""
    if cu_seqlens is None or isinstance(cu_seqlens, api.CuSeqlens):
        return cu_seqlens
    return api.CuSeqlens(cu_seqlens, device)


def _positions(layout: str, S: int, world: int, device, cu_seqlens=None):
    torch = _torch()
    cu = cu_seqlens if layout.endswith("_varlen") else None  # only the per-sequence layouts use it
    return [torch.from_numpy(api.layout_positions(layout, S, world, r, cu)).to(device) for r in range(world)]


class _VirtualRing:
    """Shared forward/backward of the virtual ring over global [b, S, h, d] tensors."""

    @staticmethod
    def forward(q, k, v, layout, world, causal, cu_seqlens, scale):
        torch = _torch()
        b, S, h, d = q.shape
        idx = _positions(layout, S, world, q.device, cu_seqlens)
        k_ring = torch.stack([k.index_select(1, i) for i in idx]).contiguous()
        v_ring = torch.stack([v.index_select(1, i) for i in idx]).contiguous()
        out = torch.empty((b, S, h, d), device=q.device, dtype=q.dtype)
        lse = torch.empty((b, h, S), device=q.device, dtype=torch.float32)
        outs, lses = [], []
        lowp = q.dtype != torch.float32
        for r in range(world):
            ql = q.index_select(1, idx[r]).contiguous()
            o32, l, olp = api.ring_fwd(layout, world, r, ql, k_ring, v_ring, causal=causal, cu_seqlens=cu_seqlens,
                                       scale=scale, want_lowp=lowp)
            outs.append(o32)
            lses.append(l)
            out.index_copy_(1, idx[r], olp if lowp else o32)
            lse.index_copy_(2, idx[r], l)
        return out, lse, (idx, k_ring, v_ring, outs, lses)

    @staticmethod
    def backward(q, dout, layout, world, causal, cu_seqlens, scale, saved):
        torch = _torch()
        idx, k_ring, v_ring, outs, lses = saved
        b, S, h, d = q.shape
        dq = torch.empty((b, S, h, d), device=q.device, dtype=torch.float32)
        dk_ring = torch.zeros(k_ring.shape, device=q.device, dtype=torch.float32)
        dv_ring = torch.zeros(v_ring.shape, device=q.device, dtype=torch.float32)
        for r in range(world):
            ql = q.index_select(1, idx[r]).contiguous()
            dol = dout.index_select(1, idx[r]).contiguous().to(q.dtype)
            dqr, _, _ = api.ring_bwd(layout, world, r, ql, k_ring, v_ring, outs[r], lses[r], dol, causal=causal,
                                     cu_seqlens=cu_seqlens, scale=scale, dk_ring=dk_ring, dv_ring=dv_ring)
            dq.index_copy_(1, idx[r], dqr)
        dk = torch.empty((b, S, h, d), device=q.device, dtype=torch.float32)
        dv = torch.empty((b, S, h, d), device=q.device, dtype=torch.float32)
        for r in range(world):
            dk.index_copy_(1, idx[r], dk_ring[r])
            dv.index_copy_(1, idx[r], dv_ring[r])
        return dq, dk, dv


def _make_function():
    torch = _torch()

    class RingAttentionFn(torch.autograd.Function):
        @staticmethod
        def forward(ctx, q, k, v, layout, world, causal, cu_seqlens, scale):
            cu_seqlens = _cu_once(cu_seqlens, q.device)
            out, lse, saved = _VirtualRing.forward(q.detach(), k.detach(), v.detach(), layout, world, causal,
                                                   cu_seqlens, scale)
            ctx.saved = saved
            ctx.args = (layout, world, causal, cu_seqlens, scale)
            ctx.save_for_backward(q.detach())
            ctx.dtypes = (q.dtype, k.dtype, v.dtype)
            ctx.mark_non_differentiable(lse)
            return out, lse

        @staticmethod
        def backward(ctx, dout, _dlse):
            (q,) = ctx.saved_tensors
            layout, world, causal, cu_seqlens, scale = ctx.args
            dq, dk, dv = _VirtualRing.backward(q, dout.contiguous(), layout, world, causal, cu_seqlens, scale,
                                               ctx.saved)
            ctx.saved = None
            qd, kd, vd = ctx.dtypes
            return _lowp(dq, qd), _lowp(dk, kd), _lowp(dv, vd), None, None, None, None, None

    return RingAttentionFn


_FN = None


def ring_attn_func(q, k, v, *, layout: str = "zigzag", world: int = 8, causal: bool = True,
                   softmax_scale: Optional[float] = None, return_lse: bool = False):
    """Exact attention of global [b, S, h, d] q/k/v through an N-rank virtual ring.

    Differentiable with respect to q, k and v.  Returns out (q.dtype) and, when
    asked, the fp32 lse [b, h, S]."""
    global _FN
    if _FN is None:
        _FN = _make_function()
    out, lse = _FN.apply(q, k, v, layout, world, causal, None, softmax_scale)
    return (out, lse) if return_lse else out


def ring_attn_varlen_func(q, k, v, cu_seqlens: Sequence[int], *, layout: str = "contiguous", world: int = 8,
                          causal: bool = True, softmax_scale: Optional[float] = None, return_lse: bool = False):
    """Packed variable-length form: q/k/v are [1, T, h, d] (or [T, h, d]) holding
    several sequences back to back, delimited by ONE cu_seqlens shared by q and
    k/v (int32 global offsets, first 0, last T).  ``layout`` lays out the packed
    stream as a whole (contiguous, zigzag, stripe) or every sequence on its own
    (zigzag_varlen, stripe_varlen: each length divisible by 2*world / world)."""
    global _FN
    if _FN is None:
        _FN = _make_function()
    squeeze = q.dim() == 3
    if squeeze:
        q, k, v = q.unsqueeze(0), k.unsqueeze(0), v.unsqueeze(0)
    out, lse = _FN.apply(q, k, v, layout, world, causal, cu_seqlens, softmax_scale)
    if squeeze:
        out = out.squeeze(0)
    return (out, lse) if return_lse else out


def ring_attn_kvpacked_func(q, kv, **kw):
    """kv: [b, S, 2, h, d] (K then V along dim 2), taken as strided views."""
    return ring_attn_func(q, kv[:, :, 0], kv[:, :, 1], **kw)


def ring_attn_qkvpacked_func(qkv, **kw):
    """qkv: [b, S, 3, h, d] (Q, K, V along dim 2), taken as strided views."""
    return ring_attn_func(qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2], **kw)


def _make_gathered_function():
    torch = _torch()

    class GatheredShareFn(torch.autograd.Function):
        """One rank's share against the whole gathered K/V (global order)."""

        @staticmethod
        def forward(ctx, q_local, k_all, v_all, layout, world, rank, causal, cu_seqlens, scale):
            q_local, k_all, v_all = q_local.detach(), k_all.detach(), v_all.detach()
            cu_seqlens = _cu_once(cu_seqlens, q_local.device)
            lowp = q_local.dtype != torch.float32
            o32, lse, olp = api.gathered_fwd(layout, world, rank, q_local, k_all, v_all, causal=causal,
                                             cu_seqlens=cu_seqlens, scale=scale, want_lowp=lowp)
            ctx.save_for_backward(q_local, k_all, v_all, o32, lse)
            ctx.args = (layout, world, rank, causal, cu_seqlens, scale)
            ctx.mark_non_differentiable(lse)
            return (olp if lowp else o32), lse

        @staticmethod
        def backward(ctx, dout, _dlse):
            q_local, k_all, v_all, o32, lse = ctx.saved_tensors
            layout, world, rank, causal, cu_seqlens, scale = ctx.args
            dq, dk, dv = api.gathered_bwd(layout, world, rank, q_local, k_all, v_all, o32, lse,
                                          dout.contiguous().to(q_local.dtype), causal=causal,
                                          cu_seqlens=cu_seqlens, scale=scale)
            return (_lowp(dq, q_local.dtype), _lowp(dk, k_all.dtype), _lowp(dv, v_all.dtype),
                    None, None, None, None, None, None)

    return GatheredShareFn


_GFN = None


def gathered_share_attn(q_local, k_all, v_all, *, layout: str = "contiguous", world: int = 8, rank: int = 0,
                        causal: bool = True, cu_seqlens=None, softmax_scale: Optional[float] = None):
    """One rank's share when all K/V have been gathered (llama3-style context
    parallelism): q_local [b, S/N, h, d] of `rank` in `layout` (contiguous, zigzag
    or stripe) attends to the whole k_all/v_all [b, S, h, d] in global order, as a
    single block step.  Returns (out in q_local's dtype, lse fp32 [b, h, S/N]);
    differentiable with respect to q_local, k_all and v_all."""
    global _GFN
    if _GFN is None:
        _GFN = _make_gathered_function()
    return _GFN.apply(q_local, k_all, v_all, layout, world, rank, causal, cu_seqlens, softmax_scale)


def _make_gathered_group_function():
    torch = _torch()

    class GatheredGroupFn(torch.autograd.Function):
        """Every rank of an N-rank llama3-style group, gradients summed over the
        ranks in fp32 before the one cast to the input dtype."""

        @staticmethod
        def forward(ctx, q, k, v, layout, world, causal, cu_seqlens, scale):
            q, k, v = q.detach(), k.detach(), v.detach()
            cu_seqlens = _cu_once(cu_seqlens, q.device)
            b, S, h, d = q.shape
            idx = _positions(layout, S, world, q.device)
            lowp = q.dtype != torch.float32
            out = torch.empty((b, S, h, d), device=q.device, dtype=q.dtype)
            lse = torch.empty((b, h, S), device=q.device, dtype=torch.float32)
            saved = []
            for r in range(world):
                ql = q.index_select(1, idx[r]).contiguous()
                o32, l, olp = api.gathered_fwd(layout, world, r, ql, k, v, causal=causal, cu_seqlens=cu_seqlens,
                                               scale=scale, want_lowp=lowp)
                saved.append((o32, l))
                out.index_copy_(1, idx[r], olp if lowp else o32)
                lse.index_copy_(2, idx[r], l)
            ctx.saved = (idx, saved)
            ctx.args = (layout, world, causal, cu_seqlens, scale)
            ctx.save_for_backward(q, k, v)
            ctx.mark_non_differentiable(lse)
            return out, lse

        @staticmethod
        def backward(ctx, dout, _dlse):
            q, k, v = ctx.saved_tensors
            idx, saved = ctx.saved
            layout, world, causal, cu_seqlens, scale = ctx.args
            b, S, h, d = q.shape
            dq = torch.empty((b, S, h, d), device=q.device, dtype=torch.float32)
            dk = torch.zeros((b, S, h, d), device=q.device, dtype=torch.float32)
            dv = torch.zeros((b, S, h, d), device=q.device, dtype=torch.float32)
            dout = dout.contiguous().to(q.dtype)
            for r in range(world):
                ql = q.index_select(1, idx[r]).contiguous()
                dol = dout.index_select(1, idx[r]).contiguous()
                o32, l = saved[r]
                dqr, _, _ = api.gathered_bwd(layout, world, r, ql, k, v, o32, l, dol, causal=causal,
                                             cu_seqlens=cu_seqlens, scale=scale, dk_all=dk, dv_all=dv)
                dq.index_copy_(1, idx[r], dqr)
            ctx.saved = None
            return (_lowp(dq, q.dtype), _lowp(dk, k.dtype), _lowp(dv, v.dtype), None, None, None, None, None)

    return GatheredGroupFn


_GGFN = None


def gathered_attn_func(q, k, v, *, layout: str = "contiguous", world: int = 8, causal: bool = True,
                       cu_seqlens=None, softmax_scale: Optional[float] = None, return_lse: bool = False):
    """Exact attention of global [b, S, h, d] q/k/v as an N-rank llama3-style group:
    every rank's local queries (in ``layout``) attend to the whole gathered K/V, and
    the ranks' outputs go back to global order.  Differentiable; the K/V gradients are
    the sum of every rank's contribution (what a reduce-scatter would return)."""
    global _GGFN
    if _GGFN is None:
        _GGFN = _make_gathered_group_function()
    out, lse = _GGFN.apply(q, k, v, layout, world, causal, cu_seqlens, softmax_scale)
    return (out, lse) if return_lse else out


def llama3_attn_varlen_func(q, k, v, cu_seqlens: Sequence[int], *, world: int = 8, causal: bool = True,
                            softmax_scale: Optional[float] = None, return_lse: bool = False):
    """Packed variable-length sequences ([1, T, h, d] or [T, h, d], ONE cu_seqlens)
    through the llama3-style group: rank r holds the r-th contiguous slice of the
    packed queries and attends to all gathered K/V of its sequences."""
    squeeze = q.dim() == 3
    if squeeze:
        q, k, v = q.unsqueeze(0), k.unsqueeze(0), v.unsqueeze(0)
    res = gathered_attn_func(q, k, v, layout="contiguous", world=world, causal=causal, cu_seqlens=cu_seqlens,
                             softmax_scale=softmax_scale, return_lse=True)
    out, lse = res
    if squeeze:
        out = out.squeeze(0)
    return (out, lse) if return_lse else out
