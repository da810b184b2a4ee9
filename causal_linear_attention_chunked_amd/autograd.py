"""Autograd wrapper: chunked causal linear attention as a differentiable PyTorch op.

The call site the Fractus page describes ("Fractus-1B training optimization",
section 2, Opt 2) runs attention chunk by chunk and carries the state (S, z)
from one chunk to the next.  This module gives that op a backward:

    o, (S_out, z_out) = linear_attention(q, k, v, S_in=None, z_in=None, chunk=128)

q, k, v are (G, T, D) CUDA tensors (bf16 or fp32; q and k already positive, e.g.
elu(x) + 1); S_in (G, D, D) and z_in (G, D) are fp32 or None for a zero carry.
Where the library's sequence entry points take the shape (bf16; D = 64 in whole
128-token chunks, or D = 128 in chunks of a multiple of 64 tokens) the sequence is
one forward and one backward launch with the carry kept on chip; a sequence longer than
those calls take (SEQ_D64_MAX_T, SEQ_D128_MAX_T tokens) runs as consecutive segments of
whole chunks, each one such pair of launches, the carry passed from one to the next;
otherwise every chunk is one forward launch and its backward
one backward launch that recomputes the chunk from its saved inputs (q, k, v and
the carry that fed it).  Either way nothing of size (G, C, D, D) or (G, C, C) is
kept between the passes, the memory-flat principle of the page's section 1.  Gradients flow to q, k, v and,
when given, S_in and z_in; a loss on S_out / z_out reaches them too.

The implementation is selectable, as the page's call site selects its attention form
(section 2, Opt 1 and Opt 2: the chunked form next to the einsum and cumsum forms it
replaces).  Here the choice is among this library's GPU paths: "seq" (the sequence entry
points), "chunk" (the chunked form, one launch per chunk and direction, the carry through
memory), "cumsum" (the cumsum form: the per-token recurrence, block = 1 in the chunk entry
points, chunk by chunk with the carry) and "auto" (seq where it takes the shape, else
chunk).  linear_attention(impl=...) picks one per call; set_attention_impl() sets the
default, which otherwise comes from the environment variable LACHUNK_ATTN_IMPL, else
"auto".  The masked-einsum form, O(C^2 D^2) per chunk, is a reference in the oracle (test
infrastructure), not a product path.

The arithmetic runs in the HIP library only: CPU tensors raise.
"""
from __future__ import annotations

import os

import torch

from . import bwd as _bwd
from . import fwd as _fwd
from . import seq_bwd as _seq_bwd
from . import seq_fwd as _seq_fwd
from . import seq_supported as _seq_supported
from . import SEQ_D64_MAX_T, SEQ_D128_MAX_T


class ChunkFunction(torch.autograd.Function):
    """One chunk: (q, k, v, S_in, z_in) -> (o, S_out, z_out), backward by recomputation; block 64
    (the chunked form) or 1 (the cumsum form); feature "elu1" maps raw q, k inside."""

    @staticmethod
    def forward(ctx, q, k, v, S_in, z_in, block, feature=None):
        q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
        o, S_out, z_out = _fwd(q, k, v, S_in, z_in, block, feature=feature)
        ctx.block, ctx.feature = block, feature
        ctx.has_carry = S_in is not None
        ctx.save_for_backward(q, k, v, S_in, z_in)
        return o, S_out, z_out

    @staticmethod
    def backward(ctx, do, dS_out, dz_out):
        q, k, v, S_in, z_in = ctx.saved_tensors
        G, C, D = q.shape
        if do is None:
            do = torch.zeros_like(q)
        # the state gradients arrive together or not at all at the library
        if dS_out is None and dz_out is not None:
            dS_out = torch.zeros((G, D, D), dtype=torch.float32, device=q.device)
        if dz_out is None and dS_out is not None:
            dz_out = torch.zeros((G, D), dtype=torch.float32, device=q.device)
        dS_out = None if dS_out is None else dS_out.float().contiguous()
        dz_out = None if dz_out is None else dz_out.float().contiguous()
        dq, dk, dv, dS_in, dz_in = _bwd(q, k, v, S_in, z_in, do.to(q.dtype).contiguous(), dS_out, dz_out,
                                        ctx.block, feature=ctx.feature)
        if not ctx.has_carry:
            dS_in = dz_in = None
        return dq, dk, dv, dS_in, dz_in, None, None


class SeqFunction(torch.autograd.Function):
    """A whole sequence of chunks in one launch per direction (the library's sequence entry
    points); saves the inputs and the final carry with its remainders, from which the
    backward recovers the state before each chunk."""

    @staticmethod
    def forward(ctx, q, k, v, S_in, z_in, chunk, block, feature):
        q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
        o, S_out, z_out, S_res, z_res = _seq_fwd(q, k, v, S_in, z_in, chunk, block, feature=feature,
                                                 residual=True)
        ctx.chunk, ctx.block, ctx.feature = chunk, block, feature
        ctx.has_carry = S_in is not None
        ctx.save_for_backward(q, k, v, S_out, z_out, S_res, z_res)
        return o, S_out, z_out

    @staticmethod
    def backward(ctx, do, dS_out, dz_out):
        q, k, v, S_out, z_out, S_res, z_res = ctx.saved_tensors
        G, T, D = q.shape
        if do is None:
            do = torch.zeros_like(q)
        if dS_out is None and dz_out is not None:
            dS_out = torch.zeros((G, D, D), dtype=torch.float32, device=q.device)
        if dz_out is None and dS_out is not None:
            dz_out = torch.zeros((G, D), dtype=torch.float32, device=q.device)
        dS_out = None if dS_out is None else dS_out.float().contiguous()
        dz_out = None if dz_out is None else dz_out.float().contiguous()
        dq, dk, dv, dS_in, dz_in = _seq_bwd(q, k, v, S_out, z_out, do.to(q.dtype).contiguous(), dS_out, dz_out,
                                            ctx.chunk, ctx.block, feature=ctx.feature, S_res=S_res, z_res=z_res)
        if not ctx.has_carry:
            dS_in = dz_in = None
        return dq, dk, dv, dS_in, dz_in, None, None, None


def chunk_attention(q, k, v, S_in=None, z_in=None, block: int = 64, feature_map=None):
    """Differentiable single-chunk op: returns (o, S_out, z_out)."""
    _check_device(q)
    return ChunkFunction.apply(q, k, v, S_in, z_in, block, _fm(feature_map))


def seq_segments(dtype, T: int, D: int, chunk: int, feature=None):
    """Token counts of the consecutive segments a (G, T, D) sequence runs as through the sequence
    entry points: [T] where they take all T tokens; for a longer sequence of a shape they take,
    segments of the most whole chunks one call takes, then the rest; None where they take no
    segment of the shape."""
    if _seq_supported(dtype, T, D, chunk, feature):
        return [T]
    tmax = SEQ_D128_MAX_T if D == 128 else SEQ_D64_MAX_T
    L = tmax - tmax % chunk if chunk >= 1 else 0
    if T <= tmax or L < 1 or not _seq_supported(dtype, L, D, chunk, feature):
        return None
    segs = [L] * (T // L)
    if T % L:
        if not _seq_supported(dtype, T % L, D, chunk, feature):
            return None
        segs.append(T % L)
    return segs


IMPLS = ("auto", "seq", "chunk", "cumsum")
IMPL_ENV = "LACHUNK_ATTN_IMPL"
_impl = None  # set by set_attention_impl; None: the environment variable, else "auto"


def _check_impl(name, where):
    if name not in IMPLS:
        raise ValueError(f"{where}: unknown attention implementation {name!r}; use one of {IMPLS}")
    return name


def set_attention_impl(name):
    """Set the implementation linear_attention uses when called without ``impl``: "auto",
    "seq", "chunk" or "cumsum"; None returns to the environment variable LACHUNK_ATTN_IMPL
    (else "auto")."""
    global _impl
    _impl = None if name is None else _check_impl(name, "set_attention_impl")


def get_attention_impl() -> str:
    """The implementation linear_attention uses when called without ``impl``."""
    if _impl is not None:
        return _impl
    return _check_impl(os.environ.get(IMPL_ENV, "auto"), IMPL_ENV)


def linear_attention(q, k, v, S_in=None, z_in=None, chunk: int = 128, block: int = 64, feature_map=None,
                     impl=None):
    """Causal linear attention over a (G, T, D) sequence in chunks of ``chunk`` tokens
    (the last one ragged), carrying (S, z) across chunks.  Returns (o, (S_out, z_out)).
    ``feature_map="elu1"``: q and k are raw inputs and elu(x) + 1 is applied inside the
    kernels (fused, on every path), gradients flowing to the raw inputs.  ``impl``: "auto",
    "seq", "chunk" or "cumsum" (None: get_attention_impl()); "seq" raises where the sequence
    entry points do not take the shape; "cumsum" runs the per-token form chunk by chunk."""
    name = get_attention_impl() if impl is None else _check_impl(impl, "linear_attention")
    _check_device(q)
    if q.dim() != 3:
        raise ValueError(f"q must be (G, T, D), got {tuple(q.shape)}")
    if chunk < 1:
        raise ValueError("chunk must be positive")
    T = q.shape[1]
    if T == 0:
        return q.new_empty(q.shape), (S_in, z_in)
    fm = _fm(feature_map)
    segs = seq_segments(q.dtype, T, q.shape[2], chunk, fm) if block == 64 else None
    if name == "seq" and segs is None:
        raise ValueError("impl='seq': the sequence entry points take bf16, block 64, and D = 64 in whole "
                         "128-token chunks or D = 128 in chunks of a multiple of 64 tokens")
    if segs is not None and name in ("seq", "auto"):
        outs = []
        S, z = S_in, z_in
        t0 = 0
        for L in segs:
            o, S, z = SeqFunction.apply(q[:, t0:t0 + L], k[:, t0:t0 + L], v[:, t0:t0 + L], S, z, chunk, block, fm)
            outs.append(o)
            t0 += L
        o = outs[0] if len(outs) == 1 else torch.cat(outs, dim=1)
        return o, (S, z)
    blk = 1 if name == "cumsum" else block
    outs = []
    S, z = S_in, z_in
    for t0 in range(0, T, chunk):
        t1 = min(T, t0 + chunk)
        o, S, z = ChunkFunction.apply(q[:, t0:t1], k[:, t0:t1], v[:, t0:t1], S, z, blk, fm)
        outs.append(o)
    o = outs[0] if len(outs) == 1 else torch.cat(outs, dim=1)
    return o, (S, z)


class CrossEntropyFunction(torch.autograd.Function):
    """Mean cross-entropy over a tied head; saves h, W, the targets and lse (the checkpoint) and
    recomputes the logits in the backward, ``ce_chunk`` tokens at a time."""

    @staticmethod
    def forward(ctx, h, W, targets, ce_chunk):
        from . import ce_fwd as _ce_fwd
        h, W = h.contiguous(), W.contiguous()
        loss, lse = _ce_fwd(h, W, targets)
        ctx.ce_chunk = ce_chunk
        ctx.save_for_backward(h, W, targets, lse)
        return loss

    @staticmethod
    def backward(ctx, g):
        from . import ce_bwd as _ce_bwd
        h, W, targets, lse = ctx.saved_tensors
        dh, dW = _ce_bwd(h, W, targets, lse, dloss=g.float().contiguous(), ce_chunk=ctx.ce_chunk)
        return dh, dW.to(W.dtype), None, None


def chunked_cross_entropy(h, W, targets, ce_chunk: int = 0):
    """The pages' chunked, checkpointed cross-entropy ("Fractus-1B training optimization",
    section 2, Opt 3): mean over the N tokens of h (N, d) of the loss of the tied head W (V, d)
    against int32 targets, differentiable in h and W; ``ce_chunk`` tokens per backward chunk
    (0: all).  bf16 h and W; the gradient of W is computed in fp32 and returned in W's dtype."""
    _check_device(h)
    return CrossEntropyFunction.apply(h, W, targets, ce_chunk)


def _fm(feature_map):
    if feature_map in (None, "none"):
        return None
    if feature_map != "elu1":
        raise ValueError(f"unknown feature map {feature_map!r}; use None or 'elu1'")
    return feature_map


def _check_device(q):
    if not q.is_cuda:
        raise ValueError("linear attention runs in the HIP library: inputs must be CUDA tensors")
