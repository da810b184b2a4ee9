"""Autograd wrapper: chunked causal linear attention as a differentiable PyTorch op.

The call site the Fractus page describes ("Fractus-1B training optimization",
section 2, Opt 2) runs attention chunk by chunk and carries the state (S, z)
from one chunk to the next.  This module gives that op a backward:

    o, (S_out, z_out) = linear_attention(q, k, v, S_in=None, z_in=None, chunk=128)

q, k, v are (G, T, D) CUDA tensors (bf16 or fp32; q and k already positive, e.g.
elu(x) + 1); S_in (G, D, D) and z_in (G, D) are fp32 or None for a zero carry.
Every chunk is one forward launch; its backward is one backward launch that
recomputes the chunk from its saved inputs (q, k, v and the carry that fed it),
so nothing of size (G, C, D, D) or (G, C, C) is kept between the passes, the
memory-flat principle of the page's section 1.  Gradients flow to q, k, v and,
when given, S_in and z_in; a loss on S_out / z_out reaches them too.

The arithmetic runs in the HIP library only: CPU tensors raise.
"""
from __future__ import annotations

import torch

from . import bwd as _bwd
from . import fwd as _fwd


class ChunkFunction(torch.autograd.Function):
    """One chunk: (q, k, v, S_in, z_in) -> (o, S_out, z_out), backward by recomputation."""

    @staticmethod
    def forward(ctx, q, k, v, S_in, z_in, block):
        q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
        o, S_out, z_out = _fwd(q, k, v, S_in, z_in, block)
        ctx.block = block
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
                                        ctx.block)
        if not ctx.has_carry:
            dS_in = dz_in = None
        return dq, dk, dv, dS_in, dz_in, None


def chunk_attention(q, k, v, S_in=None, z_in=None, block: int = 64):
    """Differentiable single-chunk op: returns (o, S_out, z_out)."""
    _check_device(q)
    return ChunkFunction.apply(q, k, v, S_in, z_in, block)


def linear_attention(q, k, v, S_in=None, z_in=None, chunk: int = 128, block: int = 64):
    """Causal linear attention over a (G, T, D) sequence in chunks of ``chunk`` tokens
    (the last one ragged), carrying (S, z) across chunks.  Returns (o, (S_out, z_out))."""
    _check_device(q)
    if q.dim() != 3:
        raise ValueError(f"q must be (G, T, D), got {tuple(q.shape)}")
    if chunk < 1:
        raise ValueError("chunk must be positive")
    T = q.shape[1]
    if T == 0:
        return q.new_empty(q.shape), (S_in, z_in)
    outs = []
    S, z = S_in, z_in
    for t0 in range(0, T, chunk):
        t1 = min(T, t0 + chunk)
        o, S, z = ChunkFunction.apply(q[:, t0:t1], k[:, t0:t1], v[:, t0:t1], S, z, block)
        outs.append(o)
    o = outs[0] if len(outs) == 1 else torch.cat(outs, dim=1)
    return o, (S, z)


def _check_device(q):
    if not q.is_cuda:
        raise ValueError("linear attention runs in the HIP library: inputs must be CUDA tensors")
