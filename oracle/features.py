"""Positive feature map phi(x) = elu(x) + 1 (alpha = 1) in front of the op, in fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

"Fractus-1B training optimization", section 1, Bottleneck #1, needs positive queries and keys,
so that every denominator q_t . z_t is positive; the workloads get them as elu(x) + 1 of normal
draws.  With the map fused into the op, the op takes the raw x for queries and keys and its
gradients are with respect to x.  The features enter the op at its element type, as they do
when the caller maps and stores them itself (bf16 features in the bf16 workloads), so the
fused op is the plain op on phi(x) rounded to that type, and the gradient passes straight
through the rounding.  By the chain rule, with phi'(x) = 1 for x > 0 and e^x otherwise (elu
with alpha = 1 is e^x - 1 below zero):
    forward:  the plain op on (round(phi(x_q)), round(phi(x_k)), v, carry);
    backward: dx_q = dq * phi'(x_q), dx_k = dk * phi'(x_k); dv and the carry gradients unchanged.
``dtype=None`` skips the rounding (the exact composition, for finite differences).
"""
from __future__ import annotations

import numpy as np

from . import core


def _f64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):
        import torch
        return x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def elu1(x):
    """phi(x) = x + 1 for x > 0, e^x otherwise."""
    x = _f64(x)
    return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def elu1_grad(x):
    """phi'(x) = 1 for x > 0, e^x otherwise."""
    x = _f64(x)
    return np.where(x > 0, 1.0, np.exp(np.minimum(x, 0.0)))


def mapped(x, dtype=None):
    """phi(x), rounded to nearest even in the element type ("bf16" or "f32") when one is given."""
    y = elu1(x)
    if dtype is None:
        return y
    import torch
    t = {"bf16": torch.bfloat16, "f32": torch.float32}[dtype]
    return torch.from_numpy(y).to(t).double().numpy()


def fwd(xq, xk, v, S_in=None, z_in=None, dtype=None, nthreads: int = 0):
    """The op on the mapped features: (o, S_out, z_out)."""
    return core.fwd(mapped(xq, dtype), mapped(xk, dtype), v, S_in, z_in, nthreads=nthreads)


def bwd(xq, xk, v, S_in, z_in, dO, dS_out=None, dz_out=None, dtype=None, nthreads: int = 0):
    """Gradients with respect to the raw inputs: (dx_q, dx_k, dv, dS_in, dz_in)."""
    dq, dk, dv, dS, dz = core.bwd(mapped(xq, dtype), mapped(xk, dtype), v, S_in, z_in, dO, dS_out, dz_out,
                                  nthreads=nthreads)
    return dq * elu1_grad(xq), dk * elu1_grad(xk), dv, dS, dz
