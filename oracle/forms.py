"""Independent numpy fp64 forms of the same attention, used to cross-check the C oracle.

TEST INFRASTRUCTURE ONLY (see the package docstring).

None of these calls the C oracle; each is written from a different statement
of the method on "Fractus-1B training optimization":

* :func:`masked_einsum_fwd` -- section 1, Bottleneck #1: materialise every
  outer product k_j v_j^T and sum them with a lower-triangular (inclusive)
  mask, O(C^2 D^2).  The page keeps this form as its ground truth.
* :func:`blocked_fwd` -- section 2, Opt 2: blocks of ``block`` tokens; a masked
  block-by-block score matrix for the block's own tokens plus a term against the
  running state, the running state updated after the block is read; a ragged
  tail (fewer than ``block`` tokens left) by the exact per-token cumsum.
* :func:`matrix_bwd` -- the backward of one chunk as whole-chunk matrix
  products (the blocked backward with a single block covering the chunk),
  derived from the definition; it takes no scan at all.
"""
from __future__ import annotations

import numpy as np


def _zeros_carry(G, D, S_in, z_in):
    if S_in is None:
        return np.zeros((G, D, D)), np.zeros((G, D))
    return np.asarray(S_in, np.float64), np.asarray(z_in, np.float64)


def masked_einsum_fwd(q, k, v, S_in=None, z_in=None):
    """Section 1, Bottleneck #1: S_t = S_in + sum_j M[t, j] k_j v_j^T with M inclusive lower-triangular."""
    q, k, v = (np.asarray(a, np.float64) for a in (q, k, v))
    G, T, D = q.shape
    S0, z0 = _zeros_carry(G, D, S_in, z_in)
    mask = np.tril(np.ones((T, T)))                      # M[t, j] = 1 iff j <= t
    outer = np.einsum("gjp,gjc->gjpc", k, v)              # (G, T, D, D)
    S = S0[:, None] + np.einsum("tj,gjpc->gtpc", mask, outer)
    z = z0[:, None] + np.einsum("tj,gjp->gtp", mask, k)
    num = np.einsum("gtp,gtpc->gtc", q, S)
    den = np.einsum("gtp,gtp->gt", q, z)
    return num / den[..., None], S[:, -1] if T else S0, z[:, -1] if T else z0


def blocked_fwd(q, k, v, S_in=None, z_in=None, block=64):
    """Section 2, Opt 2: chunked form with a running state read before its update; ragged tail by cumsum."""
    q, k, v = (np.asarray(a, np.float64) for a in (q, k, v))
    G, T, D = q.shape
    S_run, z_run = (a.copy() for a in _zeros_carry(G, D, S_in, z_in))
    o = np.empty((G, T, D))
    nfull = T // block
    mask = np.tril(np.ones((block, block)))
    for b in range(nfull):
        sl = slice(b * block, (b + 1) * block)
        Qb, Kb, Vb = q[:, sl], k[:, sl], v[:, sl]
        A = (Qb @ Kb.transpose(0, 2, 1)) * mask          # intra-block masked scores
        num = A @ Vb + Qb @ S_run                         # + inter-block term (state before this block)
        den = A.sum(axis=2) + np.einsum("gtp,gp->gt", Qb, z_run)
        o[:, sl] = num / den[..., None]
        S_run = S_run + Kb.transpose(0, 2, 1) @ Vb        # update after reading
        z_run = z_run + Kb.sum(axis=1)
    for t in range(nfull * block, T):                     # ragged tail: exact per-token cumsum
        S_run = S_run + np.einsum("gp,gc->gpc", k[:, t], v[:, t])
        z_run = z_run + k[:, t]
        num = np.einsum("gp,gpc->gc", q[:, t], S_run)
        den = np.einsum("gp,gp->g", q[:, t], z_run)
        o[:, t] = num / den[:, None]
    return o, S_run, z_run


def matrix_bwd(q, k, v, S_in, z_in, dO, dS_out=None, dz_out=None):
    """Backward of one chunk by whole-chunk matrix products.

    With A = (Q K^T) masked inclusively, num = A V + Q S_in, den = A 1 + Q z_in and
    O = num / den (row-wise), the loss L = <dO, O> + <dS_out, S_out> + dz_out . z_out
    has, writing dN = dO / den and dden = -rowsum(dO * O) / den,
        dP    = (dN V^T + dden 1^T) masked
        dQ    = dP K + dN S_in^T + dden z_in^T
        dK    = dP^T Q + V dS_out^T + 1 dz_out^T
        dV    = A^T dN + K dS_out
        dS_in = dS_out + Q^T dN,     dz_in = dz_out + Q^T dden.
    """
    q, k, v, dO = (np.asarray(a, np.float64) for a in (q, k, v, dO))
    G, T, D = q.shape
    S0, z0 = _zeros_carry(G, D, S_in, z_in)
    if dS_out is None:
        dS_out, dz_out = np.zeros((G, D, D)), np.zeros((G, D))
    dS_out, dz_out = np.asarray(dS_out, np.float64), np.asarray(dz_out, np.float64)
    mask = np.tril(np.ones((T, T)))
    Kt = k.transpose(0, 2, 1)
    A = (q @ Kt) * mask
    num = A @ v + q @ S0
    den = A.sum(axis=2) + np.einsum("gtp,gp->gt", q, z0)
    O = num / den[..., None]
    dN = dO / den[..., None]
    dden = -(dO * O).sum(axis=2) / den
    dP = (dN @ v.transpose(0, 2, 1) + dden[..., None]) * mask
    dq = dP @ k + dN @ S0.transpose(0, 2, 1) + dden[..., None] * z0[:, None, :]
    dk = dP.transpose(0, 2, 1) @ q + v @ dS_out.transpose(0, 2, 1) + dz_out[:, None, :]
    dv = A.transpose(0, 2, 1) @ dN + k @ dS_out
    dS_in = dS_out + q.transpose(0, 2, 1) @ dN
    dz_in = dz_out + np.einsum("gtp,gt->gp", q, dden)
    return dq, dk, dv, dS_in, dz_in
