"""Cross-entropy over a tied output head, in fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

"Fractus-1B training optimization", section 1, Bottleneck #3: the head ties the 50257-token
embedding W (V x d) to the output, so every token's logits are h_i W^T (a (tokens, V) matrix
that the plain loss materialises, together with its softmax backward).  Section 2, Opt 3,
replaces it with a chunked, checkpointed cross-entropy: the same mean loss and the same
gradients (up to the summation order of fp32), computed over one chunk of tokens at a time,
the chunk's logits recomputed in the backward instead of kept.

The loss is the mean over the N tokens of the negative log-likelihood of the target class:
    logit_iv = h_i . W_v,   lse_i = log sum_v exp(logit_iv),   loss = (1/N) sum_i (lse_i - logit_{i,t_i})
and, for an upstream gradient g of the loss, with p_iv = exp(logit_iv - lse_i) and y the one-hot
targets,
    dh_i = (g/N) sum_v (p_iv - y_iv) W_v,   dW_v = (g/N) sum_i (p_iv - y_iv) h_i.

Inputs are the stored values (bf16 or fp32), upcast exactly to fp64; everything is computed in
fp64.  :func:`forward` / :func:`backward` are the definition written out with whole-matrix
products; :func:`chunked_forward` / :func:`chunked_backward` follow the pages' chunked form,
``ce_chunk`` tokens at a time, each chunk's logits formed afresh in the backward.
"""
from __future__ import annotations

import numpy as np


def _f64(x):
    if hasattr(x, "detach"):
        import torch
        return x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def _targets(t):
    if hasattr(t, "detach"):
        t = t.detach().to("cpu").numpy()
    return np.asarray(t, dtype=np.int64)


def _lse(logits):
    """Row-wise log sum exp, shifted by the row maximum (exact in fp64 up to rounding)."""
    m = logits.max(axis=1, keepdims=True)
    return (m + np.log(np.exp(logits - m).sum(axis=1, keepdims=True)))[:, 0]


def forward(h, W, targets):
    """Bottleneck #3's loss by its definition: returns (loss, lse) with lse of shape (N,)."""
    h, W, t = _f64(h), _f64(W), _targets(targets)
    logits = h @ W.T
    lse = _lse(logits)
    nll = lse - logits[np.arange(len(t)), t]
    return float(nll.mean()), lse


def backward(h, W, targets, dloss=1.0):
    """Gradients of g * loss with respect to h and W, g = ``dloss``: returns (dh, dW)."""
    h, W, t = _f64(h), _f64(W), _targets(targets)
    N = h.shape[0]
    logits = h @ W.T
    p = np.exp(logits - _lse(logits)[:, None])
    p[np.arange(N), t] -= 1.0
    p *= float(dloss) / N
    return p @ W, p.T @ h


def chunked_forward(h, W, targets, ce_chunk):
    """Opt 3's chunked form: the tokens in chunks of ``ce_chunk``, one chunk's logits at a time;
    the per-token losses are summed over the chunks and divided by N at the end."""
    h, W, t = _f64(h), _f64(W), _targets(targets)
    N = h.shape[0]
    total, lse = 0.0, np.empty(N)
    for a in range(0, N, ce_chunk):
        b = min(N, a + ce_chunk)
        logits = h[a:b] @ W.T
        lse[a:b] = _lse(logits)
        total += float((lse[a:b] - logits[np.arange(b - a), t[a:b]]).sum())
    return total / N, lse


def chunked_backward(h, W, targets, ce_chunk, dloss=1.0):
    """The backward of the chunked form: each chunk's logits recomputed (the checkpoint), its
    softmax minus one-hot scaled by g/N, and the chunk's contributions to dh (its own rows) and
    dW (summed over the chunks)."""
    h, W, t = _f64(h), _f64(W), _targets(targets)
    N = h.shape[0]
    dh, dW = np.empty_like(h), np.zeros_like(W)
    for a in range(0, N, ce_chunk):
        b = min(N, a + ce_chunk)
        logits = h[a:b] @ W.T
        p = np.exp(logits - _lse(logits)[:, None])
        p[np.arange(b - a), t[a:b]] -= 1.0
        p *= float(dloss) / N
        dh[a:b] = p @ W
        dW += p.T @ h[a:b]
    return dh, dW
