"""Pins of the cross-entropy oracle (oracle/ce.py) to mathematics, not to itself.

"Fractus-1B training optimization", section 1, Bottleneck #3 (the tied head's loss) and section 2,
Opt 3 (its chunked, checkpointed form: the same mean loss and gradients).  Which pin catches what:
  C1  zero head: every logit 0, the loss is log V, dh = 0 and dW in closed form (catches a wrong
      normaliser, a dropped one-hot term, a wrong 1/N);
  C2  two classes: the loss is the logistic loss of the logit difference (catches a wrong sign or
      a target taken from the wrong row);
  C3  the columns of dW sum to zero: softmax is unchanged when one vector is added to every row of
      W (catches a dropped one-hot or softmax term);
  C4  sum_i h_i . dh_i = sum_v W_v . dW_v: both are (g/N) sum (p - y) logit (catches a transposed
      product or a misplaced scale);
  C5  central finite differences on tiny shapes, fp64;
  C6  the library routine: torch's cross_entropy in float64 on the CPU, loss and autograd
      gradients, with an upstream gradient;
  C7  the chunked form (any chunk length, ragged last chunk) equals the definition.
"""
import numpy as np
import pytest
import torch

from oracle import ce
from causal_linear_attention_chunked_amd import inputs


def rand(N, d, V, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((N, d)), rng.standard_normal((V, d)) * scale, rng.integers(0, V, N))


def test_c1_zero_head():
    N, d, V = 6, 5, 7
    h, _, t = rand(N, d, V, 1)
    W = np.zeros((V, d))
    loss, lse = ce.forward(h, W, t)
    assert loss == pytest.approx(np.log(V), rel=1e-14)
    assert np.allclose(lse, np.log(V), rtol=1e-14)
    dh, dW = ce.backward(h, W, t, dloss=2.5)
    assert np.all(dh == 0.0)
    y = np.zeros((N, V))
    y[np.arange(N), t] = 1.0
    assert np.allclose(dW, (2.5 / N) * (1.0 / V - y).T @ h, rtol=1e-13, atol=1e-15)


def test_c2_two_classes_is_the_logistic_loss():
    N, d = 9, 4
    h, W, t = rand(N, d, 2, 2)
    loss, _ = ce.forward(h, W, t)
    logits = h @ W.T
    diff = logits[np.arange(N), 1 - t] - logits[np.arange(N), t]
    assert loss == pytest.approx(float(np.mean(np.log1p(np.exp(diff)))), rel=1e-13)


def test_c3_dW_columns_sum_to_zero():
    h, W, t = rand(7, 6, 11, 3)
    dh, dW = ce.backward(h, W, t)
    scale = np.abs(dW).max()
    assert np.abs(dW.sum(axis=0)).max() < 1e-13 * scale * 11


def test_c4_bilinear_identity():
    h, W, t = rand(8, 5, 13, 4)
    dh, dW = ce.backward(h, W, t, dloss=0.7)
    a, b = float(np.sum(h * dh)), float(np.sum(W * dW))
    assert a == pytest.approx(b, rel=1e-12)


def test_c5_finite_differences():
    N, d, V = 3, 4, 5
    h, W, t = rand(N, d, V, 5)
    dh, dW = ce.backward(h, W, t)
    eps = 1e-6
    for x, g in ((h, dh), (W, dW)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + eps
            lp, _ = ce.forward(h, W, t)
            x[idx] = old - eps
            lm, _ = ce.forward(h, W, t)
            x[idx] = old
            num[idx] = (lp - lm) / (2 * eps)
        assert np.allclose(num, g, rtol=1e-6, atol=1e-9)


def test_c6_matches_torch_cross_entropy_float64():
    N, d, V = 10, 8, 17
    h, W, t = rand(N, d, V, 6, scale=0.5)
    ht = torch.tensor(h, requires_grad=True)
    Wt = torch.tensor(W, requires_grad=True)
    loss = torch.nn.functional.cross_entropy(ht @ Wt.T, torch.tensor(t))
    (3.0 * loss).backward()
    l, _ = ce.forward(h, W, t)
    dh, dW = ce.backward(h, W, t, dloss=3.0)
    assert l == pytest.approx(float(loss.detach()), rel=1e-13)
    assert np.allclose(dh, ht.grad.numpy(), rtol=1e-12, atol=1e-15)
    assert np.allclose(dW, Wt.grad.numpy(), rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("chunk", [1, 3, 7, 16])
def test_c7_chunked_form_equals_definition(chunk):
    h, W, t = rand(16, 6, 9, 7)
    l0, lse0 = ce.forward(h, W, t)
    l1, lse1 = ce.chunked_forward(h, W, t, chunk)
    assert l1 == pytest.approx(l0, rel=1e-13)
    assert np.allclose(lse1, lse0, rtol=1e-14)
    dh0, dW0 = ce.backward(h, W, t, 1.3)
    dh1, dW1 = ce.chunked_backward(h, W, t, chunk, 1.3)
    assert np.allclose(dh1, dh0, rtol=1e-12, atol=1e-16)
    assert np.allclose(dW1, dW0, rtol=1e-12, atol=1e-16)


def test_ce_inputs_deterministic_and_in_range():
    a = inputs.make_ce_inputs(8, 16, 11, seed=3)
    b = inputs.make_ce_inputs(8, 16, 11, seed=3)
    for k in a:
        assert torch.equal(a[k], b[k])
    assert int(a["targets"].min()) >= 0 and int(a["targets"].max()) < 11
    assert a["h"].dtype == torch.bfloat16 and a["targets"].dtype == torch.int32
    w = inputs.ce_workload("ce_n512_d1280_v50257_bf16")
    assert (w.N, w.d, w.V) == (512, 1280, 50257)
    # the page's fp32 logits at B = 4: about 103 MB
    assert w.N * w.V * 4 == pytest.approx(103e6, rel=0.01)
