"""GPU parity of the cross-entropy over a tied head (la_ce_fwd / la_ce_bwd through the binding)
against the fp64 oracle (oracle/ce.py).

Tolerances: the loss and lse come from fp32 sums of exact bf16 products and an fp32 log-sum-exp,
held to 1e-5 relative; dh (bf16 output) and dW (fp32 output, from the softmax rounded once to
bf16 as an MFMA operand) to the bf16 rule of tests/tol.py.
"""
import numpy as np
import pytest
import torch

import causal_linear_attention_chunked_amd as lac
from causal_linear_attention_chunked_amd import inputs as inp
from oracle import ce
from tol import RTOL, check

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def run(I, dloss=None, ce_chunk=0):
    h, W, t = (I[n].to("cuda:0").contiguous() for n in ("h", "W", "targets"))
    loss, lse = lac.ce_fwd(h, W, t)
    g = None if dloss is None else torch.tensor(dloss, dtype=torch.float32, device="cuda:0")
    dh, dW = lac.ce_bwd(h, W, t, lse, dloss=g, ce_chunk=ce_chunk)
    torch.cuda.synchronize()
    return float(loss), lse, dh, dW


def compare(I, res, dloss=1.0, label=""):
    loss, lse, dh, dW = res
    rl, rlse = ce.forward(I["h"], I["W"], I["targets"])
    rdh, rdW = ce.backward(I["h"], I["W"], I["targets"], dloss)
    say(f"  {label}loss {loss:.7f} ref {rl:.7f}")
    assert abs(loss - rl) <= 1e-5 * abs(rl)
    g = lse.double().cpu().numpy()
    assert np.max(np.abs(g - rlse) / np.abs(rlse)) < 1e-5
    for name, x, r in (("dh", dh, rdh), ("dW", dW, rdW)):
        nw = check(f"{label}{name}", x, r, RTOL["bf16"])
        say(f"  {label}{name}: normwise rel err {nw:.2e}")


@pytest.mark.parametrize("N,d,V,chunk,dloss", [
    (5, 128, 300, 0, None),       # every tile ragged
    (128, 128, 128, 0, 2.0),      # exactly one tile each way
    (130, 256, 1000, 64, 0.5),    # three backward chunks, the last of 2 tokens
    (1, 128, 2, 0, None),         # one token, two classes
    (300, 384, 5003, 128, -1.5),  # several tiles, a negative upstream gradient
])
def test_ce_against_oracle(gpu, N, d, V, chunk, dloss):
    say(f"[case] ce N={N} d={d} V={V} chunk={chunk} dloss={dloss}")
    I = inp.make_ce_inputs(N, d, V, seed=N + V)
    compare(I, run(I, dloss, chunk), 1.0 if dloss is None else dloss)


def test_ce_head_workload_full_size(gpu):
    w = inp.ce_workload("ce_n512_d1280_v50257_bf16")
    say(f"[case] ce full {w.name}")
    I = inp.ce_workload_inputs(w)
    compare(I, run(I))


def test_ce_persistent_walk_masked_features(gpu):
    # d = 640 (an odd multiple of 128: the last 256-feature tile half masked) over the full
    # vocabulary: several tiles per workgroup in the forward, dW and dh kernels, two backward
    # chunks of 128 tokens
    N, d, V = 256, 640, 50257
    say(f"[case] ce N={N} d={d} V={V} chunk=128 (persistent walk, masked feature tiles)")
    I = inp.make_ce_inputs(N, d, V, seed=17)
    compare(I, run(I, 0.75, 128), 0.75)


def test_ce_chunked_backward_matches_whole(gpu):
    # the pages' chunked form: the same gradients whatever the chunk (to the summation order)
    w = inp.ce_workload("ce_n512_d1280_v50257_bf16")
    say(f"[case] ce chunked backward {w.name}, chunks of 128 and 200 tokens")
    I = inp.ce_workload_inputs(w)
    _, _, dh0, dW0 = run(I)
    for chunk in (128, 200):
        _, _, dh1, dW1 = run(I, ce_chunk=chunk)
        for name, a, b in (("dh", dh1, dh0), ("dW", dW1, dW0)):
            rel = float((a.double() - b.double()).norm() / b.double().norm())
            say(f"  chunk {chunk} {name}: vs whole normwise {rel:.2e}")
            assert rel < 1e-3, (chunk, name, rel)


def test_ce_zero_head_closed_form(gpu):
    # W = 0: every logit is 0, the loss is log V, dh = 0 and dW = (1/N) (1/V - onehot)^T h
    N, d, V = 70, 128, 1000
    I = inp.make_ce_inputs(N, d, V, seed=3)
    I["W"] = torch.zeros_like(I["W"])
    loss, lse, dh, dW = run(I)
    assert abs(loss - np.log(V)) < 1e-5 * np.log(V)
    assert float(dh.abs().max()) == 0.0
    rdh, rdW = ce.backward(I["h"], I["W"], I["targets"])
    check("dW", dW, rdW, RTOL["bf16"])


def test_ce_autograd(gpu):
    N, d, V = 96, 256, 3001
    say(f"[case] ce autograd N={N} d={d} V={V}")
    I = inp.make_ce_inputs(N, d, V, seed=11)
    h = I["h"].to("cuda:0").requires_grad_(True)
    W = I["W"].to("cuda:0").requires_grad_(True)
    t = I["targets"].to("cuda:0")
    loss = lac.chunked_cross_entropy(h, W, t, ce_chunk=64)
    (2.5 * loss).backward()
    torch.cuda.synchronize()
    rl, _ = ce.forward(I["h"], I["W"], I["targets"])
    rdh, rdW = ce.backward(I["h"], I["W"], I["targets"], 2.5)
    assert abs(float(loss) - rl) <= 1e-5 * abs(rl)
    check("dh", h.grad, rdh, RTOL["bf16"])
    check("dW", W.grad, rdW, RTOL["bf16"])


def test_ce_rejects(gpu):
    h = torch.zeros(4, 100, dtype=torch.bfloat16, device="cuda:0")
    W = torch.zeros(10, 100, dtype=torch.bfloat16, device="cuda:0")
    t = torch.zeros(4, dtype=torch.int32, device="cuda:0")
    with pytest.raises(lac.LachunkError, match="UNSUPPORTED"):
        lac.ce_fwd(h, W, t)
    with pytest.raises(ValueError):
        lac.ce_fwd(h.float(), W.float(), t)
