"""GPU: the autograd layer (torch.autograd.Function over the HIP library) against the fp64 oracle.

A scalar loss L = sum(o * dO) + <S_out, dS_out> + z_out . dz_out is back-propagated through a
chunked sequence (ragged last chunk); the gradients of q, k, v, S_in, z_in must match the
oracle's reverse scan for the same (dO, dS_out, dz_out), to the tolerance of tests/tol.py.
"""
import numpy as np
import pytest
import torch

import causal_linear_attention_chunked_amd as lac
from causal_linear_attention_chunked_amd import inputs as inp
import oracle
from tol import RTOL, check

pytestmark = pytest.mark.gpu


def _case(dtype, carry, upstream, G=3, T=300, D=64, chunk=128, seed=11, feature_map=None, impl=None):
    I = inp.make_inputs(G=G, T=T, D=D, dtype=dtype, carry=carry, backward=True, seed=seed,
                        features="raw" if feature_map else "mapped")
    rng = np.random.default_rng(seed + 1)
    dS = torch.from_numpy(rng.standard_normal((G, D, D)).astype(np.float32)) if upstream else None
    dz = torch.from_numpy(rng.standard_normal((G, D)).astype(np.float32)) if upstream else None
    print(f"[case] autograd dtype={dtype} carry={carry} upstream={upstream} G={G} T={T} D={D} chunk={chunk} "
          f"feature_map={feature_map} impl={impl}", flush=True)
    dev = "cuda:0"
    leaf = lambda x: None if x is None else x.to(dev).clone().requires_grad_(True)
    q, k, v = leaf(I["q"]), leaf(I["k"]), leaf(I["v"])
    S_in, z_in = leaf(I["S_in"]), leaf(I["z_in"])
    o, (S_out, z_out) = lac.linear_attention(q, k, v, S_in, z_in, chunk=chunk, feature_map=feature_map, impl=impl)
    loss = (o.float() * I["dO"].to(dev).float()).sum()
    if upstream:
        loss = loss + (S_out * dS.to(dev)).sum() + (z_out * dz.to(dev)).sum()
    loss.backward()
    torch.cuda.synchronize()
    if feature_map == "elu1":
        # the features enter the op at its element type
        ro, rS, rz = oracle.features.fwd(I["q"], I["k"], I["v"], I["S_in"], I["z_in"], dtype=dtype)
        ref = oracle.features.bwd(I["q"], I["k"], I["v"], I["S_in"], I["z_in"], I["dO"], dS, dz, dtype=dtype)
    else:
        ro, rS, rz = oracle.fwd(I["q"], I["k"], I["v"], I["S_in"], I["z_in"])
        ref = oracle.bwd(I["q"], I["k"], I["v"], I["S_in"], I["z_in"], I["dO"], dS, dz)
    tol = RTOL[dtype]
    check("o", o, ro, tol)
    check("S_out", S_out, rS, tol)
    check("z_out", z_out, rz, tol)
    for name, g, r in zip(("dq", "dk", "dv"), (q.grad, k.grad, v.grad), ref[:3]):
        check(name, g, r, tol)
    if carry == "zero":
        assert S_in is None
    else:
        check("dS_in", S_in.grad, ref[3], tol)
        check("dz_in", z_in.grad, ref[4], tol)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_autograd_prior_carry_upstream(gpu, dtype):
    _case(dtype, "prior", True)


def test_autograd_zero_carry_no_upstream(gpu):
    _case("bf16", "zero", False, G=2, T=128)


def test_autograd_wide_heads(gpu):
    _case("bf16", "prior", True, G=2, T=200, D=128, chunk=100)


def test_autograd_sequence_entry_points(gpu):
    # bf16, D = 64, whole 128-token chunks: one launch per direction through the sequence path
    assert lac.seq_supported("bf16", 512, 64, 128)
    _case("bf16", "prior", True, G=3, T=512)
    _case("bf16", "zero", False, G=2, T=384)


def test_autograd_sequence_entry_points_wide_heads(gpu):
    # bf16, D = 128, 128-token chunks and a ragged end: the sequence path
    assert lac.seq_supported("bf16", 300, 128, 128)
    _case("bf16", "prior", True, G=2, T=300, D=128)


def test_autograd_sequence_longer_than_one_call(gpu):
    # D = 128 past the sequence calls' length: two segments (the longest one call takes, then 300
    # tokens with a ragged end), the carry passed from the first to the second, the gradients back
    from causal_linear_attention_chunked_amd import autograd as ag
    T = lac.SEQ_D128_MAX_T + 300
    assert ag.seq_segments(torch.bfloat16, T, 128, 128) == [lac.SEQ_D128_MAX_T, 300]
    _case("bf16", "prior", True, G=1, T=T, D=128, seed=23)


def test_autograd_fused_feature_map(gpu):
    _case("bf16", "prior", True, G=3, T=384, feature_map="elu1")


def test_autograd_fused_feature_map_wide_heads(gpu):
    # D = 128 with a ragged end: the mapped rows past the end must stay out of z
    _case("bf16", "zero", True, G=2, T=230, D=128, feature_map="elu1")


@pytest.mark.parametrize("dtype,D", [("bf16", 64), ("f32", 64), ("f32", 128)])
def test_autograd_cumsum_impl(gpu, dtype, D):
    # the per-token form chunk by chunk (block 1 in the chunk calls), ragged last chunk
    _case(dtype, "prior", True, G=2, T=200, D=D, chunk=128, impl="cumsum")


def test_autograd_fused_map_chunk_impl(gpu):
    # the map on the chunk path: a ragged D = 64 sequence (the sequence calls take whole chunks only)
    _case("bf16", "prior", True, G=3, T=300, feature_map="elu1", impl="chunk")
    _case("bf16", "zero", False, G=2, T=256, feature_map="elu1", impl="chunk")


def test_autograd_fused_map_cumsum_impl(gpu):
    _case("f32", "prior", True, G=2, T=150, D=128, chunk=64, feature_map="elu1", impl="cumsum")


def _grads(I, dO, impl, D):
    dev = "cuda:0"
    leaf = lambda x: x.to(dev).clone().requires_grad_(True)
    q, k, v, S_in, z_in = (leaf(I[n]) for n in ("q", "k", "v", "S_in", "z_in"))
    o, (S_out, z_out) = lac.linear_attention(q, k, v, S_in, z_in, chunk=128, impl=impl)
    loss = (o.float() * dO).sum() + S_out.sum() + z_out.sum()
    loss.backward()
    torch.cuda.synchronize()
    return dict(o=o, S_out=S_out, z_out=z_out, dq=q.grad, dk=k.grad, dv=v.grad, dS_in=S_in.grad, dz_in=z_in.grad)


@pytest.mark.parametrize("T,D", [(384, 64), (300, 128)])
def test_autograd_impls_agree(gpu, T, D):
    # impl="seq" (one launch per direction) and impl="chunk" (one per chunk and direction, the carry
    # through memory) compute the same op: to fp32 rounding (the sequence path keeps compensation
    # terms across chunks and takes a ragged end as a masked block)
    G = 2
    print(f"[case] autograd impls seq vs chunk G={G} T={T} D={D}", flush=True)
    I = inp.make_inputs(G=G, T=T, D=D, dtype="bf16", carry="prior", backward=True, seed=90 + D)
    dO = I["dO"].to("cuda:0").float()
    a, b, c = _grads(I, dO, "seq", D), _grads(I, dO, "chunk", D), _grads(I, dO, "cumsum", D)
    for name in a:
        x, y, u = a[name].double(), b[name].double(), c[name].double()
        rel, relc = float((x - y).norm() / y.norm()), float((u - y).norm() / y.norm())
        print(f"  {name}: seq vs chunk normwise {rel:.2e}, cumsum vs chunk {relc:.2e}", flush=True)
        assert rel < 2e-3 and relc < 2e-3, (name, rel, relc)
    lac.set_attention_impl("chunk")
    try:
        c = _grads(I, dO, None, D)  # the default from the setter
    finally:
        lac.set_attention_impl(None)
    for name in c:
        assert torch.equal(c[name], b[name]), name


def test_autograd_impl_seq_rejects_unsupported(gpu):
    q = torch.ones(2, 200, 64, dtype=torch.float32, device="cuda:0")
    with pytest.raises(ValueError, match="impl='seq'"):
        lac.linear_attention(q, q, q, impl="seq")
    x = torch.ones(2, 256, 64, dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(ValueError, match="unknown feature map"):
        lac.linear_attention(x, x, x, feature_map="relu", impl="chunk")
