"""Pins of the fp64 CPU oracle against facts other than itself.

The oracle (oracle/la_oracle.c) is the per-token recurrence and reverse scan of
"Fractus-1B training optimization", section 1 (Bottleneck #1 and its note that
the backward of a cumsum is a reverse cumsum).  Each test below pins part of it
to something independent of that code:

  golden   exact rational values (tests/golden/tiny_exact.json)        -> all outputs
  P1       zero carry: o_1 = v_1 exactly (inclusive mask)               -> forward, token 1
  P2       constant v = c: o_t = c (also with carry S_in = z_in c^T)    -> num/den pairing
  P3       constant k, zero carry: o_t = prefix mean of v               -> mask + normaliser
  P4       D = 1: weighted prefix mean, independent of q; dq = 0        -> brute force
  P5       q_t . dq_t = 0 (o_t is scale-free in q_t)                     -> dq
  P6       Euler identity in (k, S_in, z_in)                            -> dk, dS_in, dz_in
  P7       Euler identity in (v, S_in)                                  -> dv, dS_in
  P8       S_out = S_in + K^T V, z_out = z_in + K^T 1 (library matmul)   -> final state
  P9       dS_in - dS_out = Q^T dN, dz_in - dz_out = Q^T dden            -> carry gradients
  P10      chunk split with carried state == one call (values, grads)   -> carry in/out
  P11      blocked form (section 2, Opt 2) at any block size == oracle  -> block decomposition
  P12      masked-einsum form (section 1) == oracle                     -> the oracle itself
  P13      central finite differences (fp64)                            -> all gradients
  matrix   whole-chunk matrix backward == reverse scan                  -> all gradients
  F1       phi = elu + 1 at closed-form points; continuous at 0        -> oracle.features.elu1
  F2       phi' against central differences of phi                     -> oracle.features.elu1_grad
  F3       fused-map gradients against central differences of the
           loss in the raw inputs (both signs of x)                    -> oracle.features.bwd
  F4       rounding of the mapped features: round to nearest even at
           bf16 halfway points; the rounded op is the plain op on them -> oracle.features.mapped
"""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import forms
from causal_linear_attention_chunked_amd import inputs

HERE = os.path.dirname(os.path.abspath(__file__))


def rng_inputs(G, T, D, seed, carry=True, upstream=True):
    r = np.random.default_rng(seed)
    q = np.exp(r.normal(size=(G, T, D)) * 0.5)          # strictly positive features
    k = np.exp(r.normal(size=(G, T, D)) * 0.5)
    v = r.normal(size=(G, T, D))
    dO = r.normal(size=(G, T, D))
    if carry:
        kp = np.exp(r.normal(size=(G, 7, D)) * 0.5)
        vp = r.normal(size=(G, 7, D))
        S_in = kp.transpose(0, 2, 1) @ vp
        z_in = kp.sum(axis=1)
    else:
        S_in = z_in = None
    if upstream:
        dS_out = r.normal(size=(G, D, D))
        dz_out = r.normal(size=(G, D))
    else:
        dS_out = dz_out = None
    return q, k, v, S_in, z_in, dO, dS_out, dz_out


def close(a, b, rtol=1e-11, atol=1e-11):
    np.testing.assert_allclose(a, b, rtol=rtol, atol=atol)


# ---------------------------------------------------------------- golden (exact)

def _frac(x):
    from fractions import Fraction
    if isinstance(x, list):
        return [_frac(y) for y in x]
    return float(Fraction(x))


@pytest.mark.parametrize("idx", [0, 1, 2])
def test_golden_exact(idx):
    doc = json.load(open(os.path.join(HERE, "golden", "tiny_exact.json")))
    c = doc["cases"][idx]
    I = {k: np.array(_frac(v)) for k, v in c["inputs"].items()}
    E = {k: np.array(_frac(v)) for k, v in c["expected"].items()}
    q, k, v = (I[n][None] for n in ("q", "k", "v"))
    S_in, z_in = I["S_in"][None], I["z_in"][None]
    o, S_out, z_out = oracle.fwd(q, k, v, S_in, z_in)
    close(o[0], E["o"], 1e-13, 1e-13)
    close(S_out[0], E["S_out"], 1e-13, 1e-13)
    close(z_out[0], E["z_out"], 1e-13, 1e-13)
    dq, dk, dv, dS, dz = oracle.bwd(q, k, v, S_in, z_in, I["dO"][None], I["dS_out"][None], I["dz_out"][None])
    close(dq[0], E["dq"], 1e-12, 1e-12)
    close(dk[0], E["dk"], 1e-12, 1e-12)
    close(dv[0], E["dv"], 1e-12, 1e-12)
    close(dS[0], E["dS_in"], 1e-12, 1e-12)
    close(dz[0], E["dz_in"], 1e-12, 1e-12)


# ---------------------------------------------------------------- closed forms

def test_p1_first_token_returns_its_value():
    q, k, v, *_ = rng_inputs(3, 9, 5, seed=1, carry=False)
    o, _, _ = oracle.fwd(q, k, v)
    close(o[:, 0], v[:, 0], 1e-14, 1e-14)


def test_p2_constant_values():
    q, k, v, S_in, z_in, *_ = rng_inputs(2, 20, 4, seed=2)
    c = np.array([0.5, -1.25, 2.0, 3.0])
    vc = np.broadcast_to(c, v.shape).copy()
    o, _, _ = oracle.fwd(q, k, vc)
    close(o, np.broadcast_to(c, o.shape), 1e-13, 1e-13)
    S_c = z_in[:, :, None] * c[None, None, :]            # consistent carry S_in = z_in c^T
    o2, _, _ = oracle.fwd(q, k, vc, S_c, z_in)
    close(o2, np.broadcast_to(c, o2.shape), 1e-13, 1e-13)


def test_p3_constant_keys_give_prefix_mean():
    q, _, v, *_ = rng_inputs(2, 33, 6, seed=3, carry=False)
    k = np.full_like(q, 0.7)
    o, _, _ = oracle.fwd(q, k, v)
    mean = np.cumsum(v, axis=1) / np.arange(1, v.shape[1] + 1)[None, :, None]
    close(o, mean, 1e-12, 1e-12)


def test_p4_d1_weighted_prefix_mean_and_zero_dq():
    q, k, v, S_in, z_in, dO, dS, dz = rng_inputs(3, 17, 1, seed=4)
    o, S_out, z_out = oracle.fwd(q, k, v, S_in, z_in)
    num = S_in[:, 0, 0][:, None] + np.cumsum(k[..., 0] * v[..., 0], axis=1)
    den = z_in[:, 0][:, None] + np.cumsum(k[..., 0], axis=1)
    close(o[..., 0], num / den, 1e-13, 1e-13)
    o2, _, _ = oracle.fwd(q * 3.7 + 0.1, k, v, S_in, z_in)   # independent of q
    close(o2, o, 1e-13, 1e-13)
    dq, *_ = oracle.bwd(q, k, v, S_in, z_in, dO, dS, dz)
    close(dq, np.zeros_like(dq), 0, 1e-13)


# ---------------------------------------------------------------- invariants

def test_p5_p6_p7_euler_identities():
    q, k, v, S_in, z_in, dO, dS, dz = rng_inputs(3, 40, 5, seed=5)
    o, S_out, z_out = oracle.fwd(q, k, v, S_in, z_in)
    dq, dk, dv, dS_in, dz_in = oracle.bwd(q, k, v, S_in, z_in, dO, dS, dz)
    # P5: o_t is unchanged by scaling q_t
    qdq = np.sum(q * dq, axis=2)
    close(qdq, np.zeros_like(qdq), 0, 1e-11 * np.abs(q * dq).sum(axis=2).max())
    # P6: degree 0 in (k, S_in, z_in) for o, degree 1 for (S_out, z_out)
    lhs = (k * dk).sum(axis=(1, 2)) + (S_in * dS_in).sum(axis=(1, 2)) + (z_in * dz_in).sum(axis=1)
    rhs = (dS * S_out).sum(axis=(1, 2)) + (dz * z_out).sum(axis=1)
    close(lhs, rhs, 1e-10, 1e-10)
    # P7: degree 1 in (v, S_in) for o and S_out, degree 0 for z_out
    lhs = (v * dv).sum(axis=(1, 2)) + (S_in * dS_in).sum(axis=(1, 2))
    rhs = (dO * o).sum(axis=(1, 2)) + (dS * S_out).sum(axis=(1, 2))
    close(lhs, rhs, 1e-10, 1e-10)


def test_p8_final_state_is_one_matmul():
    q, k, v, S_in, z_in, *_ = rng_inputs(2, 50, 6, seed=6)
    _, S_out, z_out = oracle.fwd(q, k, v, S_in, z_in)
    close(S_out, S_in + np.matmul(k.transpose(0, 2, 1), v), 1e-12, 1e-12)
    close(z_out, z_in + k.sum(axis=1), 1e-12, 1e-12)


def test_p9_carry_gradients_are_one_matmul():
    q, k, v, S_in, z_in, dO, dS, dz = rng_inputs(2, 50, 6, seed=7)
    o, _, _ = oracle.fwd(q, k, v, S_in, z_in)
    den = np.einsum("gtp,gtp->gt", q, z_in[:, None, :] + np.cumsum(k, axis=1))
    dN = dO / den[..., None]
    dden = -(dO * o).sum(axis=2) / den
    _, _, _, dS_in, dz_in = oracle.bwd(q, k, v, S_in, z_in, dO, dS, dz)
    close(dS_in - dS, np.matmul(q.transpose(0, 2, 1), dN), 1e-11, 1e-11)
    close(dz_in - dz, np.einsum("gtp,gt->gp", q, dden), 1e-11, 1e-11)


def test_p10_chunk_split_equals_single_call():
    q, k, v, S_in, z_in, dO, dS, dz = rng_inputs(2, 100, 5, seed=8)
    chunks = [5, 64, 1, 30]
    o_all, S_all, z_all = oracle.fwd(q, k, v, S_in, z_in)
    g_all = oracle.bwd(q, k, v, S_in, z_in, dO, dS, dz)
    # forward chain
    bounds = np.cumsum([0] + chunks)
    S, z, carries = S_in, z_in, []
    for a, b in zip(bounds[:-1], bounds[1:]):
        carries.append((S, z))
        o, S, z = oracle.fwd(q[:, a:b], k[:, a:b], v[:, a:b], S, z)
        close(o, o_all[:, a:b], 1e-12, 1e-12)
    close(S, S_all, 1e-12, 1e-12)
    close(z, z_all, 1e-12, 1e-12)
    # backward chain, last chunk first, carry gradients passed down
    gS, gz = dS, dz
    dq = np.empty_like(q); dk = np.empty_like(k); dv = np.empty_like(v)
    for i in range(len(chunks) - 1, -1, -1):
        a, b = bounds[i], bounds[i + 1]
        Sc, zc = carries[i]
        dq[:, a:b], dk[:, a:b], dv[:, a:b], gS, gz = oracle.bwd(
            q[:, a:b], k[:, a:b], v[:, a:b], Sc, zc, dO[:, a:b], gS, gz)
    for got, ref in zip((dq, dk, dv, gS, gz), g_all):
        close(got, ref, 1e-11, 1e-11)


@pytest.mark.parametrize("block", [1, 7, 16, 64, 100])
def test_p11_blocked_form_equals_recurrence(block):
    q, k, v, S_in, z_in, *_ = rng_inputs(2, 100, 6, seed=9)
    o, S_out, z_out = oracle.fwd(q, k, v, S_in, z_in)
    ob, Sb, zb = forms.blocked_fwd(q, k, v, S_in, z_in, block=block)
    close(ob, o, 1e-12, 1e-12)
    close(Sb, S_out, 1e-12, 1e-12)
    close(zb, z_out, 1e-12, 1e-12)


@pytest.mark.parametrize("carry", [False, True])
def test_p12_masked_einsum_equals_recurrence(carry):
    q, k, v, S_in, z_in, *_ = rng_inputs(2, 48, 5, seed=10, carry=carry)
    o, S_out, z_out = oracle.fwd(q, k, v, S_in, z_in)
    oe, Se, ze = forms.masked_einsum_fwd(q, k, v, S_in, z_in)
    close(oe, o, 1e-12, 1e-12)
    close(Se, S_out, 1e-12, 1e-12)
    close(ze, z_out, 1e-12, 1e-12)


@pytest.mark.parametrize("carry,upstream", [(True, True), (False, False), (True, False)])
def test_matrix_backward_equals_reverse_scan(carry, upstream):
    q, k, v, S_in, z_in, dO, dS, dz = rng_inputs(2, 70, 6, seed=11, carry=carry, upstream=upstream)
    ref = oracle.bwd(q, k, v, S_in, z_in, dO, dS, dz)
    got = forms.matrix_bwd(q, k, v, S_in, z_in, dO, dS, dz)
    for a, b in zip(got, ref):
        close(a, b, 1e-10, 1e-10)


def test_p13_finite_differences():
    G, T, D = 2, 11, 3
    q, k, v, S_in, z_in, dO, dS, dz = rng_inputs(G, T, D, seed=12)
    grads = oracle.bwd(q, k, v, S_in, z_in, dO, dS, dz)

    def L(q_, k_, v_, S_, z_):
        o, So, zo = oracle.fwd(q_, k_, v_, S_, z_)
        return (dO * o).sum() + (dS * So).sum() + (dz * zo).sum()

    args = [q, k, v, S_in, z_in]
    h = 1e-6
    r = np.random.default_rng(0)
    for ai, g in enumerate(grads):
        x = args[ai]
        for _ in range(12):
            idx = tuple(int(r.integers(0, n)) for n in x.shape)
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            ap, am = list(args), list(args)
            ap[ai], am[ai] = xp, xm
            fd = (L(*ap) - L(*am)) / (2 * h)
            assert abs(fd - g[idx]) <= 1e-6 * (1 + abs(g[idx])), (ai, idx, fd, g[idx])


def test_f1_feature_map_closed_forms():
    from oracle import features
    x = np.array([0.0, 2.0, 0.5, -1.0, -30.0, 1e-12, -1e-12])
    want = np.array([1.0, 3.0, 1.5, np.exp(-1.0), np.exp(-30.0), 1.0 + 1e-12, np.exp(-1e-12)])
    np.testing.assert_allclose(features.elu1(x), want, rtol=1e-15, atol=0)
    assert np.all(features.elu1(np.linspace(-20, 20, 1001)) > 0)
    np.testing.assert_array_equal(features.elu1_grad(np.array([3.0, 1e-9])), [1.0, 1.0])
    np.testing.assert_allclose(features.elu1_grad(np.array([-2.0, 0.0])), [np.exp(-2.0), 1.0], rtol=1e-15)


def test_f2_feature_map_derivative():
    from oracle import features
    x = np.array([-4.0, -1.3, -0.2, 0.3, 1.7, 5.0])
    h = 1e-6
    fd = (features.elu1(x + h) - features.elu1(x - h)) / (2 * h)
    np.testing.assert_allclose(features.elu1_grad(x), fd, rtol=1e-8)


def test_f3_fused_map_gradients():
    from oracle import features
    G, T, D = 2, 9, 3
    r = np.random.default_rng(31)
    xq, xk = r.normal(size=(G, T, D)), r.normal(size=(G, T, D))   # both signs
    _, _, v, S_in, z_in, dO, dS, dz = rng_inputs(G, T, D, seed=32)
    grads = features.bwd(xq, xk, v, S_in, z_in, dO, dS, dz)

    def L(xq_, xk_, v_, S_, z_):
        o, So, zo = features.fwd(xq_, xk_, v_, S_, z_)
        return (dO * o).sum() + (dS * So).sum() + (dz * zo).sum()

    args = [xq, xk, v, S_in, z_in]
    h = 1e-6
    for ai, g in enumerate(grads):
        x = args[ai]
        for _ in range(10):
            idx = tuple(int(r.integers(0, n)) for n in x.shape)
            if ai < 2 and abs(x[idx]) < 10 * h:
                continue  # the map has a kink at 0
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            ap, am = list(args), list(args)
            ap[ai], am[ai] = xp, xm
            fd = (L(*ap) - L(*am)) / (2 * h)
            assert abs(fd - g[idx]) <= 1e-6 * (1 + abs(g[idx])), (ai, idx, fd, g[idx])


def test_f4_feature_rounding():
    from oracle import features
    # x > 0 maps to x + 1: 1 + 2^-8 is halfway between bf16 neighbours 1 and 1 + 2^-7 -> even (1.0);
    # 1 + 3 * 2^-8 is halfway between 1 + 2^-7 and 1 + 2^-6 -> even (1 + 2^-6)
    x = np.array([2.0 ** -8, 3 * 2.0 ** -8, 0.5])
    np.testing.assert_array_equal(features.mapped(x, "bf16"), [1.0, 1.0 + 2.0 ** -6, 1.5])
    np.testing.assert_array_equal(features.mapped(np.array([-1.0]), "f32"), [np.float32(np.exp(-1.0))])
    r = np.random.default_rng(5)
    xq, xk = r.normal(size=(1, 6, 3)), r.normal(size=(1, 6, 3))
    v = r.normal(size=(1, 6, 3))
    got = features.fwd(xq, xk, v, dtype="bf16")
    want = oracle.fwd(features.mapped(xq, "bf16"), features.mapped(xk, "bf16"), v)
    for a, b in zip(got, want):
        np.testing.assert_array_equal(a, b)


def test_denominator_guard():
    q, k, v, *_ = rng_inputs(1, 4, 2, seed=13, carry=False)
    q[0, 2] = -q[0, 2]
    with pytest.raises(FloatingPointError):
        oracle.fwd(q, k, v)


# ---------------------------------------------------------------- input recipe

def test_inputs_deterministic_and_positive():
    a = inputs.make_inputs(G=3, T=20, D=8, dtype="bf16", carry="prior", backward=True, seed=0, prior_len=16)
    b = inputs.make_inputs(G=3, T=20, D=8, dtype="bf16", carry="prior", backward=True, seed=0, prior_len=16)
    for key in ("q", "k", "v", "dO", "S_in", "z_in"):
        assert a[key].shape == b[key].shape
        assert bool((a[key] == b[key]).all()), key
    import torch
    assert a["q"].dtype == torch.bfloat16 and a["S_in"].dtype == torch.float32
    assert bool((a["q"] > 0).all()) and bool((a["k"] > 0).all())
    assert bool((a["z_in"] > 0).all())


def test_inputs_group_sampling_matches_full_draw():
    full = inputs.make_inputs(G=6, T=10, D=4, dtype="f32", carry="prior", backward=True, seed=0, prior_len=8)
    part = inputs.make_inputs(G=6, T=10, D=4, dtype="f32", carry="prior", backward=True, seed=0, prior_len=8,
                              groups=[1, 4])
    for key in ("q", "k", "v", "dO", "S_in", "z_in"):
        assert bool((full[key][[1, 4]] == part[key]).all()), key


def test_workload_table():
    w = inputs.workload("g160_63x128p100_d128_bf16_fwdbwd")
    assert w.T == 63 * 128 + 100 and w.chunks[-1] == 100 and w.D == 128
    assert inputs.workload("g1280_8x128_d64_bf16_fwdbwd").T == 1024
    assert inputs.workload("g160_c128_d64_bf16_fwdbwd").G == 160


def test_raw_feature_inputs():
    # raw draws: the mapped inputs are elu(x)+1 of them, same draw order.  The mapped ones are
    # computed in fp32 as (e^x - 1) + 1, whose last addition rounds to 2^-24 absolute.
    a = inputs.make_inputs(G=2, T=16, D=8, dtype="f32", carry="prior", backward=True, seed=4, prior_len=8)
    b = inputs.make_inputs(G=2, T=16, D=8, dtype="f32", carry="prior", backward=True, seed=4, prior_len=8,
                           features="raw")
    from oracle import features
    np.testing.assert_allclose(features.elu1(b["q"]), a["q"].numpy(), rtol=2e-7, atol=1.2e-7)
    np.testing.assert_allclose(features.elu1(b["k"]), a["k"].numpy(), rtol=2e-7, atol=1.2e-7)
    for key in ("v", "dO", "S_in", "z_in"):
        assert np.array_equal(a[key].numpy(), b[key].numpy())
    assert (b["q"] < 0).any() and (b["q"] > 0).any()
