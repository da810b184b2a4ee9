"""GPU parity: the HIP library (through its C ABI) against the fp64 CPU oracle.

Inputs come from causal_linear_attention_chunked_amd.inputs (seeded); expected
values from oracle/ only.  Tolerance (tests/tol.py): per tensor, elementwise
|x - r| <= rtol (|r| + rms(r)), rtol = 1e-4 for fp32 inputs, 2e-2 for bf16.
Full-size workloads are computed on the GPU for every group and compared on a
sample of groups, which the oracle computes in full (groups are independent).
"""
import numpy as np
import pytest
import torch

import causal_linear_attention_chunked_amd as lac
from causal_linear_attention_chunked_amd import inputs as inp
import oracle  # noqa: E402
from tol import RTOL, check

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def to_dev(x):
    return None if x is None else x.to("cuda:0").contiguous()


def chunks_of(x, bounds):
    return [x[:, a:b].contiguous() for a, b in bounds]


def run_gpu(I, chunks, backward):
    """Chained forward (and backward) over the chunk list; returns host fp64 numpy results."""
    bounds = inp.chunk_bounds(chunks)
    q, k, v = (to_dev(I[n]) for n in ("q", "k", "v"))
    S_in, z_in = to_dev(I["S_in"]), to_dev(I["z_in"])
    qc, kc, vc = chunks_of(q, bounds), chunks_of(k, bounds), chunks_of(v, bounds)
    outs, carries, (S_out, z_out) = lac.chain_fwd(qc, kc, vc, S_in, z_in)
    res = {"o": torch.cat(outs, dim=1), "S_out": S_out, "z_out": z_out}
    if backward:
        gc = chunks_of(to_dev(I["dO"]), bounds)
        dqs, dks, dvs, dS, dz = lac.chain_bwd(qc, kc, vc, carries, gc)
        res.update(dq=torch.cat(dqs, 1), dk=torch.cat(dks, 1), dv=torch.cat(dvs, 1), dS_in=dS, dz_in=dz)
    torch.cuda.synchronize()
    return res


def run_oracle(I, backward, groups=None):
    sel = (lambda x: x) if groups is None else (lambda x: None if x is None else x[groups])
    q, k, v, S_in, z_in = (sel(I[n]) for n in ("q", "k", "v", "S_in", "z_in"))
    o, S_out, z_out = oracle.fwd(q, k, v, S_in, z_in)
    ref = {"o": o, "S_out": S_out, "z_out": z_out}
    if backward:
        dq, dk, dv, dS, dz = oracle.bwd(q, k, v, S_in, z_in, sel(I["dO"]))
        ref.update(dq=dq, dk=dk, dv=dv, dS_in=dS, dz_in=dz)
    return ref


def compare(res, ref, dtype, groups=None, label=""):
    for name, r in ref.items():
        g = res[name]
        if groups is not None:
            g = g[torch.as_tensor(groups, device=g.device)]
        nw = check(f"{label}{name}", g, r, RTOL[dtype])
        say(f"  {label}{name}: normwise rel err {nw:.2e}")


def workload_case(name, dtype=None, G=None, sample=None):
    w = inp.workload(name)
    dt = dtype or w.dtype
    I = inp.make_inputs(G=G or w.G, T=w.T, D=w.D, dtype=dt, carry=w.carry, backward=w.backward,
                        seed=w.seed, prior_len=w.prior_len)
    say(f"[case] {name} dtype={dt} G={G or w.G} chunks={len(w.chunks)} T={w.T} D={w.D} bwd={w.backward}")
    res = run_gpu(I, list(w.chunks), w.backward)
    groups = sample
    ref = run_oracle(I, w.backward, groups)
    compare(res, ref, dt, groups)


# ---------------------------------------------------------------- the five workloads, full size

def test_g1_fp32_forward(gpu):
    workload_case("g1_c128_d64_f32_fwd")


def test_headline_forward(gpu):
    workload_case("g160_c128_d64_bf16_fwd")


def test_headline_forward_backward(gpu):
    workload_case("g160_c128_d64_bf16_fwdbwd")


def test_long_batch_eight_chunks(gpu):
    workload_case("g1280_8x128_d64_bf16_fwdbwd", sample=[0, 1, 2, 333, 640, 901, 1278, 1279])


def test_wide_heads_ragged(gpu):
    workload_case("g160_63x128p100_d128_bf16_fwdbwd", sample=[0, 57, 159])


# ---------------------------------------------------------------- fp32 instantiations on the same shapes

@pytest.mark.parametrize("name,G", [
    ("g160_c128_d64_bf16_fwdbwd", 16),
    ("g1280_8x128_d64_bf16_fwdbwd", 8),
])
def test_fp32_on_workload_shapes(gpu, name, G):
    workload_case(name, dtype="f32", G=G)


def test_fp32_wide_heads_forward(gpu):
    # fp32 at D=128 has a forward only (the backward's LDS budget does not fit fp32 tiles)
    w = inp.workload("g160_63x128p100_d128_bf16_fwdbwd")
    I = inp.make_inputs(G=3, T=w.T, D=128, dtype="f32", carry="prior", backward=False)
    say(f"[case] fp32 D=128 forward, G=3, T={w.T}")
    res = run_gpu(I, list(w.chunks), False)
    compare(res, run_oracle(I, False), "f32")


# ---------------------------------------------------------------- maximum sizes

@pytest.mark.parametrize("dtype,D", [("f32", 64), ("bf16", 64), ("bf16", 128)])
def test_longest_backward_chunk(gpu, dtype, D):
    # the backward's limit: LA_BWD_MAX_C tokens in one call (per-token den and dden held on chip)
    C = lac.BWD_MAX_C
    I = inp.make_inputs(G=2, T=C, D=D, dtype=dtype, carry="prior", backward=True, seed=51)
    say(f"[case] longest backward chunk C={C} dtype={dtype} D={D}")
    compare(run_gpu(I, [C], True), run_oracle(I, True), dtype)


def test_whole_sequence_in_one_forward_call(gpu):
    # the wide-head sequence (8164 tokens, ragged 36-token tail) as a single forward chunk
    T = 63 * 128 + 100
    I = inp.make_inputs(G=2, T=T, D=128, dtype="bf16", carry="prior", backward=False, seed=52)
    say(f"[case] one forward call over T={T} at D=128")
    compare(run_gpu(I, [T], False), run_oracle(I, False), "bf16")


# ---------------------------------------------------------------- ragged, short and long chunks

@pytest.mark.parametrize("C", [1, 5, 37, 63, 64, 65, 100, 127, 128, 130, 192, 200, 256])
@pytest.mark.parametrize("dtype,D", [("f32", 64), ("bf16", 64), ("bf16", 128)])
def test_chunk_lengths(gpu, C, dtype, D):
    I = inp.make_inputs(G=3, T=C, D=D, dtype=dtype, carry="prior", backward=True, seed=C)
    g = torch.Generator().manual_seed(1000 + C)
    dS = torch.randn((3, D, D), generator=g)
    dz = torch.randn((3, D), generator=g)
    say(f"[case] C={C} D={D} dtype={dtype}")
    q, k, v, S_in, z_in, dO = (to_dev(I[n]) for n in ("q", "k", "v", "S_in", "z_in", "dO"))
    o, S_out, z_out = lac.fwd(q, k, v, S_in, z_in)
    dq, dk, dv, dS_in, dz_in = lac.bwd(q, k, v, S_in, z_in, dO, to_dev(dS), to_dev(dz))
    torch.cuda.synchronize()
    ro, rS, rz = oracle.fwd(I["q"], I["k"], I["v"], I["S_in"], I["z_in"])
    rdq, rdk, rdv, rdS, rdz = oracle.bwd(I["q"], I["k"], I["v"], I["S_in"], I["z_in"], I["dO"], dS, dz)
    tol = RTOL[dtype]
    for n, a, b in (("o", o, ro), ("S_out", S_out, rS), ("z_out", z_out, rz), ("dq", dq, rdq),
                    ("dk", dk, rdk), ("dv", dv, rdv), ("dS_in", dS_in, rdS), ("dz_in", dz_in, rdz)):
        check(n, a, b, tol)


@pytest.mark.parametrize("dtype,D", [("f32", 64), ("bf16", 128)])
def test_zero_carry_and_no_upstream(gpu, dtype, D):
    I = inp.make_inputs(G=2, T=100, D=D, dtype=dtype, carry="zero", backward=True, seed=3)
    say(f"[case] zero carry D={D} dtype={dtype}")
    q, k, v, dO = (to_dev(I[n]) for n in ("q", "k", "v", "dO"))
    o, S_out, z_out = lac.fwd(q, k, v)
    dq, dk, dv, dS_in, dz_in = lac.bwd(q, k, v, None, None, dO)
    torch.cuda.synchronize()
    ro, rS, rz = oracle.fwd(I["q"], I["k"], I["v"])
    g = oracle.bwd(I["q"], I["k"], I["v"], None, None, I["dO"])
    for n, a, b in zip(("o", "S_out", "z_out", "dq", "dk", "dv", "dS_in", "dz_in"),
                       (o, S_out, z_out, dq, dk, dv, dS_in, dz_in), (ro, rS, rz) + tuple(g)):
        check(n, a, b, RTOL[dtype])


# ---------------------------------------------------------------- properties

def test_closed_forms_on_gpu(gpu):
    say("[case] closed forms fp32")
    I = inp.make_inputs(G=4, T=130, D=64, dtype="f32", carry="zero", backward=False, seed=5)
    q, k = to_dev(I["q"]), to_dev(I["k"])
    v = to_dev(I["v"])
    o, _, _ = lac.fwd(q, k, v)
    torch.cuda.synchronize()
    # zero carry: the first token returns its own value
    check("o_1", o[:, 0], I["v"][:, 0].double().numpy(), 1e-5)
    c = torch.linspace(-2, 3, 64)
    vc = c.expand(4, 130, 64).contiguous()
    o2, _, _ = lac.fwd(q, k, to_dev(vc))
    torch.cuda.synchronize()
    check("o const", o2, vc.double().numpy(), 1e-5)


def test_euler_identities_on_gpu_gradients(gpu):
    say("[case] Euler identities fp32")
    I = inp.make_inputs(G=4, T=200, D=64, dtype="f32", carry="prior", backward=True, seed=6)
    g = torch.Generator().manual_seed(6)
    dS = torch.randn((4, 64, 64), generator=g)
    dz = torch.randn((4, 64), generator=g)
    q, k, v, S_in, z_in, dO = (to_dev(I[n]) for n in ("q", "k", "v", "S_in", "z_in", "dO"))
    o, S_out, z_out = lac.fwd(q, k, v, S_in, z_in)
    dq, dk, dv, dS_in, dz_in = lac.bwd(q, k, v, S_in, z_in, dO, to_dev(dS), to_dev(dz))
    torch.cuda.synchronize()
    f = lambda x: x.double().cpu()
    q, k, v, S_in, z_in, dO, o, S_out, z_out = map(f, (q, k, v, S_in, z_in, dO, o, S_out, z_out))
    dq, dk, dv, dS_in, dz_in, dS, dz = map(f, (dq, dk, dv, dS_in, dz_in, dS, dz))
    qdq = (q * dq).sum(-1)
    assert float(qdq.abs().max()) <= 1e-4 * float((q * dq).abs().sum(-1).max())
    lhs = (k * dk).sum((1, 2)) + (S_in * dS_in).sum((1, 2)) + (z_in * dz_in).sum(1)
    rhs = (dS * S_out).sum((1, 2)) + (dz * z_out).sum(1)
    scale = (k * dk).abs().sum((1, 2)) + (S_in * dS_in).abs().sum((1, 2)) + (dS * S_out).abs().sum((1, 2))
    assert bool(((lhs - rhs).abs() <= 1e-4 * scale).all())
    lhs = (v * dv).sum((1, 2)) + (S_in * dS_in).sum((1, 2))
    rhs = (dO * o).sum((1, 2)) + (dS * S_out).sum((1, 2))
    scale = (v * dv).abs().sum((1, 2)) + (S_in * dS_in).abs().sum((1, 2)) + (dO * o).abs().sum((1, 2))
    assert bool(((lhs - rhs).abs() <= 1e-4 * scale).all())


def test_chunk_split_equals_single_call(gpu):
    say("[case] chunk split vs single call fp32")
    I = inp.make_inputs(G=3, T=256, D=64, dtype="f32", carry="prior", backward=True, seed=7)
    one = run_gpu(I, [256], True)
    split = run_gpu(I, [64, 37, 128, 27], True)
    for n in one:
        check(f"split/{n}", split[n], one[n].double().cpu().numpy(), 1e-4)


def test_bitwise_deterministic(gpu):
    say("[case] determinism bf16 headline shape")
    I = inp.workload_inputs(inp.workload("g160_c128_d64_bf16_fwdbwd"))
    a = run_gpu(I, [128], True)
    b = run_gpu(I, [128], True)
    for n in a:
        assert torch.equal(a[n], b[n]), n


def test_every_output_written(gpu):
    say("[case] NaN-poisoned outputs")
    for dtype, D, C in (("bf16", 64, 128), ("bf16", 128, 100), ("f32", 64, 37)):
        I = inp.make_inputs(G=5, T=C, D=D, dtype=dtype, carry="prior", backward=True, seed=8)
        q, k, v, S_in, z_in, dO = (to_dev(I[n]) for n in ("q", "k", "v", "S_in", "z_in", "dO"))
        nan = lambda t: torch.full_like(t, float("nan"))
        out = (nan(q), nan(S_in), nan(z_in))
        lac.fwd(q, k, v, S_in, z_in, out=out)
        gout = (nan(q), nan(q), nan(q), nan(S_in), nan(z_in))
        lac.bwd(q, k, v, S_in, z_in, dO, out=gout)
        torch.cuda.synchronize()
        for t in out + gout:
            assert bool(torch.isfinite(t).all()), (dtype, D, C)
