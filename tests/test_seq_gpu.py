"""GPU parity of the sequence entry points (la_seq_fwd / la_seq_bwd through the binding),
at D = 64 (128-token chunks) and D = 128 (any length, ragged end).

Against the fp64 oracle (one call over the whole sequence is the chain of its chunks),
to the tolerance of tests/tol.py; and against chained per-chunk calls: the forward
state S bit for bit, z and o to fp32 rounding (the sequence keeps z's compensation
term across chunks), the backward to fp32 rounding (its forward states come from the
final carry by subtraction).
"""
import numpy as np
import pytest
import torch

import causal_linear_attention_chunked_amd as lac
from causal_linear_attention_chunked_amd import inputs as inp
import oracle
from tol import RTOL, check

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def dev(x):
    return None if x is None else x.to("cuda:0").contiguous()


def upstream(G, D, seed):
    rng = np.random.default_rng(seed)
    return (torch.from_numpy(rng.standard_normal((G, D, D)).astype(np.float32)),
            torch.from_numpy(rng.standard_normal((G, D)).astype(np.float32)))


def run_seq(I, dS=None, dz=None, feature=None, chunk=128, residual=True):
    # residual: the final carry's remainders go from the forward to the backward (as the autograd
    # layer passes them); without, the backward starts from the rounded carry
    q, k, v, dO = (dev(I[n]) for n in ("q", "k", "v", "dO"))
    S_res = z_res = None
    if residual:
        o, S_out, z_out, S_res, z_res = lac.seq_fwd(q, k, v, dev(I["S_in"]), dev(I["z_in"]), chunk=chunk,
                                                    feature=feature, residual=True)
    else:
        o, S_out, z_out = lac.seq_fwd(q, k, v, dev(I["S_in"]), dev(I["z_in"]), chunk=chunk, feature=feature)
    dq, dk, dv, dS_in, dz_in = lac.seq_bwd(q, k, v, S_out, z_out, dO, dev(dS), dev(dz), chunk=chunk,
                                           feature=feature, S_res=S_res, z_res=z_res)
    torch.cuda.synchronize()
    return dict(o=o, S_out=S_out, z_out=z_out, dq=dq, dk=dk, dv=dv, dS_in=dS_in, dz_in=dz_in)


def oracle_ref(I, dS=None, dz=None, groups=None, feature=None):
    sel = (lambda x: x) if groups is None else (lambda x: None if x is None else x[groups])
    args = [sel(I[n]) for n in ("q", "k", "v", "S_in", "z_in")]
    if feature == "elu1":
        # the features enter the op at its element type (bf16)
        o, S_out, z_out = oracle.features.fwd(*args, dtype="bf16")
        dq, dk, dv, dS_in, dz_in = oracle.features.bwd(*args, sel(I["dO"]), sel(dS), sel(dz), dtype="bf16")
    else:
        o, S_out, z_out = oracle.fwd(*args)
        dq, dk, dv, dS_in, dz_in = oracle.bwd(*args, sel(I["dO"]), sel(dS), sel(dz))
    return dict(o=o, S_out=S_out, z_out=z_out, dq=dq, dk=dk, dv=dv, dS_in=dS_in, dz_in=dz_in)


def compare(res, ref, groups=None, label=""):
    for name, r in ref.items():
        g = res[name]
        if groups is not None:
            g = g[torch.as_tensor(groups, device=g.device)]
        nw = check(f"{label}{name}", g, r, RTOL["bf16"])
        say(f"  {label}{name}: normwise rel err {nw:.2e}")


@pytest.mark.parametrize("G,nchunk,carry,up,res", [
    (5, 5, "zero", False, True),
    (3, 3, "prior", True, True),
    (1, 1, "prior", False, True),
    (2, 10, "zero", True, True),
    (3, 4, "prior", True, False),   # without the remainders (short: the rounded carry suffices)
])
def test_seq_against_oracle(gpu, G, nchunk, carry, up, res):
    T = 128 * nchunk
    say(f"[case] seq G={G} T={T} carry={carry} upstream={up} remainders={res}")
    I = inp.make_inputs(G=G, T=T, D=64, dtype="bf16", carry=carry, backward=True, seed=7 + nchunk)
    dS, dz = upstream(G, 64, 99) if up else (None, None)
    compare(run_seq(I, dS, dz, residual=res), oracle_ref(I, dS, dz))


def test_seq_long_sequence(gpu):
    # 64 chunks: the recovered forward states are 64 subtractions away from the final carry
    G, T = 2, 128 * 64
    say(f"[case] seq long G={G} T={T}")
    I = inp.make_inputs(G=G, T=T, D=64, dtype="bf16", carry="prior", backward=True, seed=3)
    dS, dz = upstream(G, 64, 5)
    compare(run_seq(I, dS, dz), oracle_ref(I, dS, dz))


def test_seq_very_long_sequence(gpu):
    # 2048 chunks (262144 tokens) in one launch per direction: the carry and the recovered
    # forward states over a long run, and buffer ranges far past one chunk
    G, T = 1, 128 * 2048
    say(f"[case] seq very long G={G} T={T}")
    I = inp.make_inputs(G=G, T=T, D=64, dtype="bf16", carry="prior", backward=True, seed=9)
    compare(run_seq(I), oracle_ref(I))


def test_seq_longest_sequence_zero_carry(gpu):
    # the longest supported sequence from a zero carry: the first tokens' states are tiny next to
    # the final carry they are recovered from (exact only with the remainders)
    G, T = 1, lac.SEQ_D64_MAX_T
    say(f"[case] seq longest, zero carry, G={G} T={T}")
    I = inp.make_inputs(G=G, T=T, D=64, dtype="bf16", carry="zero", backward=True, seed=10)
    dS, dz = upstream(G, 64, 11)
    compare(run_seq(I, dS, dz), oracle_ref(I, dS, dz))


def test_seq_eight_chunks_full_size(gpu):
    # eight 128-token chunks at G = 1280, every group computed, a sample compared
    w = inp.workload("g1280_8x128_d64_bf16_fwdbwd")
    say(f"[case] seq full {w.name}")
    I = inp.workload_inputs(w)
    groups = [0, 1, 255, 256, 640, 1023, 1279]
    compare(run_seq(I), oracle_ref(I, groups=groups), groups)


def test_seq_matches_chained_calls(gpu):
    G, n = 6, 4
    T = 128 * n
    say(f"[case] seq vs chain G={G} T={T}")
    I = inp.make_inputs(G=G, T=T, D=64, dtype="bf16", carry="prior", backward=True, seed=21)
    dS, dz = upstream(G, 64, 22)
    res = run_seq(I, dS, dz)
    bounds = inp.chunk_bounds([128] * n)
    cut = lambda x: [dev(x)[:, a:b].contiguous() for a, b in bounds]
    qc, kc, vc, gc = cut(I["q"]), cut(I["k"]), cut(I["v"]), cut(I["dO"])
    outs, carries, (S_out, z_out) = lac.chain_fwd(qc, kc, vc, dev(I["S_in"]), dev(I["z_in"]))
    dqs, dks, dvs, dS_in, dz_in = lac.chain_bwd(qc, kc, vc, carries, gc, dev(dS), dev(dz))
    torch.cuda.synchronize()
    # forward: S and z to their last bits (the sequence carries their compensation terms across
    # chunks, the chain rounds them at every chunk boundary), o to the rounding that follows
    assert float(((res["S_out"] - S_out).norm() / S_out.norm())) < 1e-6
    assert float(((res["z_out"] - z_out).abs() / z_out.abs()).max()) < 1e-6
    o_rel = float((res["o"].double() - torch.cat(outs, 1).double()).norm() / torch.cat(outs, 1).double().norm())
    say(f"  o: seq vs chain normwise {o_rel:.2e}")
    assert o_rel < 1e-3
    # backward: within fp32 rounding of the recovered states (normwise)
    for name, a, b in (("dq", res["dq"], torch.cat(dqs, 1)), ("dk", res["dk"], torch.cat(dks, 1)),
                       ("dv", res["dv"], torch.cat(dvs, 1)), ("dS_in", res["dS_in"], dS_in),
                       ("dz_in", res["dz_in"], dz_in)):
        a, b = a.double(), b.double()
        rel = float((a - b).norm() / b.norm())
        say(f"  {name}: seq vs chain normwise {rel:.2e}")
        assert rel < 2e-3, (name, rel)


@pytest.mark.parametrize("G,nchunk,carry,up", [(3, 3, "prior", True), (2, 10, "zero", False), (1, 1, "zero", True)])
def test_seq_fused_feature_map(gpu, G, nchunk, carry, up):
    # raw q, k (both signs); the op applies elu(x)+1 and returns gradients of the raw inputs
    T = 128 * nchunk
    say(f"[case] seq elu1 G={G} T={T} carry={carry} upstream={up}")
    I = inp.make_inputs(G=G, T=T, D=64, dtype="bf16", carry=carry, backward=True, seed=40 + nchunk,
                        features="raw")
    dS, dz = upstream(G, 64, 41) if up else (None, None)
    compare(run_seq(I, dS, dz, feature="elu1"), oracle_ref(I, dS, dz, feature="elu1"))


@pytest.mark.parametrize("shift", [-4.0, 4.0])
def test_seq_fused_feature_map_branches(gpu, shift):
    # raw inputs pushed deep into one branch of elu: e^x (small features) or x + 1
    G, T = 2, 256
    say(f"[case] seq elu1 raw inputs shifted by {shift}")
    I = inp.make_inputs(G=G, T=T, D=64, dtype="bf16", carry="zero", backward=True, seed=44, features="raw")
    for n in ("q", "k"):
        I[n] = (I[n].float() + shift).to(torch.bfloat16)
    compare(run_seq(I, feature="elu1"), oracle_ref(I, feature="elu1"))


def test_seq_fused_feature_map_full_size(gpu):
    w = inp.workload("g1280_8x128_d64_bf16_fwdbwd")
    say(f"[case] seq elu1 full {w.name}")
    I = inp.make_inputs(G=w.G, T=w.T, D=w.D, dtype=w.dtype, carry=w.carry, backward=True, seed=w.seed,
                        features="raw")
    groups = [0, 511, 1279]
    compare(run_seq(I, feature="elu1"), oracle_ref(I, groups=groups, feature="elu1"), groups)


# ---------------------------------------------------------------- D = 128

def run_seq_d128(I, dS=None, dz=None, chunk=128, residual=True):
    return run_seq(I, dS, dz, chunk=chunk, residual=residual)


@pytest.mark.parametrize("G,T,carry,up,res", [
    (3, 64, "prior", True, True),     # one full block
    (2, 200, "zero", True, True),     # three blocks and an 8-token ragged end
    (3, 1000, "prior", False, True),  # 15 blocks and 40 tokens
    (1, 1, "prior", True, True),      # a single token
    (2, 63, "prior", True, True),     # less than one block
    (2, 129, "zero", False, True),    # one token past two blocks
    (2, 700, "prior", True, False),   # without the remainders
])
def test_seq_d128_against_oracle(gpu, G, T, carry, up, res):
    say(f"[case] seq D=128 G={G} T={T} carry={carry} upstream={up} remainders={res}")
    I = inp.make_inputs(G=G, T=T, D=128, dtype="bf16", carry=carry, backward=True, seed=60 + T)
    dS, dz = upstream(G, 128, 61) if up else (None, None)
    compare(run_seq_d128(I, dS, dz, residual=res), oracle_ref(I, dS, dz))


def test_seq_d128_single_token_zero_carry(gpu):
    # The degenerate case: one token from a zero carry gives o_1 = v_1 whatever q_1 is, so the
    # exact dq_1 is 0 (its two terms, S_1 dO_1 / den_1 and z_1 (o_1 . dO_1) / den_1, cancel).
    # dq is held to fp32 rounding of those terms; the other outputs to the oracle's tolerance.
    G, T, D = 3, 1, 128
    say(f"[case] seq D=128 single token, zero carry, G={G}")
    I = inp.make_inputs(G=G, T=T, D=D, dtype="bf16", carry="zero", backward=True, seed=67)
    dS, dz = upstream(G, D, 68)
    res, ref = run_seq_d128(I, dS, dz), oracle_ref(I, dS, dz)
    dq = ref.pop("dq")
    assert float(np.abs(dq).max()) < 1e-12  # the oracle's own rounding
    compare({n: res[n] for n in ref}, ref)
    q, k, v, dO = (I[n][:, 0].double().numpy() for n in ("q", "k", "v", "dO"))
    den = np.sum(q * k, axis=1, keepdims=True)
    term = np.abs(k) * np.abs(np.sum(v * dO, axis=1, keepdims=True)) / den  # |S_1 dO_1| / den_1
    got = res["dq"][:, 0].double().cpu().numpy()
    ratio = float(np.max(np.abs(got) / term))
    say(f"  dq: max |dq| / |term| = {ratio:.2e}")
    assert ratio < 1e-5


def test_seq_d128_wide_head_workload(gpu):
    # 160 groups of 63 x 128 + 100 tokens at D = 128 in one launch per direction, a sample compared
    w = inp.workload("g160_63x128p100_d128_bf16_fwdbwd")
    say(f"[case] seq D=128 full {w.name}")
    I = inp.workload_inputs(w)
    groups = [0, 57, 159]
    compare(run_seq_d128(I), oracle_ref(I, groups=groups), groups)


def test_seq_d128_longest_sequence(gpu):
    # the longest supported sequence from a zero carry: the recovered states are 256 subtractions
    # away from the final carry, and the first ones are tiny next to it
    G, T = 1, lac.SEQ_D128_MAX_T
    say(f"[case] seq D=128 longest, zero carry, G={G} T={T}")
    I = inp.make_inputs(G=G, T=T, D=128, dtype="bf16", carry="zero", backward=True, seed=63)
    dS, dz = upstream(G, 128, 64)
    compare(run_seq_d128(I, dS, dz), oracle_ref(I, dS, dz))


@pytest.mark.parametrize("G,T,carry,up,res", [
    (2, 200, "zero", True, True),      # an 8-token ragged end: phi(0) = 1 must not enter z past it
    (3, 64, "prior", False, True),     # one full block
    (1, 1, "prior", True, True),       # a single token (from a zero carry its exact dq is 0: degenerate)
    (2, 1000, "prior", True, True),    # 15 blocks and 40 tokens
    (2, 700, "prior", True, False),    # without the remainders: the backward starts from the rounded carry
])
def test_seq_d128_fused_feature_map(gpu, G, T, carry, up, res):
    # raw q, k (both signs) at D = 128; the op applies elu(x)+1, gradients of the raw inputs
    say(f"[case] seq D=128 elu1 G={G} T={T} carry={carry} upstream={up} remainders={res}")
    I = inp.make_inputs(G=G, T=T, D=128, dtype="bf16", carry=carry, backward=True, seed=70 + T,
                        features="raw")
    dS, dz = upstream(G, 128, 71) if up else (None, None)
    compare(run_seq(I, dS, dz, feature="elu1", residual=res), oracle_ref(I, dS, dz, feature="elu1"))


@pytest.mark.parametrize("shift", [-4.0, 4.0])
def test_seq_d128_fused_feature_map_branches(gpu, shift):
    # raw inputs pushed deep into one branch of elu: e^x (small features) or x + 1
    G, T = 2, 300
    say(f"[case] seq D=128 elu1 raw inputs shifted by {shift}")
    I = inp.make_inputs(G=G, T=T, D=128, dtype="bf16", carry="zero", backward=True, seed=74, features="raw")
    for n in ("q", "k"):
        I[n] = (I[n].float() + shift).to(torch.bfloat16)
    compare(run_seq(I, feature="elu1"), oracle_ref(I, feature="elu1"))


def test_seq_d128_fused_feature_map_wide_head_workload(gpu):
    # the wide-head workload's shapes (63 x 128 + 100 tokens, 160 groups) on raw inputs
    w = inp.workload("g160_63x128p100_d128_bf16_fwdbwd")
    say(f"[case] seq D=128 elu1 full {w.name}")
    I = inp.make_inputs(G=w.G, T=w.T, D=w.D, dtype=w.dtype, carry=w.carry, backward=True, seed=w.seed,
                        features="raw")
    groups = [0, 101, 159]
    compare(run_seq(I, feature="elu1"), oracle_ref(I, groups=groups, feature="elu1"), groups)


def test_seq_d128_matches_chained_calls(gpu):
    # the chunk length (a multiple of 64) does not change the arithmetic: results bit for bit;
    # against the chained calls, to fp32 rounding (compensated carry, the ragged end as a
    # masked block instead of token by token)
    G, chunks = 4, [128, 128, 128, 72]
    T = sum(chunks)
    say(f"[case] seq D=128 vs chain G={G} T={T}")
    I = inp.make_inputs(G=G, T=T, D=128, dtype="bf16", carry="prior", backward=True, seed=65)
    dS, dz = upstream(G, 128, 66)
    res = run_seq_d128(I, dS, dz)
    res64 = run_seq_d128(I, dS, dz, chunk=64)
    for name in res:
        assert torch.equal(res[name], res64[name]), name
    bounds = inp.chunk_bounds(chunks)
    cut = lambda x: [dev(x)[:, a:b].contiguous() for a, b in bounds]
    qc, kc, vc, gc = cut(I["q"]), cut(I["k"]), cut(I["v"]), cut(I["dO"])
    outs, carries, (S_out, z_out) = lac.chain_fwd(qc, kc, vc, dev(I["S_in"]), dev(I["z_in"]))
    dqs, dks, dvs, dS_in, dz_in = lac.chain_bwd(qc, kc, vc, carries, gc, dev(dS), dev(dz))
    torch.cuda.synchronize()
    assert float(((res["S_out"] - S_out).norm() / S_out.norm())) < 1e-6
    assert float(((res["z_out"] - z_out).abs() / z_out.abs()).max()) < 1e-6
    o_chain = torch.cat(outs, 1).double()
    o_rel = float((res["o"].double() - o_chain).norm() / o_chain.norm())
    say(f"  o: seq vs chain normwise {o_rel:.2e}")
    assert o_rel < 1e-3
    for name, a, b in (("dq", res["dq"], torch.cat(dqs, 1)), ("dk", res["dk"], torch.cat(dks, 1)),
                       ("dv", res["dv"], torch.cat(dvs, 1)), ("dS_in", res["dS_in"], dS_in),
                       ("dz_in", res["dz_in"], dz_in)):
        a, b = a.double(), b.double()
        rel = float((a - b).norm() / b.norm())
        say(f"  {name}: seq vs chain normwise {rel:.2e}")
        assert rel < 2e-3, (name, rel)


@pytest.mark.parametrize("C,feature", [(1, None), (100, None), (128, "elu1"), (640, None), (2048, None)])
def test_chunk_d128_backward_from_the_carry_before(gpu, C, feature):
    # la_chunk_bwd at bf16, D = 128 builds the carry after the chunk from the carry before it, then
    # walks back like la_seq_bwd: against the oracle, and against la_seq_bwd given the forward's
    # final carry with its remainders (the same walk: to fp32 rounding)
    G = 3
    say(f"[case] chunk bwd D=128 from S_in, C={C}, feature={feature}")
    I = inp.make_inputs(G=G, T=C, D=128, dtype="bf16", carry="prior", backward=True, seed=70 + C,
                        features="raw" if feature else "mapped")
    dS, dz = upstream(G, 128, 71)
    q, k, v, dO = (dev(I[n]) for n in ("q", "k", "v", "dO"))
    S_in, z_in = dev(I["S_in"]), dev(I["z_in"])
    assert lac.kernel_name(True, "bf16", C, 128, feature=feature) == (
        "la_bwd_d128_elu1_kernel" if feature else "la_bwd_d128_kernel")
    o, S_out, z_out = lac.fwd(q, k, v, S_in, z_in, feature=feature)
    dq, dk, dv, dS_in, dz_in = lac.bwd(q, k, v, S_in, z_in, dO, dev(dS), dev(dz), feature=feature)
    _, S2, z2, Sr, zr = lac.seq_fwd(q, k, v, S_in, z_in, chunk=128 * ((C + 127) // 128), feature=feature,
                                    residual=True)
    ref = lac.seq_bwd(q, k, v, S2, z2, dO, dev(dS), dev(dz), chunk=128 * ((C + 127) // 128), feature=feature,
                      S_res=Sr, z_res=zr)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv", "dS_in", "dz_in"), (dq, dk, dv, dS_in, dz_in), ref):
        a, b = a.double(), b.double()
        rel = float((a - b).norm() / b.norm())
        say(f"  {name}: chunk call vs sequence call normwise {rel:.2e}")
        assert rel < 1e-3, (name, rel)
    res = {"o": o, "S_out": S_out, "z_out": z_out, "dq": dq, "dk": dk, "dv": dv, "dS_in": dS_in, "dz_in": dz_in}
    if feature:
        a = [I[n] for n in ("q", "k", "v", "S_in", "z_in")]
        ro, rS, rz = oracle.features.fwd(*a, dtype="bf16")
        rb = oracle.features.bwd(*a, I["dO"], dS, dz, dtype="bf16")
    else:
        ro, rS, rz = oracle.fwd(I["q"], I["k"], I["v"], I["S_in"], I["z_in"])
        rb = oracle.bwd(I["q"], I["k"], I["v"], I["S_in"], I["z_in"], I["dO"], dS, dz)
    for name, r in zip(("o", "S_out", "z_out", "dq", "dk", "dv", "dS_in", "dz_in"), (ro, rS, rz, *rb)):
        check(name, res[name], r, RTOL["bf16"])


def test_seq_rejects_unsupported(gpu):
    x = torch.ones(2, 200, 64, dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(lac.LachunkError, match="UNSUPPORTED"):
        lac.seq_fwd(x, x, x)
    with pytest.raises(ValueError):
        lac.seq_fwd(x[:, :128], x[:, :128], x[:, :128], feature="relu")
    y = torch.ones(2, 200, 128, dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(lac.LachunkError, match="UNSUPPORTED"):
        lac.seq_fwd(y, y, y, chunk=100)
    with pytest.raises(lac.LachunkError, match="UNSUPPORTED"):
        lac.seq_fwd(y, y, y, chunk=96, feature="elu1")
