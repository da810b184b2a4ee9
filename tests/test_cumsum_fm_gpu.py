"""GPU parity for the per-token (cumsum) form, the fp32 backward at D = 128 and the fused feature
map on the one-chunk entry points, through the C ABI, against the fp64 oracle.

* block = 1 selects the cumsum form of "Fractus-1B training optimization" (section 2, Opt 1 and
  Opt 2): the exact per-token recurrence.  It is held to the same tolerance as the blocked form
  (tests/tol.py: 1e-4 for fp32, 2e-2 for bf16) on the workloads' shapes, on ragged chunk
  lengths around its 32-token staging batches, and up to the longest backward chunk.
* The fp32 backward at D = 128 (the wide-head workload's head size) runs that form: fp32 parity
  at 1e-4 on the wide-head workload's chunking (128-token chunks, a 100-token ragged tail).
* feature = "elu1" takes raw q, k: checked against the oracle's feature layer both on the
  reading the kernels follow (features rounded to the element type) and on the unrounded
  composition, at the bf16 bound.
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


def chain(I, chunks, block, feature=None, backward=True, dS_out=None, dz_out=None):
    """Chained chunk calls over the chunk list (carry and carry gradient passed along)."""
    bounds = inp.chunk_bounds(chunks)
    q, k, v = (dev(I[n]) for n in ("q", "k", "v"))
    cut = lambda x: [x[:, a:b].contiguous() for a, b in bounds]
    qc, kc, vc = cut(q), cut(k), cut(v)
    S, z = dev(I["S_in"]), dev(I["z_in"])
    outs, carries = [], []
    for a, b, c in zip(qc, kc, vc):
        carries.append((S, z))
        o, S, z = lac.fwd(a, b, c, S, z, block=block, feature=feature)
        outs.append(o)
    res = {"o": torch.cat(outs, 1), "S_out": S, "z_out": z}
    if backward:
        gc = cut(dev(I["dO"]))
        gS, gz = dev(dS_out), dev(dz_out)
        dq, dk, dv = [None] * len(qc), [None] * len(qc), [None] * len(qc)
        for i in range(len(qc) - 1, -1, -1):
            dq[i], dk[i], dv[i], gS, gz = lac.bwd(qc[i], kc[i], vc[i], *carries[i], gc[i], gS, gz, block=block,
                                                  feature=feature)
        res.update(dq=torch.cat(dq, 1), dk=torch.cat(dk, 1), dv=torch.cat(dv, 1), dS_in=gS, dz_in=gz)
    torch.cuda.synchronize()
    return res


def reference(I, backward=True, groups=None, feature=None, fdtype=None, dS_out=None, dz_out=None):
    sel = (lambda x: x) if groups is None else (lambda x: None if x is None else x[groups])
    a = [sel(I[n]) for n in ("q", "k", "v", "S_in", "z_in")]
    dS, dz = sel(dS_out), sel(dz_out)
    if feature == "elu1":
        o, S, z = oracle.features.fwd(*a, dtype=fdtype)
        ref = {"o": o, "S_out": S, "z_out": z}
        if backward:
            ref.update(zip(("dq", "dk", "dv", "dS_in", "dz_in"),
                           oracle.features.bwd(*a, sel(I["dO"]), dS, dz, dtype=fdtype)))
        return ref
    o, S, z = oracle.fwd(*a)
    ref = {"o": o, "S_out": S, "z_out": z}
    if backward:
        ref.update(zip(("dq", "dk", "dv", "dS_in", "dz_in"), oracle.bwd(*a, sel(I["dO"]), dS, dz)))
    return ref


def compare(res, ref, rtol, groups=None, label=""):
    for name, r in ref.items():
        g = res[name]
        if groups is not None:
            g = g[torch.as_tensor(groups, device=g.device)]
        nw = check(f"{label}{name}", g, r, rtol)
        say(f"  {label}{name}: normwise rel err {nw:.2e}")


# ---------------------------------------------------------------- the cumsum form (block = 1)

@pytest.mark.parametrize("name,dtype,G,sample", [
    ("g1_c128_d64_f32_fwd", None, None, None),
    ("g160_c128_d64_bf16_fwdbwd", None, None, [0, 77, 159]),
    ("g160_c128_d64_bf16_fwdbwd", "f32", 16, None),
    ("g1280_8x128_d64_bf16_fwdbwd", "f32", 8, None),
    ("g160_63x128p100_d128_bf16_fwdbwd", None, 4, None),
])
def test_cumsum_form_on_workload_shapes(gpu, name, dtype, G, sample):
    w = inp.workload(name)
    dt = dtype or w.dtype
    I = inp.make_inputs(G=G or w.G, T=w.T, D=w.D, dtype=dt, carry=w.carry, backward=w.backward, seed=w.seed,
                        prior_len=w.prior_len)
    say(f"[case] cumsum form {name} dtype={dt} G={G or w.G} chunks={len(w.chunks)}")
    res = chain(I, list(w.chunks), block=1, backward=w.backward)
    compare(res, reference(I, w.backward, sample), RTOL[dt], sample)


@pytest.mark.parametrize("dtype,D", [("f32", 64), ("bf16", 64), ("f32", 128), ("bf16", 128)])
@pytest.mark.parametrize("C", [1, 5, 31, 32, 33, 100, 257])
def test_cumsum_form_chunk_lengths(gpu, dtype, D, C):
    I = inp.make_inputs(G=3, T=C, D=D, dtype=dtype, carry="prior", backward=True, seed=C + D)
    rng = np.random.default_rng(C)
    dS = torch.from_numpy(rng.standard_normal((3, D, D)).astype(np.float32))
    dz = torch.from_numpy(rng.standard_normal((3, D)).astype(np.float32))
    say(f"[case] cumsum form C={C} D={D} {dtype}, carry and upstream")
    res = chain(I, [C], block=1, dS_out=dS, dz_out=dz)
    compare(res, reference(I, dS_out=dS, dz_out=dz), RTOL[dtype])


def test_cumsum_form_longest_backward_chunk_zero_carry(gpu):
    C = lac.BWD_MAX_C
    I = inp.make_inputs(G=2, T=C, D=64, dtype="f32", carry="zero", backward=True, seed=5)
    say(f"[case] cumsum form C={C} fp32 zero carry")
    res = chain(I, [C], block=1)
    compare(res, reference(I), RTOL["f32"])


def test_cumsum_and_blocked_forms_agree(gpu):
    # the same function in two summation orders: to fp32 rounding on fp32 inputs
    I = inp.make_inputs(G=8, T=300, D=64, dtype="f32", carry="prior", backward=True, seed=3)
    a = chain(I, [128, 128, 44], block=1)
    b = chain(I, [128, 128, 44], block=64)
    for n in a:
        x, y = a[n].double(), b[n].double()
        rel = float((x - y).norm() / y.norm())
        say(f"  {n}: cumsum vs blocked {rel:.2e}")
        assert rel < 1e-5, (n, rel)


# ---------------------------------------------------------------- the fp32 backward at D = 128

def test_fp32_wide_heads_backward(gpu):
    # the wide-head workload's chunking (63 x 128 + 100 tokens) on sampled groups' worth of G, fp32
    w = inp.workload("g160_63x128p100_d128_bf16_fwdbwd")
    I = inp.make_inputs(G=3, T=w.T, D=128, dtype="f32", carry="prior", backward=True, seed=w.seed)
    say(f"[case] fp32 D=128 forward+backward, G=3, {len(w.chunks)} chunks, T={w.T}")
    assert lac.kernel_name(True, "float32", 128, 128) == "la_cumsum_bwd_kernel"
    res = chain(I, list(w.chunks), block=64)
    compare(res, reference(I), RTOL["f32"])


# ---------------------------------------------------------------- fused feature map, chunk calls

@pytest.mark.parametrize("dtype,D,chunks,G", [
    ("bf16", 64, [128], 160),          # the 128-token kernels with the map
    ("bf16", 64, [128, 128, 100], 4),  # a ragged D = 64 sequence through the chunk calls
    ("bf16", 128, [128, 100], 4),
    ("f32", 64, [128, 37], 4),
    ("f32", 128, [64, 64], 2),
])
def test_fused_map_chunk_calls(gpu, dtype, D, chunks, G):
    T = sum(chunks)
    I = inp.make_inputs(G=G, T=T, D=D, dtype=dtype, carry="prior", backward=True, seed=40 + D, features="raw")
    say(f"[case] fused map, chunk calls {chunks} D={D} {dtype} G={G}")
    res = chain(I, chunks, block=64, feature="elu1")
    # the reading the kernels follow: phi rounded to the element type
    compare(res, reference(I, feature="elu1", fdtype=dtype), RTOL[dtype], label="rounded ")
    # the unrounded composition: the reading is not load-bearing at the bf16 bound
    compare(res, reference(I, feature="elu1", fdtype=None), RTOL["bf16"], label="exact ")


def test_fused_map_cumsum_form(gpu):
    I = inp.make_inputs(G=4, T=160, D=64, dtype="bf16", carry="zero", backward=True, seed=8, features="raw")
    say("[case] fused map, cumsum form, zero carry")
    res = chain(I, [64, 96], block=1, feature="elu1")
    compare(res, reference(I, feature="elu1", fdtype="bf16"), RTOL["bf16"])


def test_fused_map_inputs_deep_in_each_branch(gpu):
    # raw inputs far below zero (phi = e^x, small) and far above (phi = x + 1)
    I = inp.make_inputs(G=4, T=128, D=64, dtype="bf16", carry="prior", backward=True, seed=12, features="raw")
    for n, shift in (("q", -3.0), ("k", 2.5)):
        I[n] = (I[n].float() + shift).to(torch.bfloat16)
    say("[case] fused map, shifted raw inputs, the 128-token kernels")
    res = chain(I, [128], block=64, feature="elu1")
    compare(res, reference(I, feature="elu1", fdtype="bf16"), RTOL["bf16"])
