"""The Python binding refuses wrong device buffers before anything reaches the library.

The C ABI can check only alignment and overlap of the pointers it gets, so an output of the
wrong size, a host tensor or a wrong element type must be caught in Python: each case here
raises ValueError, and the library is never called (its entry points are replaced by a function
that fails the test if reached).
"""
import pytest
import torch

import causal_linear_attention_chunked_amd as lac

pytestmark = pytest.mark.gpu


@pytest.fixture
def no_launch(monkeypatch):
    lib = lac.load_library()

    class Guard:
        def __getattr__(self, name):
            if name.startswith("la_") and name not in ("la_status_str", "la_ce_workspace_bytes",
                                                       "la_ce_fwd_workspace_bytes"):
                def fail(*a):
                    raise AssertionError(f"{name} was called with arguments the binding should refuse")
                return fail
            return getattr(lib, name)

    monkeypatch.setattr(lac, "_lib", Guard())
    yield


def _tok(G=4, C=128, D=64, dtype=torch.bfloat16):
    return torch.rand(G, C, D, device="cuda").to(dtype) + 0.5


def test_fwd_out_checked(gpu, no_launch):
    q = _tok()
    G, C, D = q.shape
    good = lambda: [torch.empty_like(q), torch.empty(G, D, D, device="cuda"), torch.empty(G, D, device="cuda")]
    for i, bad in [(0, torch.empty(G, C - 1, D, device="cuda", dtype=q.dtype)),   # short o
                   (0, torch.empty(G, C, D, device="cuda")),                      # fp32 o for bf16 inputs
                   (0, torch.empty(G, C, D, dtype=q.dtype)),                      # host o
                   (1, torch.empty(G, D, D - 1, device="cuda")),                  # short S_out
                   (1, torch.empty(G, D, D, device="cuda", dtype=torch.float64)),
                   (2, torch.empty(G, D + 1, device="cuda")),
                   (2, None)]:
        out = good()
        out[i] = bad
        with pytest.raises(ValueError):
            lac.fwd(q, q, q, out=tuple(out))


def test_bwd_and_seq_out_checked(gpu, no_launch):
    q = _tok()
    G, C, D = q.shape
    S = torch.zeros(G, D, D, device="cuda")
    z = torch.ones(G, D, device="cuda")
    out = [torch.empty_like(q) for _ in range(3)] + [torch.empty(G, D, D, device="cuda"), torch.empty(G, D, device="cuda")]
    out[2] = torch.empty(G, C, D // 2, device="cuda", dtype=q.dtype)
    with pytest.raises(ValueError):
        lac.bwd(q, q, q, S, z, q, out=tuple(out))
    with pytest.raises(ValueError):
        lac.seq_bwd(q, q, q, S, z, q, out=tuple(out))
    fout = (torch.empty_like(q), torch.empty(G, D, D, device="cuda"), torch.empty(G, D, device="cuda"),
            torch.empty(G, D, D, device="cuda"), torch.empty(G, 3, device="cuda"))   # short z_res
    with pytest.raises(ValueError):
        lac.seq_fwd(q, q, q, S, z, out=fout, residual=True)


def test_ce_arguments_checked(gpu, no_launch):
    N, d, V = 8, 128, 300
    h = torch.randn(N, d, device="cuda").bfloat16()
    W = torch.randn(V, d, device="cuda").bfloat16()
    t = torch.randint(0, V, (N,), device="cuda", dtype=torch.int32)
    lse = torch.zeros(N, device="cuda")
    cases = [dict(lse=lse.cpu()), dict(lse=lse.double()), dict(lse=lse[:-1]),
             dict(dloss=torch.tensor(2.0)),                              # a host scalar
             dict(dloss=torch.tensor(2.0, device="cuda", dtype=torch.float64)),
             dict(dloss=torch.ones(2, device="cuda")),
             dict(out=(torch.empty(N, d, device="cuda"), torch.empty(V, d, device="cuda"))),      # fp32 dh
             dict(out=(torch.empty_like(h), torch.empty(V, d - 1, device="cuda"))),
             dict(workspace=torch.empty(1 << 20, dtype=torch.uint8))]  # host workspace
    for kw in cases:
        args = dict(lse=lse, dloss=None)
        args.update(kw)
        with pytest.raises(ValueError):
            lac.ce_bwd(h, W, t, args.pop("lse"), **args)
    for out in [(torch.empty((), device="cuda", dtype=torch.float64), lse.clone()),
                (torch.empty((), device="cuda"), torch.empty(N + 1, device="cuda"))]:
        with pytest.raises(ValueError):
            lac.ce_fwd(h, W, t, out=out)
