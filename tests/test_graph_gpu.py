"""HIP-graph capture of the library's calls (the benchmark replays its steps from graphs).

A step captured in a graph must give, on every replay, the bits an eager step gives.  Each
test runs the eager step once, captures the same calls, then replays the graph several times
with eager device work and synchronisations in between (the outputs are poisoned with NaN
before every replay) and compares every replay with the eager result.  The captured calls
record kernel nodes only: no memset or copy node is involved.
"""
import pytest
import torch

import causal_linear_attention_chunked_amd as lac
from causal_linear_attention_chunked_amd import inputs

pytestmark = pytest.mark.gpu

REPLAYS = 4


def _replays_match(step, outputs):
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outputs]
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        step()
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        for t in outputs:
            t.fill_(float("nan"))
        # unrelated eager work between the replays
        x = torch.randn(1 << 20, device="cuda")
        _ = (x * x).sum().item()
        g.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(ref, outputs)):
            assert torch.equal(a, b), f"replay {r}: output {i} differs from the eager step"


def _inputs(G, T, D, carry="prior"):
    I = inputs.make_inputs(G=G, T=T, D=D, dtype="bf16", carry=carry, backward=True, seed=0)
    return {n: (None if I[n] is None else I[n].cuda().contiguous()) for n in ("q", "k", "v", "S_in", "z_in", "dO")}


def test_headline_step_replays(gpu):
    x = _inputs(160, 128, 64)
    G, C, D = x["q"].shape
    fout = (torch.empty_like(x["q"]), torch.empty(G, D, D, device="cuda"), torch.empty(G, D, device="cuda"))
    bout = (torch.empty_like(x["q"]), torch.empty_like(x["q"]), torch.empty_like(x["q"]),
            torch.empty(G, D, D, device="cuda"), torch.empty(G, D, device="cuda"))

    def step():
        lac.fwd(x["q"], x["k"], x["v"], x["S_in"], x["z_in"], out=fout)
        lac.bwd(x["q"], x["k"], x["v"], x["S_in"], x["z_in"], x["dO"], out=bout)

    _replays_match(step, [*fout, *bout])


def test_chained_ragged_step_replays(gpu):
    # general kernels: a 128-token chunk then a ragged 100-token one, carry and gradient chained
    x = _inputs(8, 228, 128)
    q, k, v, dO = (x[n] for n in ("q", "k", "v", "dO"))
    qs = [q[:, :128].contiguous(), q[:, 128:].contiguous()]
    ks = [k[:, :128].contiguous(), k[:, 128:].contiguous()]
    vs = [v[:, :128].contiguous(), v[:, 128:].contiguous()]
    ds = [dO[:, :128].contiguous(), dO[:, 128:].contiguous()]
    G, D = q.shape[0], q.shape[2]
    fo = [(torch.empty_like(a), torch.empty(G, D, D, device="cuda"), torch.empty(G, D, device="cuda")) for a in qs]
    bo = [(torch.empty_like(a), torch.empty_like(a), torch.empty_like(a), torch.empty(G, D, D, device="cuda"),
           torch.empty(G, D, device="cuda")) for a in qs]

    def step():
        lac.fwd(qs[0], ks[0], vs[0], x["S_in"], x["z_in"], out=fo[0])
        lac.fwd(qs[1], ks[1], vs[1], fo[0][1], fo[0][2], out=fo[1])
        lac.bwd(qs[1], ks[1], vs[1], fo[0][1], fo[0][2], ds[1], out=bo[1])
        lac.bwd(qs[0], ks[0], vs[0], x["S_in"], x["z_in"], ds[0], bo[1][3], bo[1][4], out=bo[0])

    _replays_match(step, [t for pair in (fo, bo) for o in pair for t in o])


@pytest.mark.parametrize("T,D", [(1024, 64), (1000, 128)])
def test_sequence_step_replays(gpu, T, D):
    x = _inputs(16, T, D)
    q = x["q"]
    G = q.shape[0]
    fout = (torch.empty_like(q), torch.empty(G, D, D, device="cuda"), torch.empty(G, D, device="cuda"),
            torch.empty(G, D, D, device="cuda"), torch.empty(G, D, device="cuda"))
    bout = (torch.empty_like(q), torch.empty_like(q), torch.empty_like(q), torch.empty(G, D, D, device="cuda"),
            torch.empty(G, D, device="cuda"))

    def step():
        lac.seq_fwd(q, x["k"], x["v"], x["S_in"], x["z_in"], out=fout, residual=True)
        lac.seq_bwd(q, x["k"], x["v"], fout[1], fout[2], x["dO"], out=bout, S_res=fout[3], z_res=fout[4])

    _replays_match(step, [*fout, *bout])
