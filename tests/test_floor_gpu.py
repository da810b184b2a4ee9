"""GPU: the launch-floor kernels (a measurement aid) move exactly the bytes they are said to move.

Each streaming kind reads its workgroups' input slabs and writes, for every thread, the xor of
its 16-byte loads plus the store's index; the result is compared with the same computed on the
CPU, so the bytes the floor figures count are the bytes the kernels touch (and nothing past the
buffers: the output's tail beyond the kind's bytes keeps its fill).
"""
import pytest
import torch

import causal_linear_attention_chunked_amd as lac

pytestmark = pytest.mark.gpu

# kind: (loads per thread, stores per thread, threads per workgroup)
SHAPES = {"fwd": (8, 4, 512), "bwd": (10, 8, 512), "fwd_small": (8, 4, 128), "bwd_small": (10, 8, 128)}


def expected(inp, nwg, nin, nout, nt):
    x = inp[: nwg * nin * nt * 4].view(nwg, nin, nt, 4)
    acc = x[:, 0]
    for i in range(1, nin):
        acc = acc ^ x[:, i]
    return torch.stack([acc + j for j in range(nout)], dim=1).reshape(-1)  # [wg][j][thread][4]


@pytest.mark.parametrize("kind", sorted(SHAPES))
def test_floor_kernels_move_their_bytes(gpu, kind):
    nin, nout, nt = SHAPES[kind]
    nwg = 37
    print(f"[case] floor kind={kind} nwg={nwg}", flush=True)
    g = torch.Generator().manual_seed(nwg + nin)
    inp = torch.randint(-2**31, 2**31 - 1, (nwg * nin * nt * 4,), dtype=torch.int32, generator=g)
    spare = 64  # int32s past the kind's output, which must keep their fill
    out = torch.full((nwg * nout * nt * 4 + spare,), -7, dtype=torch.int32, device="cuda:0")
    lac.floor_launch(kind, nwg, inp.to("cuda:0"), out)
    torch.cuda.synchronize()
    got = out.cpu()
    assert torch.equal(got[: nwg * nout * nt * 4], expected(inp, nwg, nin, nout, nt))
    assert bool((got[nwg * nout * nt * 4:] == -7).all())


def test_floor_empty_kernel_writes_nothing(gpu):
    out = torch.full((512,), 5, dtype=torch.int32, device="cuda:0")
    lac.floor_launch("empty", 160, None, out)
    torch.cuda.synchronize()
    assert bool((out == 5).all())
