"""la_ce_fwd_noalloc: the cross-entropy forward with the library's static per-device scratch as
its workspace, for callers that cannot allocate.

Called through the C ABI (ctypes, no binding logic in between) and compared bit for bit with
la_ce_fwd on a caller-owned workspace: the two run the same kernels, so loss and lse must be
identical.  Two calls in a row, the second on a smaller input, show that the scratch's leftover
contents from a larger call do not leak into a smaller one.  Also: a size beyond the scratch is
refused before anything is launched.
"""
import ctypes

import pytest
import torch

import causal_linear_attention_chunked_amd as lac
from causal_linear_attention_chunked_amd import inputs

pytestmark = pytest.mark.gpu

LA_BF16, LA_OK, LA_ERR_UNSUPPORTED = 1, 0, 2


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _case(N, d, V, seed):
    I = inputs.make_ce_inputs(N=N, d=d, V=V, seed=seed)
    return I["h"].cuda().contiguous(), I["W"].cuda().contiguous(), I["targets"].cuda().contiguous()


def _with_workspace(lib, h, W, t):
    N, d, V = h.shape[0], h.shape[1], W.shape[0]
    ws_bytes = lib.la_ce_fwd_workspace_bytes(N, d, V)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    loss, lse = torch.empty((), device="cuda"), torch.empty(N, device="cuda")
    st = lib.la_ce_fwd(h.data_ptr(), W.data_ptr(), t.data_ptr(), loss.data_ptr(), lse.data_ptr(), ws.data_ptr(),
                       ws_bytes, N, d, V, LA_BF16, _stream())
    assert st == LA_OK
    return loss, lse


def _no_alloc(lib, h, W, t, loss, lse):
    N, d, V = h.shape[0], h.shape[1], W.shape[0]
    return lib.la_ce_fwd_noalloc(h.data_ptr(), W.data_ptr(), t.data_ptr(), loss.data_ptr(), lse.data_ptr(), N, d, V,
                                 LA_BF16, _stream())


def test_no_alloc_forward_matches_the_workspace_forward(gpu):
    lib = lac.load_library()
    # the larger call first (its partials fill more of the scratch), then a smaller, ragged one
    for N, d, V, seed in ((2000, 256, 50257, 1), (37, 128, 1000, 2)):
        h, W, t = _case(N, d, V, seed)
        ref_loss, ref_lse = _with_workspace(lib, h, W, t)
        loss = torch.full((), float("nan"), device="cuda")
        lse = torch.full((N,), float("nan"), device="cuda")
        assert _no_alloc(lib, h, W, t, loss, lse) == LA_OK
        torch.cuda.synchronize()
        assert torch.isfinite(lse).all() and torch.isfinite(loss)
        assert torch.equal(loss, ref_loss), (N, d, V, float(loss), float(ref_loss))
        assert torch.equal(lse, ref_lse), (N, d, V)


def test_no_alloc_refuses_sizes_beyond_its_scratch(gpu):
    lib = lac.load_library()
    N, d, V = 6000, 128, 50257   # (197 + 1) x 6016 x 8 bytes > 8 MiB
    assert lib.la_ce_fwd_workspace_bytes(N, d, V) > lac.CE_NOALLOC_SCRATCH_BYTES
    h = torch.zeros(N, d, device="cuda", dtype=torch.bfloat16)
    W = torch.zeros(V, d, device="cuda", dtype=torch.bfloat16)
    t = torch.zeros(N, device="cuda", dtype=torch.int32)
    loss, lse = torch.empty((), device="cuda"), torch.empty(N, device="cuda")
    assert _no_alloc(lib, h, W, t, loss, lse) == LA_ERR_UNSUPPORTED
    with pytest.raises(lac.LachunkError, match="scratch"):
        lac.ce_fwd_noalloc(h, W, t, out=(loss, lse))
