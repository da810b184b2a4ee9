"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments before touching the device.

Only error paths are exercised: validation runs on the host before any HIP
call, so the fake device addresses below are never dereferenced.
"""
import ctypes
import os
import re

import pytest

import causal_linear_attention_chunked_amd as lac

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "la_chunk.h")

OK, INVALID, UNSUPPORTED, ALIGN, ALIAS = 0, 1, 2, 3, 4


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(lac.lib_path()):
        from causal_linear_attention_chunked_amd import build
        build.build()
    return lac.load_library()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\S.*?\b(la_[a-z_]+)\s*\(", text, flags=re.M)))


def test_header_declares_the_boundary():
    assert declared_functions() == ["la_abi_version", "la_ce_bwd", "la_ce_fwd", "la_ce_fwd_noalloc",
                                    "la_ce_fwd_workspace_bytes",
                                    "la_ce_workspace_bytes",
                                    "la_chunk_bwd", "la_chunk_fwd", "la_floor_launch", "la_kernel_name",
                                    "la_seq_bwd", "la_seq_fwd", "la_seq_kernel_name", "la_status_str",
                                    "la_time_next_launch"]


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = os.popen(f"nm -D --defined-only {lac.lib_path()}").read()
    for name in declared_functions():
        assert re.search(rf"\bT {name}$", out, flags=re.M), name


def test_kernel_names(lib):
    assert lac.kernel_name(False, "bf16", 128, 64) == "la_fwd_c128_kernel"
    assert lac.kernel_name(True, "bf16", 128, 64) == "la_bwd_c128w16_kernel"
    assert lac.kernel_name(False, "bf16", 100, 128) == "la_seq_fwd_d128_kernel"
    assert lac.kernel_name(True, "bf16", 100, 128) == "la_bwd_d128_kernel"
    assert lac.kernel_name(True, "bf16", 128, 128, feature="elu1") == "la_bwd_d128_elu1_kernel"
    assert lac.kernel_name(False, "bf16", 16385, 128) == "la_fwd_kernel"
    assert lac.kernel_name(False, "bf16", 16384, 128) == "la_seq_fwd_d128_kernel"
    assert lac.kernel_name(True, "float32", 128, 64) == "la_bwd_kernel"
    # the fp32 backward at D = 128 runs the per-token form
    assert lac.kernel_name(True, "float32", 128, 128) == "la_cumsum_bwd_kernel"
    assert lac.kernel_name(False, "float32", 128, 128) == "la_fwd_kernel"
    assert lac.kernel_name(False, "bf16", 128, 96) is None
    # block 1: the cumsum form on every shape; the fused map: the 128-token kernels at their
    # shape, the per-token form elsewhere
    assert lac.kernel_name(False, "bf16", 128, 64, block=1) == "la_cumsum_fwd_kernel"
    assert lac.kernel_name(True, "float32", 37, 128, block=1) == "la_cumsum_bwd_kernel"
    assert lac.kernel_name(False, "bf16", 128, 64, feature="elu1") == "la_fwd_c128_elu1_kernel"
    assert lac.kernel_name(True, "bf16", 128, 64, feature="elu1") == "la_bwd_c128w16_elu1_kernel"
    assert lac.kernel_name(True, "bf16", 100, 64, feature="elu1") == "la_cumsum_bwd_kernel"
    assert lac.kernel_name(True, "bf16", lac.BWD_MAX_C + 1, 64, block=1) is None
    assert lac.kernel_name(False, "bf16", 128, 64, block=16) is None


def test_sequence_limits_match_the_header():
    text = open(HEADER).read()
    for name, value in (("LA_SEQ_D64_MAX_T", lac.SEQ_D64_MAX_T), ("LA_SEQ_D128_MAX_T", lac.SEQ_D128_MAX_T)):
        assert int(re.search(rf"#define {name} (\d+)", text).group(1)) == value, name


def test_version_and_status_strings(lib):
    assert lac.abi_version() == 6
    for s in range(6):
        assert len(lac.status_str(s)) > 0
    assert lac.status_str(99) == "unknown status"


# fake, 16-byte aligned, non-overlapping device addresses (never dereferenced)
BASE = 1 << 40
STEP = 1 << 32


def addr(i):
    return ctypes.c_void_p(BASE + i * STEP)


def fwd_call(lib, G=4, C=128, D=64, block=64, dt=1, feature=0, **over):
    args = {n: addr(i) for i, n in enumerate(["q", "k", "v", "S_in", "z_in", "o", "S_out", "z_out"])}
    args.update(over)
    return lib.la_chunk_fwd(args["q"], args["k"], args["v"], args["S_in"], args["z_in"], args["o"],
                            args["S_out"], args["z_out"], G, C, D, block, feature, dt, None)


def bwd_call(lib, G=4, C=128, D=64, block=64, dt=1, feature=0, **over):
    names = ["q", "k", "v", "S_in", "z_in", "dO", "dS_out", "dz_out", "dq", "dk", "dv", "dS_in", "dz_in"]
    args = {n: addr(i) for i, n in enumerate(names)}
    args.update(over)
    return lib.la_chunk_bwd(*[args[n] for n in names], G, C, D, block, feature, dt, None)


@pytest.mark.parametrize("kw,status", [
    (dict(G=0), INVALID), (dict(C=0), INVALID), (dict(G=-3), INVALID),
    (dict(D=32), UNSUPPORTED), (dict(D=96), UNSUPPORTED), (dict(block=32), UNSUPPORTED),
    (dict(block=2), UNSUPPORTED), (dict(block=0), UNSUPPORTED), (dict(dt=7), UNSUPPORTED),
    (dict(feature=2), INVALID), (dict(feature=-1, block=1), INVALID),
    (dict(q=None), INVALID), (dict(o=None), INVALID), (dict(S_out=None), INVALID),
    (dict(S_in=None), INVALID),                          # z_in given without S_in
    (dict(q=ctypes.c_void_p(BASE + 8)), ALIGN),
    (dict(o=addr(0)), ALIAS),                            # o == q
    (dict(S_out=addr(3)), ALIAS),                        # S_out == S_in (the call is pure)
    (dict(z_out=ctypes.c_void_p(BASE + 5 * STEP + 64)), ALIAS),  # z_out inside o
])
def test_fwd_rejects(lib, kw, status):
    assert fwd_call(lib, **kw) == status


def test_fwd_size_overflow(lib):
    assert fwd_call(lib, G=2**31 - 1, C=2**31 - 1, D=128) in (INVALID,)


@pytest.mark.parametrize("kw,status", [
    (dict(G=0), INVALID), (dict(D=48), UNSUPPORTED), (dict(block=16), UNSUPPORTED),
    (dict(C=lac.BWD_MAX_C + 1), UNSUPPORTED), (dict(C=lac.BWD_MAX_C + 1, block=1), UNSUPPORTED),
    (dict(feature=3), INVALID),
    (dict(dO=None), INVALID), (dict(dS_in=None), INVALID),
    (dict(dS_out=None), INVALID),                        # dz_out without dS_out
    (dict(z_in=None), INVALID),
    (dict(dk=ctypes.c_void_p(BASE + 9 * STEP + 4)), ALIGN),
    (dict(dq=addr(5)), ALIAS),                           # dq == dO
    (dict(dS_in=addr(6)), ALIAS),                        # dS_in == dS_out
    (dict(dv=addr(9)), ALIAS),                           # dv == dk
])
def test_bwd_rejects(lib, kw, status):
    assert bwd_call(lib, **kw) == status


def test_fwd_chunk_beyond_32bit_offsets(lib):
    # (C + 256) * D * 2 bytes must stay below 2^31
    assert fwd_call(lib, G=1, C=(1 << 31) // (128 * 2), D=128) == UNSUPPORTED
    assert fwd_call(lib, G=1, C=(1 << 31) // (128 * 4) - 200, D=128, dt=0) == UNSUPPORTED
    assert bwd_call(lib, G=1, C=(1 << 31) // (64 * 2), D=64) == UNSUPPORTED


SEQ_FWD_ARGS = ["q", "k", "v", "S_in", "z_in", "o", "S_out", "z_out", "S_res", "z_res"]


def seq_fwd_call(lib, G=4, T=512, D=64, chunk=128, block=64, feature=0, dt=1, **over):
    args = {n: addr(i) for i, n in enumerate(SEQ_FWD_ARGS)}
    args.update(over)
    return lib.la_seq_fwd(*[args[n] for n in SEQ_FWD_ARGS], G, T, D, chunk, block, feature, dt, None)


def seq_bwd_call(lib, G=4, T=512, D=64, chunk=128, block=64, feature=0, dt=1, **over):
    names = ["q", "k", "v", "S_last", "z_last", "S_res", "z_res", "dO", "dS_out", "dz_out", "dq", "dk", "dv",
             "dS_in", "dz_in"]
    args = {n: addr(i) for i, n in enumerate(names)}
    args.update(over)
    return lib.la_seq_bwd(*[args[n] for n in names], G, T, D, chunk, block, feature, dt, None)


@pytest.mark.parametrize("kw,status", [
    (dict(G=0), INVALID), (dict(T=0), INVALID), (dict(chunk=0), INVALID),
    (dict(T=500), UNSUPPORTED),                          # not whole chunks
    (dict(chunk=64, T=512), UNSUPPORTED), (dict(dt=0), UNSUPPORTED),
    # D = 128: chunks a multiple of 64, T up to the limit
    (dict(D=128, chunk=100, T=500), UNSUPPORTED), (dict(D=128, feature=1, T=500, chunk=96), UNSUPPORTED),
    (dict(D=128, T=lac.SEQ_D128_MAX_T + 1), UNSUPPORTED), (dict(D=128, T=0), INVALID),
    (dict(block=32), UNSUPPORTED), (dict(T=lac.SEQ_D64_MAX_T + 128), UNSUPPORTED),
    (dict(q=None), INVALID), (dict(S_in=None), INVALID),
    (dict(v=ctypes.c_void_p(BASE + 2 * STEP + 8)), ALIGN),
    (dict(o=addr(1)), ALIAS), (dict(S_out=addr(3)), ALIAS),
    (dict(feature=2), INVALID), (dict(feature=-1), INVALID), (dict(feature=2, D=128), INVALID),
    (dict(S_res=None), INVALID), (dict(z_res=None), INVALID),   # the remainders come together
    (dict(S_res=addr(6)), ALIAS),                        # S_res == S_out
    (dict(z_res=ctypes.c_void_p(BASE + 9 * STEP + 8)), ALIGN),
])
def test_seq_fwd_rejects(lib, kw, status):
    assert seq_fwd_call(lib, **kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(G=0), INVALID), (dict(T=384 + 1), UNSUPPORTED), (dict(D=128, chunk=96), UNSUPPORTED),
    (dict(D=128, T=lac.SEQ_D128_MAX_T + 64), UNSUPPORTED),
    (dict(S_last=None), INVALID), (dict(z_last=None), INVALID),   # the final carry is required
    (dict(dS_out=None), INVALID),                        # dz_out without dS_out
    (dict(dq=None), INVALID),
    (dict(dk=ctypes.c_void_p(BASE + 9 * STEP + 4)), ALIGN),
    (dict(dq=addr(5)), ALIAS), (dict(dS_in=addr(3)), ALIAS),
    (dict(feature=7), INVALID),
    (dict(z_res=None), INVALID),                         # S_res without z_res
    (dict(dS_in=addr(5)), ALIAS),                        # dS_in == S_res
])
def test_seq_bwd_rejects(lib, kw, status):
    assert seq_bwd_call(lib, **kw) == status


def test_seq_kernel_names(lib):
    assert lac.seq_kernel_name(False, "bf16", 128, 64) == "la_seq_fwd_c128_kernel"
    assert lac.seq_kernel_name(True, "bf16", 128, 64) == "la_seq_bwd_c128w16_kernel"
    assert lac.seq_kernel_name(True, "float32", 128, 64) is None
    assert lac.seq_kernel_name(False, "bf16", 128, 64, "elu1") == "la_seq_fwd_c128_elu1_kernel"
    assert lac.seq_kernel_name(True, "bf16", 128, 64, "elu1") == "la_seq_bwd_c128w16_elu1_kernel"
    with pytest.raises(ValueError):
        lac.seq_kernel_name(True, "bf16", 128, 64, "relu")
    assert lac.seq_supported("bf16", 1024, 64, 128) and not lac.seq_supported("bf16", 1000, 64, 128)
    assert not lac.seq_supported("float32", 1024, 64, 128) and not lac.seq_supported("float32", 1024, 128, 128)
    assert lac.seq_kernel_name(False, "bf16", 128, 128) == "la_seq_fwd_d128_kernel"
    assert lac.seq_kernel_name(True, "bf16", 64, 128) == "la_seq_bwd_d128_kernel"
    assert lac.seq_kernel_name(True, "bf16", 128, 128, "elu1") == "la_seq_bwd_d128_elu1_kernel"
    assert lac.seq_kernel_name(False, "bf16", 192, 128, "elu1") == "la_seq_fwd_d128_elu1_kernel"
    assert lac.seq_kernel_name(True, "bf16", 100, 128) is None
    assert lac.seq_supported("bf16", 8164, 128, 128) and lac.seq_supported("bf16", 1, 128, 64)
    assert not lac.seq_supported("bf16", 8164, 128, 100) and not lac.seq_supported("bf16", 16448, 128, 128)
    assert lac.seq_supported("bf16", 1 << 20, 64, 128) and not lac.seq_supported("bf16", (1 << 20) + 128, 64, 128)
    assert lac.seq_supported("bf16", 1000, 128, 128, "elu1")
    assert not lac.seq_supported("bf16", 1000, 64, 128, "elu1")


CE_WS = 1 << 30  # a fake workspace size large enough for every shape below


def ce_fwd_call(lib, N=512, d=1280, V=50257, dt=1, ws_bytes=CE_WS, **over):
    names = ["h", "W", "targets", "loss", "lse", "ws"]
    args = {n: addr(i) for i, n in enumerate(names)}
    args.update(over)
    return lib.la_ce_fwd(*[args[n] for n in names], ws_bytes, N, d, V, dt, None)


def ce_bwd_call(lib, N=512, d=1280, V=50257, chunk=0, dt=1, ws_bytes=CE_WS, **over):
    names = ["h", "W", "targets", "lse", "dloss", "dh", "dW", "ws"]
    args = {n: addr(i) for i, n in enumerate(names)}
    args.update(over)
    return lib.la_ce_bwd(*[args[n] for n in names], ws_bytes, N, d, V, chunk, dt, None)


@pytest.mark.parametrize("kw,status", [
    (dict(N=0), INVALID), (dict(V=1), INVALID), (dict(d=0), INVALID),
    (dict(d=1000), UNSUPPORTED), (dict(d=8192 + 128), UNSUPPORTED), (dict(dt=0), UNSUPPORTED),
    (dict(V=1 << 20), UNSUPPORTED),                      # V d beyond 32-bit byte offsets
    (dict(lse=None), INVALID), (dict(ws=None), INVALID),
    (dict(ws_bytes=1000), INVALID),                      # workspace too small
    (dict(h=ctypes.c_void_p(BASE + 8)), ALIGN),
    (dict(loss=addr(0)), ALIAS),                         # loss inside h
    (dict(ws=addr(1)), ALIAS),                           # workspace == W
])
def test_ce_fwd_rejects(lib, kw, status):
    assert ce_fwd_call(lib, **kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(N=-1), INVALID), (dict(d=64), UNSUPPORTED), (dict(dh=None), INVALID), (dict(dW=None), INVALID),
    (dict(ws_bytes=4096), INVALID), (dict(dW=addr(3)), ALIAS), (dict(dh=addr(5 + 1)), ALIAS),
    (dict(dloss=ctypes.c_void_p(BASE + 4 * STEP + 4)), ALIGN),
])
def test_ce_bwd_rejects(lib, kw, status):
    assert ce_bwd_call(lib, **kw) == status


def test_ce_workspace_sizes(lib):
    full = lac.ce_workspace_bytes(512, 1280, 50257)
    chunked = lac.ce_workspace_bytes(512, 1280, 50257, 128)
    # the backward's P of one chunk (bf16, padded to 128 x 128 tiles) and the dh partial sums
    assert full >= 512 * 50304 * 2 and chunked >= 128 * 50304 * 2 and chunked < full
    assert lac.ce_workspace_bytes(512, 100, 50257) == 0  # d not a multiple of 128
    # the forward needs its partial sums only: (V / 256 class tiles + 1) x N_pad x 8 bytes, the
    # same whatever the backward's chunk
    assert lac.ce_fwd_workspace_bytes(512, 1280, 50257) == (197 + 1) * 512 * 8
    assert lac.ce_fwd_workspace_bytes(512, 1280, 50257) < chunked


def test_ce_fwd_takes_shapes_whose_whole_p_would_not_fit(lib):
    # N x V_pad >= 2^30: the backward must chunk (a whole-N P is beyond 32-bit offsets), the
    # forward never forms P and takes the shape with its own small workspace
    N, d, V = 30000, 128, 50257
    fwd_ws = lac.ce_fwd_workspace_bytes(N, d, V)
    assert fwd_ws == (197 + 1) * 30080 * 8
    assert lac.ce_workspace_bytes(N, d, V) == 0
    assert lac.ce_workspace_bytes(N, d, V, 1024) > fwd_ws
    assert ce_fwd_call(lib, N=N, d=d, V=V, ws_bytes=fwd_ws - 1) == INVALID
    # with enough workspace every check before the overlap check passes (the workspace here
    # is placed on W, so the call stops there, before any launch)
    assert ce_fwd_call(lib, N=N, d=d, V=V, ws_bytes=fwd_ws, ws=addr(1)) == ALIAS
    assert ce_bwd_call(lib, N=N, d=d, V=V, chunk=0, ws_bytes=CE_WS) == UNSUPPORTED
    assert ce_bwd_call(lib, N=N, d=d, V=V, chunk=1024, ws_bytes=CE_WS, ws=addr(1)) == ALIAS


def test_ce_fwd_noalloc_limits(lib):
    names = ["h", "W", "targets", "loss", "lse"]
    call = lambda N, d=128, V=50257, **over: lib.la_ce_fwd_noalloc(
        *[over.get(n, addr(i)) for i, n in enumerate(names)], N, d, V, 1, None)
    limit = lac.CE_NOALLOC_SCRATCH_BYTES
    # the largest token count whose forward workspace fits the library's scratch at V = 50257
    fits = max(n for n in range(128, 8192, 128) if lac.ce_fwd_workspace_bytes(n, 128, 50257) <= limit)
    assert fits == 5248
    assert call(fits + 1) == UNSUPPORTED                   # beyond the scratch: refused before launch
    assert call(fits, lse=None) == INVALID
    assert call(fits, loss=addr(0)) == ALIAS               # checks pass up to the overlap check
    assert call(0) == INVALID and call(16, d=100) == UNSUPPORTED


def test_floor_launch_rejects(lib):
    # the measurement aid's host checks: kinds 0-4, buffer sizes per kind (512-thread and 128-thread
    # workgroups), alignment and overlap; nothing here reaches a launch
    call = lambda kind, nwg, ib, ob, i=addr(0), o=addr(1): lib.la_floor_launch(kind, nwg, i, ib, o, ob, None)
    per = {1: (65536, 32768), 2: (81920, 65536), 3: (16384, 8192), 4: (20480, 16384)}
    for kind, (pi, po) in per.items():
        assert call(kind, 160, pi * 160 - 1, po * 160) == INVALID   # input one byte short
        assert call(kind, 160, pi * 160, po * 160 - 1) == INVALID   # output one byte short
        assert call(kind, 160, pi * 160, po * 160, i=None) == INVALID
        assert call(kind, 160, pi * 160, po * 160, i=ctypes.c_void_p(BASE + 8)) == ALIGN
        assert call(kind, 160, pi * 160, po * 160, o=ctypes.c_void_p(BASE + 4096)) == ALIAS
    assert call(5, 160, 1 << 30, 1 << 30) == INVALID and call(-1, 160, 1 << 30, 1 << 30) == INVALID
    assert call(1, 0, 1 << 30, 1 << 30) == INVALID
    assert call(0, 160, 0, 512 * 4 - 1, i=None) == INVALID       # the empty kernel's never-written buffer
    assert lac.FLOOR_KINDS == {"empty": 0, "fwd": 1, "bwd": 2, "fwd_small": 3, "bwd_small": 4}


def test_time_next_launch_pairs(lib):
    assert lib.la_time_next_launch(addr(0), None) == INVALID
    assert lib.la_time_next_launch(None, addr(1)) == INVALID
    assert lib.la_time_next_launch(None, None) == OK
    # a pending request is taken by the next call even when that call is rejected
    assert lib.la_time_next_launch(addr(0), addr(1)) == OK
    assert fwd_call(lib, G=0) == INVALID
    assert lib.la_time_next_launch(None, None) == OK


def test_python_binding_rejects_cpu_tensors(lib):
    import torch
    q = torch.ones(2, 8, 64)
    with pytest.raises(ValueError):
        lac.fwd(q, q, q)


def test_autograd_rejects_host_tensors():
    import torch
    import causal_linear_attention_chunked_amd as lac
    x = torch.ones(1, 4, 64)
    with pytest.raises(ValueError, match="CUDA"):
        lac.linear_attention(x, x, x)
