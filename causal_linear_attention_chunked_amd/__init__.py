"""Chunked causal linear attention with a carried state on AMD MI355X (gfx950).

Python binding of the C ABI in ``include/la_chunk.h`` (library ``liblachunk.so``
in this directory, built by ``python -m causal_linear_attention_chunked_amd.build``).
The binding only marshals arguments: every step of the computation runs in the
library's HIP kernels, and importing or calling it without the built library
raises.  PyTorch supplies device memory and the current stream.

    o, S_out, z_out = fwd(q, k, v, S_in=None, z_in=None)
    dq, dk, dv, dS_in, dz_in = bwd(q, k, v, S_in, z_in, dO, dS_out=None, dz_out=None)
    o, S_out, z_out = seq_fwd(q, k, v, S_in, z_in, chunk=128)     # (G, T, D): all chunks, one launch
    dq, dk, dv, dS_in, dz_in = seq_bwd(q, k, v, S_out, z_out, dO)   # from the final carry
    time_next_launch(start_event, stop_event)   # kernel-only timing of the next call
    o, (S_out, z_out) = linear_attention(q, k, v, S_in, z_in, chunk=128)   # differentiable (autograd)
    loss, lse = ce_fwd(h, W, targets)                   # cross-entropy over a tied head
    dh, dW = ce_bwd(h, W, targets, lse, dloss=None, ce_chunk=0)
    loss = chunked_cross_entropy(h, W, targets, ce_chunk)  # differentiable (autograd)

q, k, v, dO: contiguous (G, C, D) (one chunk) or (G, T, D) (a sequence) CUDA
tensors, float32 or bfloat16 (one dtype for all); S: (G, D, D) float32 with S[p][c] (p key feature, c value feature);
z: (G, D) float32.  See the header for the operation and its rules.
"""
from __future__ import annotations

import ctypes
import os
import threading

__all__ = ["fwd", "bwd", "seq_fwd", "seq_bwd", "seq_supported", "seq_kernel_name", "chain_fwd", "chain_bwd", "linear_attention", "chunk_attention", "ChunkFunction", "LachunkError", "lib_path", "load_library",
           "abi_version", "status_str", "time_next_launch", "kernel_name", "BWD_MAX_C", "ce_fwd", "ce_bwd",
           "ce_workspace_bytes", "ce_fwd_workspace_bytes", "chunked_cross_entropy", "set_attention_impl", "get_attention_impl", "IMPLS"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liblachunk.so")
_lock = threading.Lock()
_lib = None

LA_F32, LA_BF16 = 0, 1
BWD_MAX_C = 2048
_STATUS = {0: "LA_OK", 1: "LA_ERR_INVALID", 2: "LA_ERR_UNSUPPORTED", 3: "LA_ERR_ALIGN",
           4: "LA_ERR_ALIAS", 5: "LA_ERR_LAUNCH"}


class LachunkError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn}: {_STATUS.get(status, status)}: {msg}")
        self.status = status


def lib_path() -> str:
    return _LIB_PATH


def load_library():
    """Load liblachunk.so; raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                               "`python -m causal_linear_attention_chunked_amd.build`")
        lib = ctypes.CDLL(_LIB_PATH)
        vp, i = ctypes.c_void_p, ctypes.c_int
        lib.la_chunk_fwd.restype = i
        lib.la_chunk_fwd.argtypes = [vp] * 8 + [i] * 6 + [vp]
        lib.la_chunk_bwd.restype = i
        lib.la_chunk_bwd.argtypes = [vp] * 13 + [i] * 6 + [vp]
        lib.la_status_str.restype = ctypes.c_char_p
        lib.la_status_str.argtypes = [i]
        lib.la_abi_version.restype = i
        lib.la_abi_version.argtypes = []
        lib.la_time_next_launch.restype = i
        lib.la_time_next_launch.argtypes = [vp, vp]
        lib.la_kernel_name.restype = ctypes.c_char_p
        lib.la_kernel_name.argtypes = [i] * 6
        lib.la_seq_fwd.restype = i
        lib.la_seq_fwd.argtypes = [vp] * 10 + [i] * 7 + [vp]
        lib.la_seq_bwd.restype = i
        lib.la_seq_bwd.argtypes = [vp] * 15 + [i] * 7 + [vp]
        lib.la_ce_workspace_bytes.restype = ctypes.c_size_t
        lib.la_ce_workspace_bytes.argtypes = [i] * 4
        lib.la_ce_fwd_workspace_bytes.restype = ctypes.c_size_t
        lib.la_ce_fwd_workspace_bytes.argtypes = [i] * 3
        lib.la_ce_fwd.restype = i
        lib.la_ce_fwd.argtypes = [vp] * 6 + [ctypes.c_size_t] + [i] * 4 + [vp]
        lib.la_ce_bwd.restype = i
        lib.la_ce_bwd.argtypes = [vp] * 8 + [ctypes.c_size_t] + [i] * 5 + [vp]
        lib.la_seq_kernel_name.restype = ctypes.c_char_p
        lib.la_seq_kernel_name.argtypes = [i, i, i, i, i]
        lib.la_ce_fwd_noalloc.restype = i
        lib.la_ce_fwd_noalloc.argtypes = [vp] * 5 + [i] * 4 + [vp]
        lib.la_floor_launch.restype = i
        lib.la_floor_launch.argtypes = [i, i, vp, ctypes.c_size_t, vp, ctypes.c_size_t, vp]
        _lib = lib
        return lib


def abi_version() -> int:
    return int(load_library().la_abi_version())


def status_str(s: int) -> str:
    return load_library().la_status_str(int(s)).decode()


def _dt_code(dtype):
    return LA_BF16 if str(dtype).replace("torch.", "") in ("bf16", "bfloat16") else LA_F32


FEATURES = {None: 0, "none": 0, "elu1": 1}


def _feature_code(feature):
    if feature not in FEATURES:
        raise ValueError(f"unknown feature map {feature!r}; use None or 'elu1'")
    return FEATURES[feature]


def kernel_name(backward: bool, dtype, C: int, D: int, block: int = 64, feature=None):
    """Name of the kernel a fwd (backward=False) or bwd call launches for this element type
    ("bf16"/"float32" or a torch dtype), chunk length, head dimension, block (64: the blocked
    form, 1: the cumsum form) and feature map; None if unsupported."""
    name = load_library().la_kernel_name(int(bool(backward)), _dt_code(dtype), int(C), int(D), int(block),
                                         _feature_code(feature))
    return None if name is None else name.decode()


def seq_kernel_name(backward: bool, dtype, chunk: int, D: int, feature=None):
    """Name of the kernel seq_fwd / seq_bwd launch for this element type, chunk length, D and
    feature map."""
    name = load_library().la_seq_kernel_name(int(bool(backward)), _dt_code(dtype), int(chunk), int(D),
                                             _feature_code(feature))
    return None if name is None else name.decode()


SEQ_D64_MAX_T = 1 << 20    # LA_SEQ_D64_MAX_T
SEQ_D128_MAX_T = 16384     # LA_SEQ_D128_MAX_T


def seq_supported(dtype, T: int, D: int, chunk: int, feature=None) -> bool:
    """Whether seq_fwd / seq_bwd take a (G, T, D) sequence in chunks of ``chunk`` tokens:
    bf16, and either D = 64 with 128-token chunks, whole chunks only (T up to SEQ_D64_MAX_T), or
    D = 128 with chunks a multiple of 64 tokens, the last one possibly shorter, T up to
    SEQ_D128_MAX_T; either with or without the fused feature map."""
    if _dt_code(dtype) != LA_BF16 or T < 1:
        return False
    if D == 64:
        return chunk == 128 and T % chunk == 0 and T <= SEQ_D64_MAX_T
    if D == 128:
        _feature_code(feature)  # raises for an unknown feature map
        return chunk >= 64 and chunk % 64 == 0 and T <= SEQ_D128_MAX_T
    return False


def time_next_launch(start_event, stop_event):
    """Have the next fwd/bwd call on this thread record two ``torch.cuda.Event``
    (created with ``enable_timing=True``) on its kernel dispatch itself, so that
    ``start_event.elapsed_time(stop_event)`` is the kernel's own duration."""
    evs = []
    for e in (start_event, stop_event):
        if e.cuda_event == 0:  # torch creates the underlying event on first record
            e.record()
        evs.append(ctypes.c_void_p(e.cuda_event))
    _check("la_time_next_launch", load_library().la_time_next_launch(*evs))


def _ptr(t):
    # ctypes passes a Python int or None for a c_void_p argument
    return None if t is None else t.data_ptr()


def _check(fn, status):
    if status != 0:
        raise LachunkError(fn, status, status_str(status))


def _dtype_code(t):
    import torch
    if t.dtype == torch.float32:
        return LA_F32
    if t.dtype == torch.bfloat16:
        return LA_BF16
    raise TypeError(f"unsupported element type {t.dtype}; use float32 or bfloat16")


def _validate_tokens(names, tensors):
    """(G, C, D, device index) of the token tensors, which must agree in shape, dtype and device
    and be contiguous CUDA tensors.  The common case costs a few attribute reads per tensor."""
    ref = tensors[0]
    shape, dtype, dev = ref.shape, ref.dtype, ref.get_device()
    if len(shape) == 3 and dev >= 0:
        for t in tensors:
            if t.get_device() != dev or t.dtype is not dtype or t.shape != shape or not t.is_contiguous():
                break
        else:
            return shape[0], shape[1], shape[2], dev
    if ref.dim() != 3:
        raise ValueError(f"{names[0]} must be (G, C, D), got {tuple(ref.shape)}")
    for n, t in zip(names, tensors):
        if not t.is_cuda:
            raise ValueError(f"{n} must be a CUDA tensor")
        if t.shape != ref.shape or t.dtype != ref.dtype or t.device != ref.device:
            raise ValueError(f"{n}: shape/dtype/device {tuple(t.shape)}/{t.dtype}/{t.device} differs from "
                             f"{names[0]} {tuple(ref.shape)}/{ref.dtype}/{ref.device}")
        if not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous")
    raise AssertionError("unreachable")


def _validate_state(name, t, shape, dev):
    import torch
    if t is None:
        return
    if t.dtype is not torch.float32 or t.shape != shape or t.get_device() != dev or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous float32 tensor of shape {shape} on cuda:{dev}")


def _validate_outputs(names, tokens, states, ref, G, D, dev):
    """Caller-supplied output tensors: `tokens` like `ref` (shape, dtype, device, contiguous),
    `states` fp32 (G, D, D) then (G, D) pairs.  The library can check only alignment and
    overlap, so a wrong buffer here would be written out of bounds."""
    nt = len(tokens)
    for n, t in zip(names[:nt], tokens):
        if t is None:
            raise ValueError(f"out: {n} is missing")
        _validate_tokens(("the inputs", n), (ref, t))
    for j, (n, t) in enumerate(zip(names[nt:], states)):
        if t is None:
            raise ValueError(f"out: {n} is missing")
        _validate_state(n, t, (G, D, D) if j % 2 == 0 else (G, D), dev)


def _stream(dev):
    """Raw handle of the current stream on device index ``dev``."""
    import torch
    return torch._C._cuda_getCurrentRawStream(dev)


def fwd(q, k, v, S_in=None, z_in=None, block: int = 64, out=None, feature=None):
    """Forward over one chunk: returns (o, S_out, z_out).  ``out`` may supply them.  ``block``:
    64, the blocked (chunked) form; 1, the cumsum form (the per-token recurrence).
    ``feature="elu1"``: q, k are raw inputs and elu(x) + 1 is applied inside."""
    lib = _lib or load_library()
    G, C, D, dev = _validate_tokens(("q", "k", "v"), (q, k, v))
    if (S_in is None) != (z_in is None):
        raise ValueError("S_in and z_in must be given together")
    _validate_state("S_in", S_in, (G, D, D), dev)
    _validate_state("z_in", z_in, (G, D), dev)
    if out is None:
        import torch
        o = torch.empty_like(q)
        S_out = torch.empty((G, D, D), dtype=torch.float32, device=q.device)
        z_out = torch.empty((G, D), dtype=torch.float32, device=q.device)
    else:
        o, S_out, z_out = out
        _validate_outputs(("o", "S_out", "z_out"), (o,), (S_out, z_out), q, G, D, dev)
    _check("la_chunk_fwd", lib.la_chunk_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), _ptr(S_in), _ptr(z_in),
                                            o.data_ptr(), S_out.data_ptr(), z_out.data_ptr(), G, C, D, int(block),
                                            _feature_code(feature), _dtype_code(q), _stream(dev)))
    return o, S_out, z_out


def bwd(q, k, v, S_in, z_in, dO, dS_out=None, dz_out=None, block: int = 64, out=None, feature=None):
    """Backward over one chunk: returns (dq, dk, dv, dS_in, dz_in); ``block`` and ``feature`` as
    in ``fwd`` (with the map, dq and dk are the gradients of the raw inputs)."""
    lib = _lib or load_library()
    G, C, D, dev = _validate_tokens(("q", "k", "v", "dO"), (q, k, v, dO))
    if (S_in is None) != (z_in is None) or (dS_out is None) != (dz_out is None):
        raise ValueError("S_in/z_in and dS_out/dz_out must each be given together")
    _validate_state("S_in", S_in, (G, D, D), dev)
    _validate_state("z_in", z_in, (G, D), dev)
    _validate_state("dS_out", dS_out, (G, D, D), dev)
    _validate_state("dz_out", dz_out, (G, D), dev)
    if out is None:
        import torch
        dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
        dS_in = torch.empty((G, D, D), dtype=torch.float32, device=q.device)
        dz_in = torch.empty((G, D), dtype=torch.float32, device=q.device)
    else:
        dq, dk, dv, dS_in, dz_in = out
        _validate_outputs(("dq", "dk", "dv", "dS_in", "dz_in"), (dq, dk, dv), (dS_in, dz_in), q, G, D, dev)
    _check("la_chunk_bwd", lib.la_chunk_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), _ptr(S_in), _ptr(z_in),
                                            dO.data_ptr(), _ptr(dS_out), _ptr(dz_out), dq.data_ptr(),
                                            dk.data_ptr(), dv.data_ptr(), dS_in.data_ptr(), dz_in.data_ptr(),
                                            G, C, D, int(block), _feature_code(feature), _dtype_code(q),
                                            _stream(dev)))
    return dq, dk, dv, dS_in, dz_in


def seq_fwd(q, k, v, S_in=None, z_in=None, chunk: int = 128, block: int = 64, out=None, feature=None,
            residual: bool = False):
    """Forward over a whole (G, T, D) sequence of chunks in one launch, carry on chip:
    returns (o, S_out, z_out), equal to chaining fwd over the chunks.  ``feature="elu1"``
    takes raw q, k and applies elu(x) + 1 inside.  ``residual=True`` also returns the final
    carry's remainders (S_res, z_res): its exact value is S_out + S_res, z_out + z_res, and
    seq_bwd takes them to recover the early states accurately."""
    lib = _lib or load_library()
    G, T, D, dev = _validate_tokens(("q", "k", "v"), (q, k, v))
    if (S_in is None) != (z_in is None):
        raise ValueError("S_in and z_in must be given together")
    _validate_state("S_in", S_in, (G, D, D), dev)
    _validate_state("z_in", z_in, (G, D), dev)
    if out is None:
        import torch
        o = torch.empty_like(q)
        S_out = torch.empty((G, D, D), dtype=torch.float32, device=q.device)
        z_out = torch.empty((G, D), dtype=torch.float32, device=q.device)
        S_res = torch.empty((G, D, D), dtype=torch.float32, device=q.device) if residual else None
        z_res = torch.empty((G, D), dtype=torch.float32, device=q.device) if residual else None
    else:
        o, S_out, z_out, S_res, z_res = out if residual else (*out, None, None)
        _validate_outputs(("o", "S_out", "z_out"), (o,), (S_out, z_out), q, G, D, dev)
        if residual:
            _validate_outputs(("S_res", "z_res"), (), (S_res, z_res), q, G, D, dev)
    _check("la_seq_fwd", lib.la_seq_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), _ptr(S_in), _ptr(z_in),
                                        o.data_ptr(), S_out.data_ptr(), z_out.data_ptr(), _ptr(S_res), _ptr(z_res),
                                        G, T, D, int(chunk), int(block), _feature_code(feature), _dtype_code(q),
                                        _stream(dev)))
    return (o, S_out, z_out, S_res, z_res) if residual else (o, S_out, z_out)


def seq_bwd(q, k, v, S_last, z_last, dO, dS_out=None, dz_out=None, chunk: int = 128, block: int = 64, out=None,
            feature=None, S_res=None, z_res=None):
    """Backward over a whole sequence in one launch, last chunk first, reverse state on chip.
    (S_last, z_last) is the carry after the last chunk: seq_fwd's (S_out, z_out); (S_res,
    z_res), optional, its remainders from seq_fwd(..., residual=True).
    Returns (dq, dk, dv, dS_in, dz_in); with ``feature="elu1"`` dq and dk are the gradients
    of the raw inputs."""
    lib = _lib or load_library()
    G, T, D, dev = _validate_tokens(("q", "k", "v", "dO"), (q, k, v, dO))
    if S_last is None or z_last is None:
        raise ValueError("S_last and z_last (the forward's final carry) are required")
    if (dS_out is None) != (dz_out is None):
        raise ValueError("dS_out and dz_out must be given together")
    _validate_state("S_last", S_last, (G, D, D), dev)
    _validate_state("z_last", z_last, (G, D), dev)
    _validate_state("dS_out", dS_out, (G, D, D), dev)
    _validate_state("dz_out", dz_out, (G, D), dev)
    if (S_res is None) != (z_res is None):
        raise ValueError("S_res and z_res must be given together")
    _validate_state("S_res", S_res, (G, D, D), dev)
    _validate_state("z_res", z_res, (G, D), dev)
    if out is None:
        import torch
        dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
        dS_in = torch.empty((G, D, D), dtype=torch.float32, device=q.device)
        dz_in = torch.empty((G, D), dtype=torch.float32, device=q.device)
    else:
        dq, dk, dv, dS_in, dz_in = out
        _validate_outputs(("dq", "dk", "dv", "dS_in", "dz_in"), (dq, dk, dv), (dS_in, dz_in), q, G, D, dev)
    _check("la_seq_bwd", lib.la_seq_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), S_last.data_ptr(),
                                        z_last.data_ptr(), _ptr(S_res), _ptr(z_res), dO.data_ptr(), _ptr(dS_out),
                                        _ptr(dz_out),
                                        dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), dS_in.data_ptr(),
                                        dz_in.data_ptr(), G, T, D, int(chunk), int(block), _feature_code(feature),
                                        _dtype_code(q), _stream(dev)))
    return dq, dk, dv, dS_in, dz_in


def ce_workspace_bytes(N: int, d: int, V: int, ce_chunk: int = 0) -> int:
    """Bytes of device workspace ce_bwd needs at this chunk, enough for ce_fwd too, so one
    buffer serves both (0: shape not supported)."""
    return int(load_library().la_ce_workspace_bytes(int(N), int(d), int(V), int(ce_chunk)))


def ce_fwd_workspace_bytes(N: int, d: int, V: int) -> int:
    """Bytes of device workspace ce_fwd needs: its per-tile partial sums, no logits (0: shape not
    supported)."""
    return int(load_library().la_ce_fwd_workspace_bytes(int(N), int(d), int(V)))


def _ce_check(h, W, targets):
    import torch
    for n, t in (("h", h), ("W", W), ("targets", targets)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{n} must be a contiguous CUDA tensor")
    if h.dim() != 2 or W.dim() != 2 or h.shape[1] != W.shape[1]:
        raise ValueError(f"h (N, d) and W (V, d) expected, got {tuple(h.shape)} and {tuple(W.shape)}")
    if h.dtype is not torch.bfloat16 or W.dtype is not torch.bfloat16:
        raise ValueError("h and W must be bfloat16")
    if targets.dtype is not torch.int32 or targets.shape != (h.shape[0],):
        raise ValueError("targets must be int32 of shape (N,)")
    if h.device != W.device or h.device != targets.device:
        raise ValueError("h, W and targets must be on one device")
    return h.shape[0], h.shape[1], W.shape[0], h.get_device()


def _workspace(ws, nbytes, dev):
    import torch
    if ws is None:
        return torch.empty(max(nbytes, 16), dtype=torch.uint8, device=f"cuda:{dev}")
    if ws.get_device() != dev or not ws.is_contiguous():
        raise ValueError(f"workspace must be a contiguous tensor on cuda:{dev}")
    if ws.numel() * ws.element_size() < nbytes:
        raise ValueError(f"workspace of {ws.numel() * ws.element_size()} bytes, {nbytes} needed")
    return ws


def _ce_f32(name, t, shape, dev):
    """A float32 tensor of `shape` on cuda:dev, contiguous (a scalar may be 0-dim or one element)."""
    import torch
    ok = (t is not None and t.dtype is torch.float32 and t.get_device() == dev and t.is_contiguous()
          and (tuple(t.shape) == shape or (shape == () and t.numel() == 1)))
    if not ok:
        what = "scalar" if shape == () else f"tensor of shape {shape}"
        raise ValueError(f"{name} must be a contiguous float32 {what} on cuda:{dev}")


def ce_fwd(h, W, targets, workspace=None, out=None):
    """Mean cross-entropy of the tied head W (V, d) over the tokens h (N, d) with int32 targets:
    returns (loss, lse), a 0-dim float32 tensor and (N,) float32.  The logits are never stored."""
    import torch
    lib = _lib or load_library()
    N, d, V, dev = _ce_check(h, W, targets)
    nbytes = ce_fwd_workspace_bytes(N, d, V)
    if nbytes == 0:
        raise LachunkError("la_ce_fwd", 2, status_str(2))
    ws = _workspace(workspace, nbytes, dev)
    if out is None:
        loss = torch.empty((), dtype=torch.float32, device=h.device)
        lse = torch.empty((N,), dtype=torch.float32, device=h.device)
    else:
        loss, lse = out
        _ce_f32("loss", loss, (), dev)
        _ce_f32("lse", lse, (N,), dev)
    _check("la_ce_fwd", lib.la_ce_fwd(h.data_ptr(), W.data_ptr(), targets.data_ptr(), loss.data_ptr(),
                                      lse.data_ptr(), ws.data_ptr(), nbytes, N, d, V, LA_BF16, _stream(dev)))
    return loss, lse


CE_NOALLOC_SCRATCH_BYTES = 8 << 20  # LA_CE_NOALLOC_SCRATCH_BYTES


def ce_fwd_noalloc(h, W, targets, out):
    """ce_fwd for callers that cannot allocate: the library's own static per-device scratch is the
    workspace, and the caller passes the outputs ``out = (loss, lse)``; nothing is allocated.
    Calls that overlap on one device race on that scratch.  Shapes whose forward workspace
    exceeds CE_NOALLOC_SCRATCH_BYTES raise (LA_ERR_UNSUPPORTED)."""
    lib = _lib or load_library()
    N, d, V, dev = _ce_check(h, W, targets)
    loss, lse = out
    _ce_f32("loss", loss, (), dev)
    _ce_f32("lse", lse, (N,), dev)
    st = lib.la_ce_fwd_noalloc(h.data_ptr(), W.data_ptr(), targets.data_ptr(), loss.data_ptr(), lse.data_ptr(),
                               N, d, V, LA_BF16, _stream(dev))
    if st == 2 and ce_fwd_workspace_bytes(N, d, V) > CE_NOALLOC_SCRATCH_BYTES:
        raise LachunkError("la_ce_fwd_noalloc", st,
                           f"{status_str(st)}: its workspace of {ce_fwd_workspace_bytes(N, d, V)} bytes exceeds the "
                           f"library's scratch of {CE_NOALLOC_SCRATCH_BYTES}")
    _check("la_ce_fwd_noalloc", st)
    return loss, lse


def ce_bwd(h, W, targets, lse, dloss=None, ce_chunk: int = 0, workspace=None, out=None):
    """Gradients of dloss * loss (dloss a float32 CUDA scalar, None = 1) with respect to h and W:
    returns (dh bf16 (N, d), dW float32 (V, d)).  The logits are recomputed ``ce_chunk`` tokens at
    a time (0: all at once), each chunk's softmax kept in bf16 only while its products run."""
    import torch
    lib = _lib or load_library()
    N, d, V, dev = _ce_check(h, W, targets)
    _ce_f32("lse", lse, (N,), dev)
    if dloss is not None:
        _ce_f32("dloss", dloss, (), dev)
    nbytes = ce_workspace_bytes(N, d, V, ce_chunk)
    if nbytes == 0:
        raise LachunkError("la_ce_bwd", 2, status_str(2))
    ws = _workspace(workspace, nbytes, dev)
    if out is None:
        dh = torch.empty_like(h)
        dW = torch.empty((V, d), dtype=torch.float32, device=h.device)
    else:
        dh, dW = out
        if (dh is None or dh.dtype is not torch.bfloat16 or dh.shape != h.shape or dh.get_device() != dev
                or not dh.is_contiguous()):
            raise ValueError(f"out: dh must be a contiguous bfloat16 tensor of shape {tuple(h.shape)} on cuda:{dev}")
        _ce_f32("dW", dW, (V, d), dev)
    _check("la_ce_bwd", lib.la_ce_bwd(h.data_ptr(), W.data_ptr(), targets.data_ptr(), lse.data_ptr(), _ptr(dloss),
                                      dh.data_ptr(), dW.data_ptr(), ws.data_ptr(), nbytes, N, d, V, int(ce_chunk),
                                      LA_BF16, _stream(dev)))
    return dh, dW


FLOOR_KINDS = {"empty": 0, "fwd": 1, "bwd": 2, "fwd_small": 3, "bwd_small": 4}
FLOOR_NAMES = {0: "la_floor_empty_kernel", 1: "la_floor_stream_kernel<8, 4, 512>", 2: "la_floor_stream_kernel<10, 8, 512>",
               3: "la_floor_stream_kernel<8, 4, 128>", 4: "la_floor_stream_kernel<10, 8, 128>"}


def floor_launch(kind: str, nwg: int, inp, out):
    """Measurement aid: one launch-floor kernel (no arithmetic) of ``nwg`` workgroups on the
    current stream.  kind "empty", or "fwd" / "bwd": every workgroup reads 65536 / 81920 bytes of
    ``inp`` and writes 32768 / 65536 bytes of ``out`` (contiguous CUDA tensors, any dtype);
    "fwd_small" / "bwd_small": a quarter of that per workgroup (128 threads instead of 512)."""
    lib = _lib or load_library()
    if kind not in FLOOR_KINDS:
        raise ValueError(f"unknown floor kind {kind!r}; use one of {sorted(FLOOR_KINDS)}")
    if not out.is_cuda or not out.is_contiguous() or (inp is not None and (not inp.is_cuda or not inp.is_contiguous())):
        raise ValueError("floor buffers must be contiguous CUDA tensors")
    nb = lambda t: 0 if t is None else t.numel() * t.element_size()
    _check("la_floor_launch", lib.la_floor_launch(FLOOR_KINDS[kind], int(nwg), _ptr(inp), nb(inp), out.data_ptr(),
                                                  nb(out), _stream(out.get_device())))


def chain_fwd(q_chunks, k_chunks, v_chunks, S_in=None, z_in=None, block: int = 64):
    """Forward over consecutive chunks (lists of (G, C_i, D) tensors), carrying (S, z).

    Returns (list of o chunks, list of (S_in_i, z_in_i) that fed each chunk, (S_out, z_out)).
    The per-chunk carries are what ``chain_bwd`` needs; they stay on the device."""
    outs, carries = [], []
    S, z = S_in, z_in
    for qc, kc, vc in zip(q_chunks, k_chunks, v_chunks):
        carries.append((S, z))
        o, S, z = fwd(qc, kc, vc, S, z, block)
        outs.append(o)
    return outs, carries, (S, z)


def chain_bwd(q_chunks, k_chunks, v_chunks, carries, dO_chunks, dS_out=None, dz_out=None, block: int = 64):
    """Backward over consecutive chunks, last chunk first, passing (dS, dz) down the chain.

    Returns (dq chunks, dk chunks, dv chunks, dS_in, dz_in) for the whole sequence."""
    n = len(q_chunks)
    dqs, dks, dvs = [None] * n, [None] * n, [None] * n
    gS, gz = dS_out, dz_out
    for i in range(n - 1, -1, -1):
        S, z = carries[i]
        dqs[i], dks[i], dvs[i], gS, gz = bwd(q_chunks[i], k_chunks[i], v_chunks[i], S, z, dO_chunks[i],
                                             gS, gz, block)
    return dqs, dks, dvs, gS, gz


def __getattr__(name):
    # the autograd layer imports torch; load it on first use
    if name in ("linear_attention", "chunk_attention", "ChunkFunction", "chunked_cross_entropy",
                "set_attention_impl", "get_attention_impl", "IMPLS"):
        from . import autograd
        return getattr(autograd, name)
    raise AttributeError(f"module {__name__!r} has no attribute {name!r}")
