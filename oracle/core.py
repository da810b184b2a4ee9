"""ctypes front end of the fp64 C oracle (``la_oracle.c``).

TEST INFRASTRUCTURE ONLY (see the package docstring).

``fwd`` and ``bwd`` take numpy or torch CPU arrays of any float dtype, upcast
them exactly to fp64, and return fp64 numpy arrays.  The C code is the plain
definition of "Fractus-1B training optimization", section 1, Bottleneck #1
(state as a prefix sum of k v^T, inclusive of the current token) and the
reverse cumsum the same section gives for the backward.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "la_oracle.c")
_LIB = os.path.join(_HERE, "liblaoracle.so")
_lock = threading.Lock()
_lib = None


def lib_path() -> str:
    return _LIB


def build(force: bool = True) -> str:
    """Compile ``la_oracle.c`` with gcc (-O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", _SRC, "-o", tmp]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB):
                build(force=True)
            lib = ctypes.CDLL(_LIB)
            dp = ctypes.POINTER(ctypes.c_double)
            lib.la_oracle_fwd.restype = ctypes.c_int
            lib.la_oracle_fwd.argtypes = [ctypes.c_int] * 3 + [dp] * 8 + [ctypes.c_int]
            lib.la_oracle_bwd.restype = ctypes.c_int
            lib.la_oracle_bwd.argtypes = [ctypes.c_int] * 3 + [dp] * 13 + [ctypes.c_int]
            lib.la_oracle_max_threads.restype = ctypes.c_int
            _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().la_oracle_max_threads())


def _f64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor (bf16 has no numpy dtype: upcast in torch first)
        import torch
        x = x.detach().to("cpu", torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    if a is None:
        return ctypes.POINTER(ctypes.c_double)()
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def fwd(q, k, v, S_in=None, z_in=None, nthreads: int = 0):
    """Forward over the whole (G, T, D) sequence; returns (o, S_out, z_out) in fp64."""
    q, k, v, S_in, z_in = map(_f64, (q, k, v, S_in, z_in))
    G, T, D = q.shape
    assert k.shape == q.shape and v.shape == q.shape
    o = np.empty((G, T, D))
    S_out = np.empty((G, D, D))
    z_out = np.empty((G, D))
    rc = _load().la_oracle_fwd(G, T, D, _ptr(q), _ptr(k), _ptr(v), _ptr(S_in), _ptr(z_in),
                               _ptr(o), _ptr(S_out), _ptr(z_out), int(nthreads))
    if rc == 2:
        raise FloatingPointError("oracle: a denominator q_t . z_t was not > 0")
    if rc != 0:
        raise ValueError(f"oracle: la_oracle_fwd returned {rc}")
    return o, S_out, z_out


def bwd(q, k, v, S_in, z_in, dO, dS_out=None, dz_out=None, nthreads: int = 0):
    """Backward; returns (dq, dk, dv, dS_in, dz_in) in fp64."""
    q, k, v, S_in, z_in, dO, dS_out, dz_out = map(_f64, (q, k, v, S_in, z_in, dO, dS_out, dz_out))
    G, T, D = q.shape
    dq = np.empty((G, T, D))
    dk = np.empty((G, T, D))
    dv = np.empty((G, T, D))
    dS_in = np.empty((G, D, D))
    dz_in = np.empty((G, D))
    rc = _load().la_oracle_bwd(G, T, D, _ptr(q), _ptr(k), _ptr(v), _ptr(S_in), _ptr(z_in), _ptr(dO),
                               _ptr(dS_out), _ptr(dz_out), _ptr(dq), _ptr(dk), _ptr(dv),
                               _ptr(dS_in), _ptr(dz_in), int(nthreads))
    if rc == 2:
        raise FloatingPointError("oracle: a denominator q_t . z_t was not > 0")
    if rc != 0:
        raise ValueError(f"oracle: la_oracle_bwd returned {rc}")
    return dq, dk, dv, dS_in, dz_in

