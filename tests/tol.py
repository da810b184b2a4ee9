"""Parity tolerance used by every comparison against the fp64 oracle.

Per output tensor, elementwise:  |x - r| <= rtol * (|r| + rms(r)),  r the fp64
oracle value and rms taken over that tensor.  rtol is 1e-4 for fp32 inputs and
2e-2 for bf16 inputs.  The normwise relative error ||x - r|| / ||r|| is reported
alongside.
"""
import numpy as np

RTOL = {"f32": 1e-4, "bf16": 2e-2}


def as_f64(x):
    if hasattr(x, "detach"):
        import torch
        return x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def check(name, got, ref, rtol):
    """Raise AssertionError with a useful message if ``got`` is outside tolerance of ``ref``."""
    g, r = as_f64(got), as_f64(ref)
    assert g.shape == r.shape, f"{name}: shape {g.shape} != {r.shape}"
    assert np.all(np.isfinite(g)), f"{name}: non-finite values ({np.sum(~np.isfinite(g))})"
    rms = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    err = np.abs(g - r)
    bound = rtol * (np.abs(r) + rms)
    bad = err > bound
    nrm = float(np.linalg.norm(r))
    normwise = float(np.linalg.norm(g - r)) / nrm if nrm > 0 else float(np.linalg.norm(g - r))
    if np.any(bad):
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(
            f"{name}: {int(bad.sum())}/{bad.size} elements out of tolerance (rtol={rtol}); "
            f"worst at {tuple(int(x) for x in i)}: got {g[i]!r} ref {r[i]!r} "
            f"(bound {bound[i]:.3g}); normwise rel err {normwise:.3g}")
    return normwise
