"""Seeded synthetic inputs for chunked causal linear attention.

This module draws random numbers and packs them into tensors of the shapes the
Fractus-1B optimisation log ("Fractus-1B training optimization", section 1,
"Diagnosis") gives for its attention: G = B * 2 levels * 20 heads groups, C = 128
tokens per chunk, head dim 64, processing block 64.  It holds none of the
attention arithmetic.  Both the GPU path and the CPU oracle take their inputs
from here and from nowhere else.

Recipe, shared by every workload (one generator per workload, seeded):
  * fp32 standard-normal draws of whole-sequence tensors of shape (G, T, D),
    taken in this order: prior-chunk keys and values (only when the workload
    carries a state in), then q, k, v, then dO (only for a backward workload);
  * q and k are mapped to positive features with elu(x) + 1 (alpha = 1) in
    fp32, which is the feature map the workloads name; the attention itself
    never applies it;
  * everything is rounded to the workload dtype (round-to-nearest-even for
    bf16) after the map;
  * a carried-in state "from a prior random chunk" is built from that prior
    chunk's rounded keys and values: S_in = kp^T vp and z_in = kp^T 1, summed in
    fp64 and rounded once to fp32.  Both sides receive that same fp32 carry.

A sequence of T tokens per group is split into chunks by the list ``chunks``;
chunks are slices of one sequence, so a single call over T tokens and a chain
of calls over its chunks see identical tokens.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import torch

__all__ = ["Workload", "WORKLOADS", "make_inputs", "workload"]


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: sizes, dtype, carry recipe and direction."""

    name: str
    G: int
    chunks: tuple          # token count of each chunk, in order
    D: int
    dtype: str             # "f32" or "bf16"
    carry: str             # "zero" (no carry passed), "prior" (prior random chunk)
    backward: bool
    block: int = 64
    prior_len: int = 128   # tokens in the prior chunk that builds a "prior" carry
    seed: int = 0
    note: str = ""

    @property
    def T(self) -> int:
        return int(sum(self.chunks))


# The five workloads: a single-group fp32 forward, the headline G=160 chunk
# forward and forward+backward, a long batch of eight chained chunks, and a
# wide-head run with a ragged last chunk.  8192 tokens "in 128-token chunks with
# a last chunk of 100" cannot hold exactly; 63 full chunks plus a 100-token
# chunk (8164 tokens) is the reading used here.
WORKLOADS = {
    "g1_c128_d64_f32_fwd": Workload(
        "g1_c128_d64_f32_fwd", G=1, chunks=(128,), D=64, dtype="f32", carry="zero",
        backward=False, note="single group, fp32, forward only, zero carry"),
    "g160_c128_d64_bf16_fwd": Workload(
        "g160_c128_d64_bf16_fwd", G=160, chunks=(128,), D=64, dtype="bf16", carry="prior",
        backward=False, note="B=4 x 2 levels x 20 heads, carry from a prior random chunk"),
    "g160_c128_d64_bf16_fwdbwd": Workload(
        "g160_c128_d64_bf16_fwdbwd", G=160, chunks=(128,), D=64, dtype="bf16", carry="prior",
        backward=True, note="headline: forward + backward, carry from a prior random chunk"),
    "g1280_8x128_d64_bf16_fwdbwd": Workload(
        "g1280_8x128_d64_bf16_fwdbwd", G=1280, chunks=(128,) * 8, D=64, dtype="bf16",
        carry="zero", backward=True, note="B=32, eight chunks chained through the carry"),
    "g160_63x128p100_d128_bf16_fwdbwd": Workload(
        "g160_63x128p100_d128_bf16_fwdbwd", G=160, chunks=(128,) * 63 + (100,), D=128,
        dtype="bf16", carry="prior", prior_len=128, backward=True,
        note="wide heads, 8164 tokens, last chunk ragged (100 = 64 + 36)"),
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


def _torch_dtype(dtype: str) -> torch.dtype:
    if dtype == "f32":
        return torch.float32
    if dtype == "bf16":
        return torch.bfloat16
    raise ValueError(f"unknown dtype {dtype!r}")


def _feature(x: torch.Tensor) -> torch.Tensor:
    # elu(x) + 1 with alpha = 1, in fp32: strictly positive for every finite x.
    return torch.nn.functional.elu(x) + 1.0


def make_inputs(G: int, T: int, D: int, dtype: str = "bf16", carry: str = "zero",
                backward: bool = False, seed: int = 0, prior_len: int = 128,
                groups: Optional[List[int]] = None, features: str = "mapped") -> dict:
    """Draw one workload's tensors on the CPU.

    Returns a dict with ``q, k, v`` of shape (G, T, D) in the workload dtype,
    ``S_in`` (G, D, D) and ``z_in`` (G, D) in fp32 or ``None`` for a zero carry,
    and ``dO`` (G, T, D) for a backward workload.  ``groups`` keeps only the
    listed group rows after drawing the full tensors, so a sampled group holds
    exactly the values it holds in the full-size draw.  ``features="raw"`` leaves
    q and k as the normal draws (rounded to the dtype) for an op that applies
    elu(x) + 1 itself; the prior chunk's keys are mapped either way.
    """
    if carry not in ("zero", "prior"):
        raise ValueError(f"unknown carry recipe {carry!r}")
    if features not in ("mapped", "raw"):
        raise ValueError(f"unknown features option {features!r}")
    fmap = _feature if features == "mapped" else (lambda x: x)
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    tdt = _torch_dtype(dtype)

    def draw(t):
        return torch.randn((G, t, D), generator=gen, dtype=torch.float32)

    out = {}
    if carry == "prior":
        kp = _feature(draw(prior_len)).to(tdt)
        vp = draw(prior_len).to(tdt)
    q = fmap(draw(T)).to(tdt)
    k = fmap(draw(T)).to(tdt)
    v = draw(T).to(tdt)
    dO = draw(T).to(tdt) if backward else None

    sel = None if groups is None else torch.as_tensor(groups, dtype=torch.long)

    def pick(x):
        return x if (x is None or sel is None) else x.index_select(0, sel).contiguous()

    if carry == "prior":
        kp, vp = pick(kp), pick(vp)
        kp64 = kp.double()
        out["S_in"] = (kp64.transpose(1, 2) @ vp.double()).float().contiguous()
        out["z_in"] = kp64.sum(dim=1).float().contiguous()
    else:
        out["S_in"] = None
        out["z_in"] = None
    out["q"], out["k"], out["v"] = pick(q), pick(k), pick(v)
    out["dO"] = pick(dO)
    return out


def workload_inputs(w: Workload, groups: Optional[List[int]] = None, G: Optional[int] = None) -> dict:
    """Inputs for a named workload; ``G`` overrides the group count (same recipe)."""
    return make_inputs(G=w.G if G is None else G, T=w.T, D=w.D, dtype=w.dtype, carry=w.carry,
                       backward=w.backward, seed=w.seed, prior_len=w.prior_len, groups=groups)


def chunk_bounds(chunks) -> List[tuple]:
    """(start, end) token offsets of each chunk."""
    out, s = [], 0
    for c in chunks:
        out.append((s, s + int(c)))
        s += int(c)
    return out


# ---------------------------------------------------------------- cross-entropy over the tied head

@dataclass(frozen=True)
class CeWorkload:
    """One cross-entropy workload: N tokens of width d against a V-token tied head."""
    name: str
    N: int
    d: int
    V: int
    dtype: str = "bf16"
    w_std: float = 0.02   # the embedding's init scale
    seed: int = 0


# The head of "Fractus-1B training optimization" (Bottleneck #3): 50257 tokens, width 1280
# (its 64.3M head multiply-adds per token over the vocabulary), for the B = 4 batch of 128-token
# chunks whose fp32 logits are the page's 103 MB (4 x 128 x 50257 x 4 bytes).
CE_WORKLOADS = {
    "ce_n512_d1280_v50257_bf16": CeWorkload("ce_n512_d1280_v50257_bf16", N=512, d=1280, V=50257),
}


def ce_workload(name: str) -> CeWorkload:
    return CE_WORKLOADS[name]


def make_ce_inputs(N: int, d: int, V: int, dtype: str = "bf16", w_std: float = 0.02, seed: int = 0) -> dict:
    """Hidden states ``h`` (N, d) ~ N(0, 1), the tied embedding ``W`` (V, d) ~ N(0, w_std^2), both
    drawn in fp32 and rounded to the dtype, and ``targets`` (N,) int32 uniform over the vocabulary;
    drawn in that order from one seeded CPU generator."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    tdt = _torch_dtype(dtype)
    h = torch.randn((N, d), generator=gen, dtype=torch.float32).to(tdt)
    W = (torch.randn((V, d), generator=gen, dtype=torch.float32) * w_std).to(tdt)
    targets = torch.randint(0, V, (N,), generator=gen, dtype=torch.int64).to(torch.int32)
    return {"h": h, "W": W, "targets": targets}


def ce_workload_inputs(w: CeWorkload) -> dict:
    return make_ce_inputs(w.N, w.d, w.V, w.dtype, w.w_std, w.seed)
