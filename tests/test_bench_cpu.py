"""Host-side checks of bench.py's byte accounting (no GPU)."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from causal_linear_attention_chunked_amd import inputs as inp  # noqa: E402


def _bytes(name):
    w = inp.workload(name)
    esz = 2 if w.dtype == "bf16" else 4
    return bench.plan_launches(w.G, w.chunks, w.D, esz, w.carry != "zero")


def test_headline_bytes():
    # G=160, C=128, D=64, bf16 tokens, fp32 carry in and out: 4 token streams + 2 carries forward,
    # 7 token streams + 2 carries backward
    L = _bytes("g160_c128_d64_bf16_fwdbwd")
    assert [k for k, *_ in L] == ["fwd", "bwd"]
    tok, carry = 160 * 128 * 64 * 2, 160 * (64 * 64 + 64) * 4
    assert L[0][2] == 4 * tok + 2 * carry
    assert L[1][2] == 7 * tok + 2 * carry
    assert sum(b for *_, b, _ in L) == pytest.approx(39.485e6, rel=1e-4)


def test_chained_launch_order_and_carries():
    L = _bytes("g1280_8x128_d64_bf16_fwdbwd")
    assert [(k, i) for k, _, _, i in L] == [("fwd", i) for i in range(8)] + [("bwd", i) for i in range(7, -1, -1)]
    G, tok, carry = 1280, 1280 * 128 * 64 * 2, 1280 * (64 * 64 + 64) * 4
    fwd = [b for k, _, b, _ in L if k == "fwd"]
    bwd = {i: b for k, _, b, i in L if k == "bwd"}
    # a zero initial carry is passed as NULL: chunk 0 reads no carry
    assert fwd[0] == 4 * tok + carry and all(b == 4 * tok + 2 * carry for b in fwd[1:])
    # the last chunk's backward has no upstream gradient; chunk 0's has no carry in
    assert bwd[7] == 7 * tok + 2 * carry and bwd[0] == 7 * tok + 2 * carry
    assert all(bwd[i] == 7 * tok + 3 * carry for i in range(1, 7))


def test_ragged_wide_head_bytes():
    L = _bytes("g160_63x128p100_d128_bf16_fwdbwd")
    assert [C for k, C, _, _ in L if k == "fwd"] == [128] * 63 + [100]
    assert sum(b for *_, b, _ in L) == pytest.approx(7049.5e6, rel=1e-4)


def test_sequence_launch_bytes():
    # one forward and one backward over T tokens: no carry between chunks moves; the forward
    # writes the final carry and its remainders, which the backward reads instead of
    # per-chunk carries, and writes the carry gradient
    G, T, D = 1280, 1024, 64
    tok, carry = G * T * D * 2, G * (D * D + D) * 4
    L = bench.plan_seq_launches(G, T, D, 2, carry=False)
    assert [k for k, *_ in L] == ["seqfwd", "seqbwd"]
    assert L[0][2] == 4 * tok + 2 * carry
    assert L[1][2] == 7 * tok + 3 * carry
    chained = sum(b for *_, b, _ in _bytes("g1280_8x128_d64_bf16_fwdbwd"))
    assert sum(b for *_, b, _ in L) < chained
