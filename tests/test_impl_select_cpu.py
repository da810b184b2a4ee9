"""The selectable attention implementation of the autograd layer (host logic only): the
explicit argument, set_attention_impl and the LACHUNK_ATTN_IMPL environment variable, in that
order of precedence, and the errors for unknown names."""
import pytest
import torch

import causal_linear_attention_chunked_amd as lac
from causal_linear_attention_chunked_amd import autograd as ag


@pytest.fixture(autouse=True)
def reset(monkeypatch):
    monkeypatch.delenv(ag.IMPL_ENV, raising=False)
    lac.set_attention_impl(None)
    yield
    lac.set_attention_impl(None)


def test_default_is_auto():
    assert lac.get_attention_impl() == "auto"
    assert set(lac.IMPLS) == {"auto", "seq", "chunk", "cumsum"}


def test_environment_then_setter(monkeypatch):
    monkeypatch.setenv(ag.IMPL_ENV, "chunk")
    assert lac.get_attention_impl() == "chunk"
    lac.set_attention_impl("seq")
    assert lac.get_attention_impl() == "seq"  # the setter wins over the environment
    lac.set_attention_impl(None)
    assert lac.get_attention_impl() == "chunk"


def test_unknown_names_raise(monkeypatch):
    with pytest.raises(ValueError, match="unknown attention implementation"):
        lac.set_attention_impl("einsum")
    monkeypatch.setenv(ag.IMPL_ENV, "einsum")
    with pytest.raises(ValueError, match=ag.IMPL_ENV):
        lac.get_attention_impl()


def test_impl_checked_before_the_device():
    # the name is validated first; host tensors then raise for the device
    q = torch.ones(2, 8, 64)
    with pytest.raises(ValueError, match="unknown attention implementation"):
        lac.linear_attention(q, q, q, impl="fast")
    with pytest.raises(ValueError):
        lac.linear_attention(q, q, q, impl="chunk")


def test_sequence_segments():
    # the segments a sequence runs as through the sequence entry points (host logic)
    bf, seg = torch.bfloat16, ag.seq_segments
    T128, T64 = lac.SEQ_D128_MAX_T, lac.SEQ_D64_MAX_T
    assert seg(bf, 300, 128, 128) == [300]                       # one call, a ragged last chunk
    assert seg(bf, T128, 128, 128) == [T128]
    # longer: whole-chunk segments of the longest length one call takes, then the rest
    assert seg(bf, T128 + 100, 128, 128) == [T128, 100]
    assert seg(bf, 2 * T128 + 64, 128, 192) == [T128 - T128 % 192] * 2 + [2 * T128 + 64 - 2 * (T128 - T128 % 192)]
    assert seg(bf, 3 * T128, 128, 64) == [T128] * 3
    assert seg(bf, T64 + 256, 64, 128) == [T64, 256]
    # shapes the sequence calls never take stay None, whatever the length
    assert seg(bf, T64 + 100, 64, 128) is None                   # D = 64 takes whole 128-token chunks only
    assert seg(bf, 300, 64, 64) is None
    assert seg(torch.float32, 2 * T128, 128, 128) is None        # bf16 only
    assert seg(bf, T128 + 1, 128, 100) is None                   # chunks a multiple of 64 at D = 128
    # every segment but the last is whole chunks, and they add up
    for T, D, C in ((5 * T128 + 7, 128, 128), (T128 + 64, 128, 640)):
        s = seg(bf, T, D, C)
        assert sum(s) == T and all(x % C == 0 for x in s[:-1]) and all(x <= T128 for x in s)
