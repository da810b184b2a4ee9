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
