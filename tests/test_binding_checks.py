"""The Python binding refuses tensors that the kernels would overrun, before any
call into the library (the C ABI sees only pointers).  CPU tensors only: every
case is refused before a GPU is touched."""
import types

import pytest
import torch

import q4_routed_expert_amd as q4


def _lm(V=100, d=128):
    return types.SimpleNamespace(V=V, d=d, struct=None)


def _layer(d=128, E=8, k=2):
    return types.SimpleNamespace(d=d, n_experts=E, top_k=k, inter=64, struct=None)


bf16, f32, i32 = torch.bfloat16, torch.float32, torch.int32


@pytest.mark.parametrize("kw,what", [
    (dict(logits=torch.empty(99, dtype=f32)), "logits"),
    (dict(logits=torch.empty(100, dtype=torch.float64)), "logits"),
    (dict(token=torch.empty(1, dtype=torch.int64)), "token"),
    (dict(token=torch.empty(0, dtype=i32)), "token"),
    (dict(x_next=torch.empty(127, dtype=bf16)), "x_next"),
    (dict(x=torch.empty(128, dtype=f32)), "x"),
    (dict(x=torch.empty(64, dtype=bf16)), "x"),
    (dict(), "GPU"),  # right sizes, but host memory
])
def test_lm_argmax_refuses_bad_tensors(kw, what):
    args = dict(x=torch.empty(128, dtype=bf16), logits=torch.empty(100, dtype=f32),
                token=torch.empty(1, dtype=i32), x_next=None)
    args.update(kw)
    x = args.pop("x")
    with pytest.raises(ValueError, match=what):
        q4.lm_argmax(_lm(), x, torch.empty(4096, dtype=torch.uint8), **args)


def test_given_logits_need_no_input():
    with pytest.raises(ValueError, match="logits"):
        q4.lm_argmax(_lm(), None, torch.empty(16, dtype=torch.uint8),
                     logits=torch.empty(10, dtype=f32), token=torch.empty(1, dtype=i32),
                     logits_in=True)


def test_decode_refuses_short_buffers():
    L = _layer()
    ws = torch.empty(16, dtype=torch.uint8)
    with pytest.raises(ValueError, match="y"):
        q4.decode(L, torch.empty((1, 128), dtype=bf16), ws, y=torch.empty(127, dtype=bf16))
    with pytest.raises(ValueError, match="x"):
        q4.decode_tokens(L, torch.empty((4, 100), dtype=bf16), ws,
                         y=torch.empty((4, 128), dtype=bf16))
    with pytest.raises(ValueError, match="x"):
        q4.decode(L, torch.empty((1, 128), dtype=torch.int16), ws, y=torch.empty(128, dtype=bf16))
