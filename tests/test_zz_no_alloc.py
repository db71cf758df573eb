"""moe_decode_tokens_static (the library's static device scratch, no allocation)
against moe_decode_tokens (the caller's workspace).  Both run the same kernels,
so outputs, logits, selected experts and scores must be bit-identical.  Two
calls in a row through the C ABI: the decode workload's layer on 8 tokens, then
a smaller layer on 3 tokens (the scratch keeps the first call's contents)."""
import ctypes as C

import numpy as np
import pytest
import torch

import q4_routed_expert_amd as q4
from q4_routed_expert_amd import _abi
from workloads import WORKLOADS, decode_inputs, make_layer, random_layer, random_x

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _static_call(layer, xd, T, routing, y, logits_in=False):
    flags = _abi.MOE_LOGITS_IN if logits_in else 0
    rc = _abi.lib().moe_decode_tokens_static(
        C.addressof(layer.struct), xd.data_ptr(), T, flags, C.addressof(routing.struct),
        y.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert rc == 0, _abi.lib().moe_last_error().decode()


def _case(L, xs, dev, name):
    T, d, E, k = xs.shape[0], L["d"], L["n_experts"], L["top_k"]
    layer = q4.DeviceLayer.from_host(L, dev)
    xd = torch.from_numpy(xs.view(np.int16)).to(dev).view(torch.bfloat16)
    ws = q4.workspace(layer, 1, dev)
    r_ref = q4.DeviceRouting(T, E, k, dev)
    y_ref = q4.decode_tokens(layer, xd, ws, routing=r_ref)
    r = q4.DeviceRouting(T, E, k, dev)
    y = torch.empty((T, d), dtype=torch.bfloat16, device=dev)
    _static_call(layer, xd, T, r, y)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(y), _bits(y_ref)), name
    assert np.array_equal(r.logits.cpu().numpy(), r_ref.logits.cpu().numpy()), name
    assert np.array_equal(r.topk_idx.cpu().numpy(), r_ref.topk_idx.cpu().numpy()), name
    assert np.array_equal(r.topk_w.cpu().numpy(), r_ref.topk_w.cpu().numpy()), name
    # from given logits as well
    y2 = torch.empty_like(y)
    _static_call(layer, xd, T, r, y2, logits_in=True)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(y2), _bits(y_ref)), name
    print(f"[no-alloc] {name}: T={T} d={d} E={E} k={k} bit-identical to moe_decode_tokens",
          flush=True)


def test_static_scratch_decode_matches_workspace_decode():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dev = torch.device("cuda:0")
    w = WORKLOADS["decode"]
    L, _ = make_layer(w, 5)
    _case(L, decode_inputs(w, 8), dev, "decode workload layer 5")
    rng = np.random.default_rng(31)
    Ls = random_layer(rng, 512, 128, 32, 4, router_bias=True)
    _case(Ls, random_x(rng, 3, 512), dev, "smaller layer")
