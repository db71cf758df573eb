"""Python binding of libq4moe.so, the gfx950 routed-MoE Q4 FFN layer.

Argument marshalling only: every step of the layer runs in the HIP kernels
behind the C ABI of include/q4moe.h.  PyTorch supplies device memory and the
stream.  There is no fallback: if the library is missing, loading raises.

    layer = DeviceLayer.from_host(L)           # L: dict of numpy arrays
    r = route(layer, x)                        # x: bf16 [T, d] on the GPU
    y = prefill(layer, x, r)                   # bf16 [T, d]
    y1 = decode(layer, x1, ws)                 # one token
    lm = DeviceLmHead.from_host(head, embed)     # V x d output head, embedding
    logits, tok, _ = lm_argmax(lm, h, lm_workspace(lm), x_next=x_in)  # greedy token
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np
import torch

from . import _abi

MOE_LOGITS_IN = _abi.MOE_LOGITS_IN
MAX_DECODE_TOKENS = _abi.MOE_MAX_DECODE_TOKENS
BLOCK_ROWS = _abi.MOE_BLOCK_ROWS
TILE_ROWS = _abi.MOE_TILE_ROWS
MATS = ("gate", "up", "down", "sh_gate", "sh_up", "sh_down")


class MoEError(RuntimeError):
    def __init__(self, code: int, where: str):
        lib = _abi.lib()
        self.code = code
        msg = lib.moe_strerror(code).decode()
        detail = lib.moe_last_error().decode()
        super().__init__(f"{where}: {msg} ({code}): {detail}")


def _check(code: int, where: str):
    if code != 0:
        raise MoEError(code, where)


def _stream(stream) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return int(s.cuda_stream)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _need(t, name: str, dtype, n: int):
    """The C ABI sees only pointers, so the binding checks what the kernels will
    touch: a contiguous tensor of `dtype` with at least n elements (and, through
    _on_gpu, in device memory)."""
    if t is None:
        raise ValueError(f"{name} is required")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if t.numel() < n:
        raise ValueError(f"{name}: {t.numel()} elements, the call touches {n}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _on_gpu(**tensors):
    for name, t in tensors.items():
        if t is not None and not t.is_cuda:
            raise ValueError(f"{name} must be on the GPU")


def _dev(a: np.ndarray, device) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    view = {np.dtype(np.uint32): np.int32, np.dtype(np.uint16): np.int16}.get(a.dtype, a.dtype)
    return torch.from_numpy(a.view(view)).to(device)


class DeviceLayer:
    """One layer's weights in device memory plus the moe_layer struct pointing at them."""

    def __init__(self, d, inter, n_experts, top_k, tensors: dict):
        self.d, self.inter, self.n_experts, self.top_k = d, inter, n_experts, top_k
        self.t = tensors
        mats = {m: _abi.Q4Mat(_ptr(tensors[m + "_q"]), _ptr(tensors[m + "_s"]),
                              _ptr(tensors[m + "_b"])) for m in MATS}
        self.struct = _abi.Layer(d, inter, n_experts, top_k, _ptr(tensors["w_router"]),
                                 _ptr(tensors.get("router_bias")), *[mats[m] for m in MATS])

    @classmethod
    def from_host(cls, L: dict, device="cuda"):
        t = {}
        for m in MATS:
            for suf in ("_q", "_s", "_b"):
                t[m + suf] = _dev(L[m + suf], device)
        t["w_router"] = _dev(L["w_router"].astype(np.float32), device)
        if L.get("router_bias") is not None:
            t["router_bias"] = _dev(L["router_bias"].astype(np.float32), device)
        return cls(L["d"], L["inter"], L["n_experts"], L["top_k"], t)

    def weight_bytes(self) -> int:
        return sum(v.numel() * v.element_size() for k, v in self.t.items()
                   if k.endswith(("_q", "_s", "_b")))


class DeviceRouting:
    """Device arrays of moe_routing for up to T tokens."""

    def __init__(self, T: int, n_experts: int, top_k: int, device="cuda"):
        lib = _abi.lib()
        i32 = dict(dtype=torch.int32, device=device)
        self.T, self.E, self.k = T, n_experts, top_k
        self.logits = torch.zeros((T, n_experts), dtype=torch.float32, device=device)
        self.topk_idx = torch.zeros((T, top_k), **i32)
        self.topk_w = torch.zeros((T, top_k), dtype=torch.float32, device=device)
        self.counts = torch.zeros(n_experts, **i32)
        self.offsets = torch.zeros(n_experts + 1, **i32)
        self.perm = torch.zeros(T * top_k, **i32)
        self.inv_perm = torch.zeros(T * top_k, **i32)
        nb = lib.moe_block_map_capacity(T, top_k, n_experts, BLOCK_ROWS)
        nt = lib.moe_block_map_capacity(T, top_k, n_experts, TILE_ROWS)
        self.block_map = torch.zeros((nb, 2), **i32)
        self.n_blocks = torch.zeros(1, **i32)
        self.tile_map = torch.zeros((nt, 2), **i32)
        self.n_tiles = torch.zeros(1, **i32)
        n_blk = (T + _abi.MOE_ROUTE_BLOCK - 1) // _abi.MOE_ROUTE_BLOCK
        self.blk_counts = torch.zeros((n_blk, n_experts), **i32)
        self.struct = _abi.Routing(*[_ptr(getattr(self, f)) for f, _ in _abi.Routing._fields_])


def workspace_bytes(layer: DeviceLayer, T: int) -> int:
    n = _abi.lib().moe_workspace_bytes(C.addressof(layer.struct), T)
    if n == 0:
        raise MoEError(_abi.MOE_EINVAL, "moe_workspace_bytes")
    return int(n)


def workspace(layer: DeviceLayer, T: int, device="cuda") -> torch.Tensor:
    """A zero-filled workspace for moe_prefill (T tokens) and moe_decode."""
    return torch.zeros(workspace_bytes(layer, T), dtype=torch.uint8, device=device)


def route(layer: DeviceLayer, x: torch.Tensor, routing: DeviceRouting | None = None,
          logits_in: bool = False, stream=None) -> DeviceRouting:
    T = x.shape[0]
    r = routing or DeviceRouting(T, layer.n_experts, layer.top_k, x.device)
    flags = MOE_LOGITS_IN if logits_in else 0
    if not logits_in:
        _need(x, "x", torch.bfloat16, T * layer.d)
    _need(r.logits, "routing.logits", torch.float32, T * layer.n_experts)
    _need(r.perm, "routing.perm", torch.int32, T * layer.top_k)
    _on_gpu(x=None if logits_in else x, logits=r.logits)
    _check(_abi.lib().moe_route(C.addressof(layer.struct), _ptr(x), T, flags, C.addressof(r.struct),
                                _stream(stream)), "moe_route")
    return r


_ITEM_ROWS_FLAGS = {128: 0, 64: _abi.MOE_ITEM_ROWS_64, 32: _abi.MOE_ITEM_ROWS_32,
                    16: _abi.MOE_ITEM_ROWS_16}


def prefill(layer: DeviceLayer, x: torch.Tensor, routing: DeviceRouting,
            ws: torch.Tensor | None = None, y: torch.Tensor | None = None,
            stream=None, item_rows: int = 128) -> torch.Tensor:
    """moe_prefill (item_rows = 128) or moe_prefill_ex with the gate/up work-item
    height item_rows (64, 32 or 16)."""
    if item_rows not in _ITEM_ROWS_FLAGS:
        raise ValueError(f"item_rows must be one of 128, 64, 32, 16, not {item_rows}")
    T = x.shape[0]
    if ws is None:
        ws = workspace(layer, T, x.device)
    if y is None:
        y = torch.empty((T, layer.d), dtype=torch.bfloat16, device=x.device)
    _need(x, "x", torch.bfloat16, T * layer.d)
    _need(y, "y", torch.bfloat16, T * layer.d)
    _need(routing.perm, "routing.perm", torch.int32, T * layer.top_k)
    _on_gpu(x=x, y=y, ws=ws, perm=routing.perm)
    if item_rows == 128:
        _check(_abi.lib().moe_prefill(C.addressof(layer.struct), _ptr(x), T,
                                      C.addressof(routing.struct), _ptr(ws), ws.numel(), _ptr(y),
                                      _stream(stream)),
               "moe_prefill")
    else:
        _check(_abi.lib().moe_prefill_ex(C.addressof(layer.struct), _ptr(x), T,
                                         C.addressof(routing.struct), _ptr(ws), ws.numel(),
                                         _ptr(y), _ITEM_ROWS_FLAGS[item_rows], _stream(stream)),
               "moe_prefill_ex")
    return y


def decode(layer: DeviceLayer, x: torch.Tensor, ws: torch.Tensor, y: torch.Tensor | None = None,
           routing: DeviceRouting | None = None, logits_in: bool = False,
           stream=None) -> torch.Tensor:
    if y is None:
        y = torch.empty((1, layer.d), dtype=torch.bfloat16, device=x.device)
    flags = MOE_LOGITS_IN if logits_in else 0
    rs = C.addressof(routing.struct) if routing is not None else None
    _need(x, "x", torch.bfloat16, layer.d)
    _need(y, "y", torch.bfloat16, layer.d)
    if routing is not None:
        _need(routing.logits, "routing.logits", torch.float32, layer.n_experts)
        _need(routing.topk_idx, "routing.topk_idx", torch.int32, layer.top_k)
    _on_gpu(x=x, y=y, ws=ws)
    _check(_abi.lib().moe_decode(C.addressof(layer.struct), _ptr(x), flags, rs, _ptr(ws), ws.numel(),
                                 _ptr(y), _stream(stream)), "moe_decode")
    return y


def decode_tokens(layer: DeviceLayer, x: torch.Tensor, ws: torch.Tensor,
                  y: torch.Tensor | None = None, routing: DeviceRouting | None = None,
                  logits_in: bool = False, stream=None) -> torch.Tensor:
    """The decode layer for T = x.shape[0] tokens (1 <= T <= MAX_DECODE_TOKENS)."""
    T = x.shape[0]
    if y is None:
        y = torch.empty((T, layer.d), dtype=torch.bfloat16, device=x.device)
    flags = MOE_LOGITS_IN if logits_in else 0
    rs = C.addressof(routing.struct) if routing is not None else None
    _need(x, "x", torch.bfloat16, T * layer.d)
    _need(y, "y", torch.bfloat16, T * layer.d)
    if routing is not None:
        _need(routing.logits, "routing.logits", torch.float32, T * layer.n_experts)
        _need(routing.topk_idx, "routing.topk_idx", torch.int32, T * layer.top_k)
    _on_gpu(x=x, y=y, ws=ws)
    _check(_abi.lib().moe_decode_tokens(C.addressof(layer.struct), _ptr(x), T, flags, rs, _ptr(ws),
                                        ws.numel(), _ptr(y), _stream(stream)), "moe_decode_tokens")
    return y


def dequant(q: torch.Tensor, scale: torch.Tensor, bias: torch.Tensor, stream=None) -> torch.Tensor:
    """bf16 [N, K] from one Q4 matrix (q int32 [N, K/8], scale/bias bf16 bits [N, K/64])."""
    N, K = q.shape[0], q.shape[1] * 8
    out = torch.empty((N, K), dtype=torch.bfloat16, device=q.device)
    m = _abi.Q4Mat(_ptr(q), _ptr(scale), _ptr(bias))
    _check(_abi.lib().moe_dequant(C.addressof(m), N, K, _ptr(out), _stream(stream)), "moe_dequant")
    return out


class DeviceLmHead:
    """An output head and embedding table (V x d Q4 each) in device memory, plus
    the moe_lm_head struct pointing at them."""

    def __init__(self, V: int, d: int, head: dict, embed: dict | None):
        self.V, self.d = V, d
        self.head, self.embed = head, embed  # keep the tensors alive

        def mat(m):
            return _abi.Q4Mat() if m is None else _abi.Q4Mat(_ptr(m["q"]), _ptr(m["scale"]),
                                                              _ptr(m["bias"]))
        self.struct = _abi.LmHead(V, d, mat(head), mat(embed))

    @classmethod
    def from_host(cls, head: dict, embed: dict | None = None, device="cuda"):
        """head / embed: dicts of numpy q uint32 [V, d/8], scale, bias uint16 [V, d/64]."""
        V, d = head["q"].shape[0], head["q"].shape[1] * 8
        dev = lambda m: None if m is None else {k: _dev(m[k], device) for k in ("q", "scale", "bias")}
        return cls(V, d, dev(head), dev(embed))


def lm_workspace(lm: DeviceLmHead, device="cuda") -> torch.Tensor:
    n = _abi.lib().moe_lm_workspace_bytes(C.addressof(lm.struct))
    if n == 0:
        raise MoEError(_abi.MOE_EINVAL, "moe_lm_workspace_bytes")
    return torch.empty(n, dtype=torch.uint8, device=device)


def lm_argmax(lm: DeviceLmHead, x: torch.Tensor | None, ws: torch.Tensor,
              logits: torch.Tensor | None = None, token: torch.Tensor | None = None,
              x_next: torch.Tensor | None = None, logits_in: bool = False, stream=None):
    """Greedy token hand-off: (logits fp32 [V], token int32 [1], x_next or None).
    With logits_in the given logits are read instead of computed from x."""
    dev = ws.device
    if logits is None:
        logits = torch.empty(lm.V, dtype=torch.float32, device=dev)
    if token is None:
        token = torch.empty(1, dtype=torch.int32, device=dev)
    flags = MOE_LOGITS_IN if logits_in else 0
    if not logits_in:
        _need(x, "x", torch.bfloat16, lm.d)
    _need(logits, "logits", torch.float32, lm.V)
    _need(token, "token", torch.int32, 1)
    if x_next is not None:
        _need(x_next, "x_next", torch.bfloat16, lm.d)
    _on_gpu(x=None if logits_in else x, logits=logits, token=token, x_next=x_next, ws=ws)
    _check(_abi.lib().moe_lm_argmax(C.addressof(lm.struct), _ptr(x), flags, _ptr(logits),
                                    _ptr(token), _ptr(x_next), _ptr(ws), ws.numel(),
                                    _stream(stream)), "moe_lm_argmax")
    return logits, token, x_next


def library_path() -> str:
    return _abi.LIB_PATH
