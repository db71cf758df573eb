"""ctypes front end of the CPU oracle (oracle/q4moe_oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only code that may import this package.  It shares
nothing with the HIP path (q4_routed_expert_amd); neither imports the other.
Every function takes and returns numpy arrays on the host.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "q4moe_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")


def build() -> str:
    """Compile the oracle with gcc: IEEE double arithmetic, no contraction, no fast-math."""
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-fPIC", "-shared", "-o", _LIB + ".tmp", _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


class _Q4(C.Structure):
    _fields_ = [("q", C.c_void_p), ("scale", C.c_void_p), ("bias", C.c_void_p)]


class _Layer(C.Structure):
    _fields_ = [("d", C.c_int64), ("inter", C.c_int64), ("n_experts", C.c_int64),
                ("top_k", C.c_int64), ("w_router", C.c_void_p), ("router_bias", C.c_void_p),
                ("gate", _Q4), ("up", _Q4), ("down", _Q4),
                ("sh_gate", _Q4), ("sh_up", _Q4), ("sh_down", _Q4)]


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        lib = C.CDLL(_LIB)
        vp, i64 = C.c_void_p, C.c_int64
        lib.oracle_dequant.argtypes = [vp, vp, vp, i64, i64, vp]
        lib.oracle_router_logits.argtypes = [vp, i64, i64, vp, vp, i64, vp]
        lib.oracle_route.argtypes = [vp, i64, i64, i64, vp, vp, vp, vp, vp, vp]
        lib.oracle_block_map.argtypes = [vp, vp, i64, i64, vp, vp]
        lib.oracle_expert.argtypes = [C.POINTER(_Layer), i64, vp, vp, vp]
        lib.oracle_layer_tokens.argtypes = [C.POINTER(_Layer), vp, vp, i64, vp, vp, vp, vp]
        lib.oracle_threads.restype = C.c_int
        lib.oracle_bf16_round.argtypes = [vp, i64, vp]
        lib.oracle_lm_logits.argtypes = [vp, vp, vp, i64, i64, vp, vp]
        lib.oracle_argmax.argtypes = [vp, i64]
        lib.oracle_argmax.restype = i64
        _lib = lib
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


def threads() -> int:
    return int(_load().oracle_threads())


def bf16_round(v) -> np.ndarray:
    v = _c(v, np.float64)
    out = np.empty(v.shape, np.uint16)
    _load().oracle_bf16_round(_p(v), v.size, _p(out))
    return out


def dequant(q, scale, bias) -> np.ndarray:
    """bf16 bits [N, K] of the dequantised matrix (q: uint32 [N, K/8])."""
    q, scale, bias = _c(q, np.uint32), _c(scale, np.uint16), _c(bias, np.uint16)
    N, K = q.shape[0], q.shape[1] * 8
    w = np.empty((N, K), np.uint16)
    _load().oracle_dequant(_p(q), _p(scale), _p(bias), N, K, _p(w))
    return w


def router_logits(x, w_router, router_bias=None) -> np.ndarray:
    x, W = _c(x, np.uint16), _c(w_router, np.float32)
    b = None if router_bias is None else _c(router_bias, np.float32)
    T, d = x.shape
    E = W.shape[1]
    out = np.empty((T, E), np.float32)
    _load().oracle_router_logits(_p(x), T, d, _p(W), _p(b), E, _p(out))
    return out


def route(logits, k: int) -> dict:
    logits = _c(logits, np.float32)
    T, E = logits.shape
    r = {"idx": np.empty((T, k), np.int32), "w": np.empty((T, k), np.float64),
         "counts": np.empty(E, np.int32), "offsets": np.empty(E + 1, np.int32),
         "perm": np.empty(T * k, np.int32), "inv_perm": np.empty(T * k, np.int32)}
    _load().oracle_route(_p(logits), T, E, k, _p(r["idx"]), _p(r["w"]), _p(r["counts"]),
                         _p(r["offsets"]), _p(r["perm"]), _p(r["inv_perm"]))
    return r


def block_map(counts, offsets, bm: int):
    counts, offsets = _c(counts, np.int32), _c(offsets, np.int32)
    E = counts.shape[0]
    cap = int(offsets[-1]) // bm + E
    bmap = np.empty((max(cap, 1), 2), np.int32)
    n = np.zeros(1, np.int32)
    _load().oracle_block_map(_p(counts), _p(offsets), E, bm, _p(bmap), _p(n))
    return bmap[: int(n[0])].copy(), int(n[0])


def _layer_struct(L: dict):
    keep = []

    def arr(a, dt):
        a = _c(a, dt)
        keep.append(a)
        return a.ctypes.data

    def q4(name):
        return _Q4(arr(L[name + "_q"], np.uint32), arr(L[name + "_s"], np.uint16),
                   arr(L[name + "_b"], np.uint16))

    s = _Layer(L["d"], L["inter"], L["n_experts"], L["top_k"],
               arr(L["w_router"], np.float32),
               None if L.get("router_bias") is None else arr(L["router_bias"], np.float32),
               q4("gate"), q4("up"), q4("down"), q4("sh_gate"), q4("sh_up"), q4("sh_down"))
    return s, keep


def expert(L: dict, e: int, x_t):
    """(h bf16 bits [inter], P float64 [d]) of expert e (e = -1: shared) on one token."""
    s, keep = _layer_struct(L)
    x_t = _c(x_t, np.uint16)
    h = np.empty(L["inter"], np.uint16)
    P = np.empty(L["d"], np.float64)
    _load().oracle_expert(C.byref(s), e, _p(x_t), _p(h), _p(P))
    return h, P


def layer_tokens(L: dict, x, tokens, idx, w):
    """(y_exact float64 [n, d], y bf16 bits [n, d]) for the listed tokens."""
    s, keep = _layer_struct(L)
    x = _c(x, np.uint16)
    tokens = _c(tokens, np.int32)
    idx, w = _c(idx, np.int32), _c(w, np.float64)
    n, d = tokens.shape[0], L["d"]
    y_exact = np.empty((n, d), np.float64)
    y = np.empty((n, d), np.uint16)
    _load().oracle_layer_tokens(C.byref(s), _p(x), _p(tokens), n, _p(idx), _p(w),
                                _p(y_exact), _p(y))
    return y_exact, y


def layer(L: dict, x, logits=None, tokens=None):
    """The whole layer: logits -> routing -> outputs (for all or the listed tokens)."""
    if logits is None:
        logits = router_logits(x, L["w_router"], L.get("router_bias"))
    r = route(logits, L["top_k"])
    if tokens is None:
        tokens = np.arange(x.shape[0], dtype=np.int32)
    y_exact, y = layer_tokens(L, x, tokens, r["idx"], r["w"])
    r.update(logits=logits, y_exact=y_exact, y=y, tokens=np.asarray(tokens, np.int32))
    return r


# ---- greedy decoding's token hand-off (page section "Decode: minimize bytes
# per token": the chosen token stays on the device, from the largest output
# logit into the following step's input).  The head and the embedding table
# are V x d Q4 matrices.

def lm_logits(x, q, scale, bias) -> np.ndarray:
    """fp32 [V] logits of a [V, d] Q4 matrix (q: uint32 [V, d/8]) applied to x (bf16 [d])."""
    x = _c(x, np.uint16).reshape(-1)
    q, scale, bias = _c(q, np.uint32), _c(scale, np.uint16), _c(bias, np.uint16)
    V, d = q.shape[0], q.shape[1] * 8
    assert x.size == d
    out = np.empty(V, np.float32)
    _load().oracle_lm_logits(_p(q), _p(scale), _p(bias), V, d, _p(x), _p(out))
    return out


def argmax(logits) -> int:
    """Index of the largest logit; equal logits: the lower index; NaN counts as -inf."""
    lg = _c(logits, np.float32).reshape(-1)
    return int(_load().oracle_argmax(_p(lg), lg.size))


def embed_row(q, scale, bias, token: int) -> np.ndarray:
    """The next step's input: bf16 bits [d] of row `token` of a Q4 embedding table."""
    return dequant(q[token:token + 1], scale[token:token + 1], bias[token:token + 1])[0]


def lm_step(head: dict, embed: dict | None, x):
    """One greedy hand-off: (logits, token, next input or None).  head / embed:
    dicts with q, scale, bias as above."""
    lg = lm_logits(x, head["q"], head["scale"], head["bias"])
    tok = argmax(lg)
    nxt = None if embed is None else embed_row(embed["q"], embed["scale"], embed["bias"], tok)
    return lg, tok, nxt
