"""ctypes declarations mirroring include/q4moe.h."""
from __future__ import annotations

import ctypes as C
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libq4moe.so")

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EWORKSPACE, MOE_EHIP = 0, -1, -2, -3, -4
MOE_LOGITS_IN = 1
MOE_ITEM_ROWS_64, MOE_ITEM_ROWS_32, MOE_ITEM_ROWS_16 = 2, 4, 8
MOE_BLOCK_ROWS = 32
MOE_TILE_ROWS = 128
MOE_ROUTE_BLOCK = 256
MOE_DECODE_ROUTER_ROWS = 128
MOE_MAX_DECODE_TOKENS = 8
MOE_MAX_VOCAB = 1 << 20
MOE_STATIC_SCRATCH_BYTES = 1 << 20
MOE_MAX_EXPERTS, MOE_MAX_TOPK, MOE_MAX_TOKENS, MOE_MAX_D, MOE_MAX_INTER = 256, 8, 32768, 8192, 2048

# every function include/q4moe.h declares
EXPORTS = ("moe_block_map_capacity", "moe_workspace_bytes", "moe_route", "moe_prefill",
           "moe_prefill_ex", "moe_trace_events",
           "moe_decode", "moe_decode_tokens", "moe_dequant", "moe_strerror", "moe_last_error",
           "moe_lm_workspace_bytes", "moe_lm_argmax", "moe_decode_tokens_static")


class Q4Mat(C.Structure):
    _fields_ = [("q", C.c_void_p), ("scale", C.c_void_p), ("bias", C.c_void_p)]


class Layer(C.Structure):
    _fields_ = [("d", C.c_int32), ("inter", C.c_int32), ("n_experts", C.c_int32),
                ("top_k", C.c_int32), ("w_router", C.c_void_p), ("router_bias", C.c_void_p),
                ("gate", Q4Mat), ("up", Q4Mat), ("down", Q4Mat),
                ("sh_gate", Q4Mat), ("sh_up", Q4Mat), ("sh_down", Q4Mat)]


class LmHead(C.Structure):
    _fields_ = [("V", C.c_int32), ("d", C.c_int32), ("head", Q4Mat), ("embed", Q4Mat)]


class Routing(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("logits", "topk_idx", "topk_w", "counts", "offsets",
                                          "perm", "inv_perm", "block_map", "n_blocks",
                                          "tile_map", "n_tiles", "blk_counts")]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it first "
                               "(python -c 'import __graft_entry__ as g; g.build()')")
        # torch ships its own HIP runtime; load it first so that the library's
        # libamdhip64 dependency resolves to the same runtime (one runtime per
        # process: torch's streams and allocations are then valid here).
        import torch  # noqa: F401
        L = C.CDLL(LIB_PATH)
        with open("/proc/self/maps") as f:
            runtimes = {ln.split()[-1] for ln in f if "libamdhip64" in ln}
        if len(runtimes) > 1:
            raise RuntimeError(f"two HIP runtimes loaded in one process: {sorted(runtimes)}")
        vp, i32 = C.c_void_p, C.c_int32
        L.moe_block_map_capacity.argtypes = [i32, i32, i32, i32]
        L.moe_block_map_capacity.restype = i32
        L.moe_workspace_bytes.argtypes = [vp, i32]
        L.moe_workspace_bytes.restype = C.c_size_t
        L.moe_route.argtypes = [vp, vp, i32, C.c_uint32, vp, vp]
        L.moe_prefill.argtypes = [vp, vp, i32, vp, vp, C.c_size_t, vp, vp]
        L.moe_prefill_ex.argtypes = [vp, vp, i32, vp, vp, C.c_size_t, vp, C.c_uint32, vp]
        L.moe_decode.argtypes = [vp, vp, C.c_uint32, vp, vp, C.c_size_t, vp, vp]
        L.moe_decode_tokens.argtypes = [vp, vp, i32, C.c_uint32, vp, vp, C.c_size_t, vp, vp]
        L.moe_decode_tokens_static.argtypes = [vp, vp, i32, C.c_uint32, vp, vp, vp]
        L.moe_dequant.argtypes = [vp, i32, i32, vp, vp]
        L.moe_lm_workspace_bytes.argtypes = [vp]
        L.moe_lm_workspace_bytes.restype = C.c_size_t
        L.moe_lm_argmax.argtypes = [vp, vp, C.c_uint32, vp, vp, vp, vp, C.c_size_t, vp]
        for f in ("moe_route", "moe_prefill", "moe_prefill_ex", "moe_decode", "moe_decode_tokens", "moe_dequant",
                  "moe_lm_argmax", "moe_decode_tokens_static"):
            getattr(L, f).restype = C.c_int
        L.moe_trace_events.argtypes = [vp, i32]
        L.moe_trace_events.restype = None
        L.moe_strerror.argtypes = [C.c_int]
        L.moe_strerror.restype = C.c_char_p
        L.moe_last_error.argtypes = []
        L.moe_last_error.restype = C.c_char_p
        _lib = L
    return _lib
