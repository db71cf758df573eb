"""Host-side checks of the C-ABI library: it loads, exports every function the
header declares, and refuses invalid arguments before touching the GPU.
None of these calls launches a kernel, so they run without a GPU."""
import ctypes as C
import os
import re

import pytest

from q4_routed_expert_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "q4moe.h")

# Nonzero, 16-byte aligned fake device addresses: validation only looks at them.
FAKE = 0x10000


def _header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert _header_functions() == sorted(_abi.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = _abi.lib()
    for name in _header_functions():
        assert hasattr(lib, name), name


def test_header_limits_match_binding():
    text = open(HEADER).read()
    for name in ("MOE_GROUP", "MOE_MAX_EXPERTS", "MOE_MAX_TOPK", "MOE_MAX_TOKENS", "MOE_MAX_D",
                 "MOE_MAX_INTER", "MOE_BLOCK_ROWS", "MOE_TILE_ROWS", "MOE_ROUTE_BLOCK",
                 "MOE_DECODE_ROUTER_ROWS", "MOE_MAX_DECODE_TOKENS", "MOE_LOGITS_IN",
                 "MOE_MAX_VOCAB", "MOE_ITEM_ROWS_64", "MOE_ITEM_ROWS_32", "MOE_ITEM_ROWS_16"):
        m = re.search(rf"#define {name} (\d+)", text)
        assert m, name
        if hasattr(_abi, name):
            assert int(m.group(1)) == getattr(_abi, name), name


def _layer(d=2048, inter=512, E=256, k=8, bias=False):
    mats = [_abi.Q4Mat(FAKE, FAKE, FAKE) for _ in range(6)]
    return _abi.Layer(d, inter, E, k, FAKE, FAKE if bias else None, *mats)


def _routing():
    return _abi.Routing(*[FAKE] * len(_abi.Routing._fields_))


def _route(L, T=16, r=None, x=FAKE, flags=0):
    lib = _abi.lib()
    rr = r if r is not None else _routing()
    return lib.moe_route(C.addressof(L), x, T, flags, C.addressof(rr), None)


@pytest.mark.parametrize("kw,code", [
    (dict(d=2000), _abi.MOE_EUNSUPPORTED),          # not a multiple of the group
    (dict(inter=96), _abi.MOE_EUNSUPPORTED),
    (dict(E=257), _abi.MOE_EUNSUPPORTED),
    (dict(k=9, E=256), _abi.MOE_EUNSUPPORTED),
    (dict(k=5, E=4), _abi.MOE_EUNSUPPORTED),        # k > E
    (dict(d=0), _abi.MOE_EINVAL),
    (dict(k=0), _abi.MOE_EINVAL),
    (dict(d=8256), _abi.MOE_EUNSUPPORTED),
    (dict(inter=2112), _abi.MOE_EUNSUPPORTED),
])
def test_route_rejects_unsupported_layers(kw, code):
    assert _route(_layer(**kw)) == code
    assert _abi.lib().moe_last_error()


@pytest.mark.parametrize("T,code", [(0, _abi.MOE_EINVAL), (-3, _abi.MOE_EINVAL),
                                    (_abi.MOE_MAX_TOKENS + 1, _abi.MOE_EUNSUPPORTED)])
def test_route_rejects_bad_token_counts(T, code):
    assert _route(_layer(), T=T) == code


def test_null_and_misaligned_pointers_are_rejected():
    lib = _abi.lib()
    L = _layer()
    r0 = _routing()
    assert lib.moe_route(None, FAKE, 4, 0, C.addressof(r0), None) == _abi.MOE_EINVAL
    assert _route(L, x=None) == _abi.MOE_EINVAL
    assert _route(L, x=FAKE + 2) == _abi.MOE_EINVAL
    L.gate.scale = None
    assert _route(L) == _abi.MOE_EINVAL
    assert b"gate.scale" in lib.moe_last_error()
    L = _layer()
    L.w_router = FAKE + 4
    assert _route(L) == _abi.MOE_EINVAL
    r = _routing()
    r.perm = None
    assert _route(_layer(), r=r) == _abi.MOE_EINVAL
    assert b"perm" in lib.moe_last_error()
    assert _route(_layer(), flags=0x10) == _abi.MOE_EINVAL


def test_prefill_checks_workspace_size_before_launch():
    lib = _abi.lib()
    L = _layer()
    need = lib.moe_workspace_bytes(C.addressof(L), 2048)
    assert need > 0
    r = _routing()
    rc = lib.moe_prefill(C.addressof(L), FAKE, 2048, C.addressof(r), FAKE, need - 1, FAKE, None)
    assert rc == _abi.MOE_EWORKSPACE
    rc = lib.moe_decode(C.addressof(L), FAKE, 0, None, FAKE, lib.moe_workspace_bytes(
        C.addressof(L), 1) - 256, FAKE, None)
    assert rc == _abi.MOE_EWORKSPACE
    rc = lib.moe_decode(C.addressof(L), FAKE, _abi.MOE_LOGITS_IN, None, FAKE, 1 << 30, FAKE, None)
    assert rc == _abi.MOE_EINVAL


def test_prefill_ex_checks_flags_before_launch():
    lib = _abi.lib()
    L = _layer()
    need = lib.moe_workspace_bytes(C.addressof(L), 2048)
    r = _routing()
    call = lambda flags, ws=need: lib.moe_prefill_ex(C.addressof(L), FAKE, 2048, C.addressof(r),
                                                     FAKE, ws, FAKE, flags, None)
    rows = (_abi.MOE_ITEM_ROWS_64, _abi.MOE_ITEM_ROWS_32, _abi.MOE_ITEM_ROWS_16)
    for i, f in enumerate(rows):  # any two heights together
        for g in rows[i + 1:]:
            assert call(f | g) == _abi.MOE_EINVAL
    assert call(rows[0] | rows[1] | rows[2]) == _abi.MOE_EINVAL
    assert call(1) == _abi.MOE_EINVAL
    assert call(16) == _abi.MOE_EINVAL
    # valid flags get as far as the workspace check
    for flags in (0,) + rows:
        assert call(flags, need - 1) == _abi.MOE_EWORKSPACE


@pytest.mark.parametrize("T,code", [(0, _abi.MOE_EUNSUPPORTED), (-1, _abi.MOE_EUNSUPPORTED),
                                    (_abi.MOE_MAX_DECODE_TOKENS + 1, _abi.MOE_EUNSUPPORTED)])
def test_decode_tokens_rejects_token_counts_outside_its_range(T, code):
    lib = _abi.lib()
    L = _layer()
    rc = lib.moe_decode_tokens(C.addressof(L), FAKE, T, 0, None, FAKE, 1 << 30, FAKE, None)
    assert rc == code


def test_decode_tokens_checks_workspace_and_flags_before_launch():
    lib = _abi.lib()
    L = _layer()
    need = lib.moe_workspace_bytes(C.addressof(L), 1)
    rc = lib.moe_decode_tokens(C.addressof(L), FAKE, _abi.MOE_MAX_DECODE_TOKENS, 0, None, FAKE,
                               need - 256, FAKE, None)
    assert rc == _abi.MOE_EWORKSPACE
    rc = lib.moe_decode_tokens(C.addressof(L), FAKE, 4, _abi.MOE_LOGITS_IN, None, FAKE, need,
                               FAKE, None)
    assert rc == _abi.MOE_EINVAL
    rc = lib.moe_decode_tokens(C.addressof(L), FAKE + 8, 4, 0, None, FAKE, need, FAKE, None)
    assert rc == _abi.MOE_EINVAL  # misaligned x


def test_workspace_bytes_cover_the_staged_buffers():
    lib = _abi.lib()
    for T, d, I, E, k in ((2048, 2048, 512, 256, 8), (32, 512, 128, 32, 4), (1, 2048, 512, 256, 8)):
        L = _layer(d, I, E, k)  # keep the struct alive across the call
        n = lib.moe_workspace_bytes(C.addressof(L), T)
        # h, shared h, fp16 routed outputs, their exponents (one byte per 32
        # columns of a token, slots padded to MOE_MAX_TOPK)
        staged = 2 * (T * k * I + T * I + T * k * d) + T * (d // 32) * _abi.MOE_MAX_TOPK
        # decode region for up to MOE_MAX_DECODE_TOKENS tokens: router partial
        # sums, logits, h of the k + 1 experts per token, the shared expert's
        # fp32 down outputs
        nt = _abi.MOE_MAX_DECODE_TOKENS
        dec = (4 * -(-d // _abi.MOE_DECODE_ROUTER_ROWS) * nt * E + 4 * nt * E + 2 * nt * (k + 1) * I
               + 4 * nt * d)
        assert staged + dec <= n <= staged + dec + 64 * 1024
    bad = _layer(d=100)
    assert lib.moe_workspace_bytes(C.addressof(bad), 16) == 0


def test_router_loads_stay_inside_their_k_slice():
    # The router kernel's waves each take one eighth of d; a lane of wave w
    # reads 8 consecutive k from kk at every padded K-step.  For every d the
    # ABI accepts, every read [kk, kk + 8) lies in [w*d/8, (w+1)*d/8) (so it
    # stays inside x and W_r), and every in-range step reads where it computes.
    S, waves = 4, 8
    for d in range(64, _abi.MOE_MAX_D + 1, 64):
        kq = d // waves
        n_steps = -(-(kq // 16 + (kq % 16 != 0)) // S) * S
        for w in range(waves):
            kbeg, kend = w * kq, (w + 1) * kq
            for step in range(n_steps + S - 1):  # the loads run S - 1 steps ahead
                k = kbeg + 16 * step
                for half in (0, 1):
                    kk = k + 8 * half if k + 8 * half + 8 <= kend else kbeg
                    assert kbeg <= kk and kk + 8 <= kend, (d, w, step, half)
                    if k + 8 * half < kend:
                        assert kk == k + 8 * half


def test_gate_up_activation_pieces_stay_inside_their_row():
    # The gate/up kernel stages 128-column chunks of gathered x rows, 16 bytes
    # (8 columns) per lane at logical slot s of the chunk; the pipeline runs
    # whole four-chunk groups, so chunks may lie partly or wholly past K.  For
    # every d the ABI accepts, every piece read lies inside its row of x, and
    # every piece inside K is read from where it is used.
    for d in range(64, _abi.MOE_MAX_D + 1, 64):
        n_chunks = -(-d // 128)
        n_run = -(-n_chunks // 4) * 4
        for c in range(n_run):
            for slot in range(16):
                col = c * 128 + 8 * slot
                got = col if col < d else (8 * slot) & 63
                assert 0 <= got and got + 8 <= d, (d, c, slot)
                if col < d:
                    assert got == col


def test_static_scratch_decode_validates_before_launch():
    lib = _abi.lib()
    L = _layer()
    assert lib.moe_decode_tokens_static(C.addressof(L), FAKE, 9, 0, None, FAKE,
                                        None) == _abi.MOE_EUNSUPPORTED
    assert lib.moe_decode_tokens_static(C.addressof(L), FAKE, 1, 2, None, FAKE,
                                        None) == _abi.MOE_EINVAL
    assert lib.moe_decode_tokens_static(C.addressof(L), FAKE, 1, 0, None, None,
                                        None) == _abi.MOE_EINVAL
    bad = _layer(d=100)
    assert lib.moe_decode_tokens_static(C.addressof(bad), FAKE, 1, 0, None, FAKE,
                                        None) == _abi.MOE_EUNSUPPORTED


def test_block_map_capacity_bounds_the_tile_count():
    lib = _abi.lib()
    # sum over experts of ceil(c/rows) <= floor(T*k/rows) + min(E, T*k)
    assert lib.moe_block_map_capacity(2048, 8, 256, 32) == 512 + 256
    assert lib.moe_block_map_capacity(2048, 8, 256, 128) == 128 + 256
    assert lib.moe_block_map_capacity(1, 8, 256, 32) == 0 + 8
    assert lib.moe_block_map_capacity(0, 8, 256, 32) == 0


def test_dequant_rejects_bad_shapes():
    lib = _abi.lib()
    m = _abi.Q4Mat(FAKE, FAKE, FAKE)
    assert lib.moe_dequant(C.addressof(m), 4, 100, FAKE, None) == _abi.MOE_EUNSUPPORTED
    assert lib.moe_dequant(C.addressof(m), 0, 64, FAKE, None) == _abi.MOE_EINVAL
    assert lib.moe_dequant(None, 4, 64, FAKE, None) == _abi.MOE_EINVAL


def test_strerror_names_every_code():
    lib = _abi.lib()
    names = {lib.moe_strerror(c) for c in (0, -1, -2, -3, -4)}
    assert len(names) == 5


def _lm(V=248320, d=2048, embed=True):
    m = _abi.Q4Mat(FAKE, FAKE, FAKE)
    return _abi.LmHead(V, d, m, _abi.Q4Mat(FAKE, FAKE, FAKE) if embed else _abi.Q4Mat())


def _lm_call(lm, x=FAKE, flags=0, logits=FAKE, token=FAKE, x_next=None, ws=FAKE, ws_bytes=1 << 30):
    return _abi.lib().moe_lm_argmax(C.addressof(lm), x, flags, logits, token, x_next, ws, ws_bytes,
                                    None)


def test_lm_workspace_bytes():
    lib = _abi.lib()
    for V, parts in ((248320, 15520), (1, 1), (257, 17), (_abi.MOE_MAX_VOCAB, 65536)):
        lm = _lm(V)
        n = lib.moe_lm_workspace_bytes(C.addressof(lm))
        assert 8 * parts <= n <= 8 * parts + 512, (V, n)
    for bad in (_lm(0), _lm(d=100), _lm(_abi.MOE_MAX_VOCAB + 1), _lm(d=_abi.MOE_MAX_D + 64)):
        assert lib.moe_lm_workspace_bytes(C.addressof(bad)) == 0
    assert lib.moe_lm_workspace_bytes(None) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(V=0), _abi.MOE_EINVAL), (dict(d=-64), _abi.MOE_EINVAL),
    (dict(d=100), _abi.MOE_EUNSUPPORTED), (dict(V=_abi.MOE_MAX_VOCAB + 1), _abi.MOE_EUNSUPPORTED),
])
def test_lm_argmax_rejects_unsupported_heads(kw, code):
    assert _lm_call(_lm(**kw)) == code


def test_lm_argmax_validates_before_launch():
    lib = _abi.lib()
    lm = _lm()
    need = lib.moe_lm_workspace_bytes(C.addressof(lm))
    assert _lm_call(lm, ws_bytes=need - 1) == _abi.MOE_EWORKSPACE
    assert _lm_call(lm, flags=2) == _abi.MOE_EINVAL
    assert _lm_call(lm, token=None) == _abi.MOE_EINVAL
    assert _lm_call(lm, token=FAKE + 2) == _abi.MOE_EINVAL
    assert b"token" in lib.moe_last_error()
    # a token slot needs only 4-byte alignment: this call gets as far as the workspace check
    assert _lm_call(lm, token=FAKE + 4, ws_bytes=need - 1) == _abi.MOE_EWORKSPACE
    assert _lm_call(lm, x=None) == _abi.MOE_EINVAL
    assert _lm_call(lm, logits=None) == _abi.MOE_EINVAL
    assert _lm_call(lm, x_next=FAKE + 8) == _abi.MOE_EINVAL
    assert _lm_call(_lm(embed=False), x_next=FAKE) == _abi.MOE_EINVAL
    assert b"embed" in lib.moe_last_error()
    # given logits need neither x nor the head
    nohead = _abi.LmHead(1000, 512, _abi.Q4Mat(), _abi.Q4Mat())
    assert _lm_call(nohead, x=None, flags=_abi.MOE_LOGITS_IN, ws_bytes=0) == _abi.MOE_EWORKSPACE
    assert _lm_call(nohead, x=None, flags=0, ws_bytes=0) == _abi.MOE_EINVAL
