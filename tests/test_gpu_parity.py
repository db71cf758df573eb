"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Bars:
  - dequantisation, routing indices, counts, offsets, perm, inv_perm and both
    block maps: bit-exact, routing done from the oracle's fp32 logits;
  - router logits: max |err| <= 1e-3 * RMS(oracle logits);
  - renormalised scores: |err| <= 2e-6 (fp32 against the oracle's fp64);
  - layer outputs (bf16): every element within 2e-2 * RMS(y_exact) of y_exact,
    the oracle's unrounded fp64 sum -- or, where rounding to bf16 alone can
    cost more than that (an output beyond about 5 RMS), within half a bf16
    ulp of y_exact plus 2e-3 * RMS (the fp32 sum-order noise that can move a
    value across a rounding midpoint); run-to-run bit-identical.
Full-size workloads are checked on the tokens of the first and last sorted
row of every 128-row work item of the grouped GEMMs and of every 32-token
block (the oracle computes each output token independently), so every work
item of every kernel is reached; small shapes on every token.  Routing on the
GPU's own logits must pick the oracle's expert set for every token whose k-th
and (k+1)-th oracle logits are further apart than twice the measured logit
error.
"""
import numpy as np
import pytest
import torch

import oracle
import q4_routed_expert_amd as q4
from workloads import (WORKLOADS, bits_to_f32, decode_inputs, make_layer, random_layer,
                       random_x)

pytestmark = pytest.mark.gpu

Y_TOL = 2e-2
Y_MIDPOINT_SLACK = 2e-3
LOGIT_TOL = 1e-3
W_TOL = 2e-6


def log(msg):
    print(f"[parity] {msg}", flush=True)


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def xdev(x, dev):
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(dev).view(torch.bfloat16)


def host_bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_half_ulp(v):
    """Half the spacing of bf16 numbers at |v| (8 significant bits; 0 at 0)."""
    _, e = np.frexp(np.abs(v))  # |v| in [2^(e-1), 2^e)
    return np.where(v == 0, 0.0, np.ldexp(1.0, e - 9))


def y_error(y_bits, y_exact):
    """(max |err| / RMS, RMS, worst err / allowed): allowed per element is
    max(Y_TOL * RMS, half a bf16 ulp of y_exact + Y_MIDPOINT_SLACK * RMS); the
    output passes when the last value is <= 1."""
    err = np.abs(bits_to_f32(y_bits).astype(np.float64) - y_exact)
    rms = float(np.sqrt(np.mean(y_exact ** 2)))
    allowed = np.maximum(Y_TOL * rms, bf16_half_ulp(y_exact) + Y_MIDPOINT_SLACK * rms)
    return float(err.max()) / rms, rms, float((err / allowed).max())


def compare_routing(r, ref, T, E, k, bm_ref, tm_ref):
    torch.cuda.synchronize()
    assert np.array_equal(r.topk_idx.cpu().numpy(), ref["idx"])
    assert np.abs(r.topk_w.cpu().numpy() - ref["w"]).max() <= W_TOL
    assert np.array_equal(r.counts.cpu().numpy(), ref["counts"])
    assert np.array_equal(r.offsets.cpu().numpy(), ref["offsets"])
    assert np.array_equal(r.perm.cpu().numpy(), ref["perm"])
    assert np.array_equal(r.inv_perm.cpu().numpy(), ref["inv_perm"])
    nb, nt = int(r.n_blocks.item()), int(r.n_tiles.item())
    assert nb == bm_ref[1] and nt == tm_ref[1]
    assert np.array_equal(r.block_map.cpu().numpy()[:nb], bm_ref[0])
    assert np.array_equal(r.tile_map.cpu().numpy()[:nt], tm_ref[0])


def oracle_routing(logits, k):
    ref = oracle.route(logits, k)
    bm = oracle.block_map(ref["counts"], ref["offsets"], q4.BLOCK_ROWS)
    tm = oracle.block_map(ref["counts"], ref["offsets"], q4.TILE_ROWS)
    return ref, bm, tm


def item_tokens(ref, T, k, items=None, seed=0):
    """Tokens of the first and last sorted row of every 128-row work item (or of
    `items` of them, drawn with `seed`, always including the first and the last
    items), plus the first and last token of every 32-token block (64-token
    above T = 16384, where the shared expert's items are 64 or 128 tokens):
    every work item of the grouped GEMMs and of the shared expert's GEMMs then
    has a compared output row."""
    tm, n = oracle.block_map(ref["counts"], ref["offsets"], q4.TILE_ROWS)
    sel = np.arange(n)
    if items is not None and items < n:
        rng = np.random.default_rng(seed)
        sel = np.unique(np.concatenate([[0, n - 1], rng.choice(n, items, replace=False)]))
    pick = set()
    for i in sel:
        e, r0 = int(tm[i, 0]), int(tm[i, 1])
        last = min(r0 + q4.TILE_ROWS, int(ref["offsets"][e + 1])) - 1
        pick.add(int(ref["perm"][r0]) // k)
        pick.add(int(ref["perm"][last]) // k)
    blk = 32 if T <= 16384 else 64
    for b in range(0, T, blk):
        pick.update((b, min(b + blk - 1, T - 1)))
    return np.array(sorted(pick), np.int32)


def check_own_routing(l_gpu, l_ref, own_idx, ref_idx, k):
    """Tokens whose expert set from the GPU's own logits differs from the
    oracle's; every such token must have its k-th and (k+1)-th oracle logits
    within twice the largest logit error of each other (a near tie)."""
    differ = (np.sort(own_idx, 1) != np.sort(ref_idx, 1)).any(1)
    E = l_ref.shape[1]
    if k < E:
        srt = -np.sort(-l_ref.astype(np.float64), axis=1)
        gap = srt[:, k - 1] - srt[:, k]
        bound = 2.0 * float(np.abs(l_gpu.astype(np.float64) - l_ref).max())
        assert not (differ & (gap > bound)).any(), \
            f"expert sets differ on tokens {np.where(differ & (gap > bound))[0][:8]} " \
            f"whose k-th logit gap exceeds {bound:.2e}"
    else:
        assert not differ.any()
    return int(differ.sum())


def run_layer_case(L, x, dev, tokens=None, name="", items=None):
    """Route on the GPU from the oracle's logits, run prefill, compare.
    tokens: None (every token), "items" (item_tokens, at most `items` work
    items) or an array of token indices."""
    T, E, k = x.shape[0], L["n_experts"], L["top_k"]
    layer = q4.DeviceLayer.from_host(L, dev)
    xd = xdev(x, dev)
    l_ref = oracle.router_logits(x, L["w_router"], L.get("router_bias"))
    # router logits computed on the GPU
    r_own = q4.route(layer, xd)
    torch.cuda.synchronize()
    l_gpu = r_own.logits.cpu().numpy()
    lrms = float(np.sqrt(np.mean(l_ref.astype(np.float64) ** 2)))
    lerr = float(np.abs(l_gpu.astype(np.float64) - l_ref).max()) / lrms
    own_idx = r_own.topk_idx.cpu().numpy()
    # routing from identical logits: bit-exact
    ref, bm, tm = oracle_routing(l_ref, k)
    r = q4.DeviceRouting(T, E, k, dev)
    r.logits.copy_(torch.from_numpy(l_ref))
    q4.route(layer, xd, routing=r, logits_in=True)
    compare_routing(r, ref, T, E, k, bm, tm)
    differ = check_own_routing(l_gpu, l_ref, own_idx, ref["idx"], k)
    ws = q4.workspace(layer, T, dev)
    y = q4.prefill(layer, xd, r, ws)
    y2 = q4.prefill(layer, xd, r, ws)
    torch.cuda.synchronize()
    yb, yb2 = host_bits(y), host_bits(y2)
    assert np.array_equal(yb, yb2), "prefill is not run-to-run deterministic"
    if tokens is None:
        tokens = np.arange(T, dtype=np.int32)
    elif isinstance(tokens, str):
        tokens = item_tokens(ref, T, k, items)
    y_exact, _ = oracle.layer_tokens(L, x, tokens, ref["idx"], ref["w"])
    err, rms, worst = y_error(yb[tokens], y_exact)
    log(f"{name} T={T} E={E} k={k}: logits err/rms={lerr:.2e}, tokens whose expert set "
        f"differs on GPU logits={differ}, y max err/rms={err:.3e}, worst err/allowed="
        f"{worst:.3f} (rms {rms:.3f}, {len(tokens)} tokens)")
    assert lerr <= LOGIT_TOL
    assert worst <= 1.0
    return err


# ------------------------------------------------------------------ dequantisation

def test_dequant_bit_exact(dev):
    rng = np.random.default_rng(7)
    Lr = random_layer(rng, d=512, inter=96 * 2, E=2, k=1)
    for name in ("gate", "down"):
        q, s, b = Lr[name + "_q"][1], Lr[name + "_s"][1], Lr[name + "_b"][1]
        ref = oracle.dequant(q, s, b)
        got = q4.dequant(q4._dev(q, dev), q4._dev(s, dev), q4._dev(b, dev))
        assert np.array_equal(host_bits(got), ref)
    # exact round-to-nearest-even ties: w = 1 + q/256 with bf16 spacing 2^-7
    q = np.array([[0x76543210, 0xFEDCBA98] * 4], np.uint32)
    s = np.array([[0x3B80]], np.uint16)
    b = np.array([[0x3F80]], np.uint16)
    got = q4.dequant(q4._dev(q, dev), q4._dev(s, dev), q4._dev(b, dev))
    assert np.array_equal(host_bits(got), oracle.dequant(q, s, b))
    # wide ranges: scales from 2^-107 to 2^73 of either sign (and zero), biases
    # within 2^+-10 of the scale, where q*scale + bias is exact in fp32
    N, K = 64, 512
    q = rng.integers(0, 1 << 32, size=(N, K // 8), dtype=np.uint32)
    es = rng.integers(20, 200, size=(N, K // 64))
    eb = np.clip(es + rng.integers(-10, 11, size=es.shape), 1, 254)
    sign = lambda: rng.integers(0, 2, size=es.shape) << 15
    s = (sign() | (es << 7) | rng.integers(0, 128, size=es.shape)).astype(np.uint16)
    b = (sign() | (eb << 7) | rng.integers(0, 128, size=es.shape)).astype(np.uint16)
    s[0, :] = 0
    got = q4.dequant(q4._dev(q, dev), q4._dev(s, dev), q4._dev(b, dev))
    assert np.array_equal(host_bits(got), oracle.dequant(q, s, b))


# ------------------------------------------------------------------ workloads

@pytest.mark.parametrize("name", ["tiny", "prefill512", "prefill2048", "skew4096"])
def test_workload_layer(name, dev):
    # every work item of the grouped GEMMs reached: the first and last rows of
    # each 128-row item of the hottest and of the rarest experts alike
    w = WORKLOADS[name]
    L, x = make_layer(w)
    run_layer_case(L, x, dev, None if w.T <= 64 else "items", name)


def test_decode_workload(dev):
    w = WORKLOADS["decode"]
    xs = decode_inputs(w, 6)
    for layer_i, steps in ((0, (0, 1, 2)), (7, (3, 4, 5))):
        L, _ = make_layer(w, layer_i)
        layer = q4.DeviceLayer.from_host(L, dev)
        ws = q4.workspace(layer, 1, dev)
        for st in steps:
            x = xs[st:st + 1]
            xd = xdev(x, dev)
            ref_all = oracle.layer(L, x)
            r = q4.DeviceRouting(1, w.n_experts, w.top_k, dev)
            y_own = q4.decode(layer, xd, ws, routing=r)
            torch.cuda.synchronize()
            l_gpu = r.logits.cpu().numpy()
            lrms = float(np.sqrt(np.mean(ref_all["logits"].astype(np.float64) ** 2)))
            lerr = float(np.abs(l_gpu - ref_all["logits"]).max()) / lrms
            # from identical logits: same experts, same scores, y within tolerance
            r.logits.copy_(torch.from_numpy(ref_all["logits"]))
            y = q4.decode(layer, xd, ws, routing=r, logits_in=True)
            y_again = q4.decode(layer, xd, ws, routing=r, logits_in=True)
            torch.cuda.synchronize()
            assert np.array_equal(r.topk_idx.cpu().numpy(), ref_all["idx"])
            assert np.abs(r.topk_w.cpu().numpy() - ref_all["w"]).max() <= W_TOL
            err, rms, worst = y_error(host_bits(y), ref_all["y_exact"])
            err_own, _, _ = y_error(host_bits(y_own), ref_all["y_exact"])
            assert np.array_equal(host_bits(y), host_bits(y_again))
            log(f"decode layer {layer_i} step {st}: logits err/rms={lerr:.2e}, y err/rms="
                f"{err:.3e} (own routing {err_own:.3e}), rms {rms:.3f}")
            assert lerr <= LOGIT_TOL
            assert worst <= 1.0


def _decode_tokens_case(L, xs, dev, name):
    """moe_decode_tokens on T tokens: every output, the logits and the routing
    bit-equal to T single-token moe_decode calls; from the oracle's logits the
    same experts and scores as the oracle and y within tolerance."""
    T, E, k = xs.shape[0], L["n_experts"], L["top_k"]
    layer = q4.DeviceLayer.from_host(L, dev)
    ws = q4.workspace(layer, 1, dev)
    xd = xdev(xs, dev)
    r = q4.DeviceRouting(T, E, k, dev)
    y = q4.decode_tokens(layer, xd, ws, routing=r)
    torch.cuda.synchronize()
    y_bits, l_gpu = host_bits(y), r.logits.cpu().numpy()
    idx_gpu, w_gpu = r.topk_idx.cpu().numpy(), r.topk_w.cpu().numpy()
    for t in range(T):
        r1 = q4.DeviceRouting(1, E, k, dev)
        y1 = q4.decode(layer, xd[t:t + 1], ws, routing=r1)
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(y1)[0], y_bits[t]), (name, t)
        assert np.array_equal(r1.logits.cpu().numpy()[0], l_gpu[t]), (name, t)
        assert np.array_equal(r1.topk_idx.cpu().numpy()[0], idx_gpu[t]), (name, t)
        assert np.array_equal(r1.topk_w.cpu().numpy()[0], w_gpu[t]), (name, t)
    ref = oracle.layer(L, xs)
    lrms = float(np.sqrt(np.mean(ref["logits"].astype(np.float64) ** 2)))
    lerr = float(np.abs(l_gpu - ref["logits"]).max()) / lrms
    r.logits.copy_(torch.from_numpy(ref["logits"]))
    y2 = q4.decode_tokens(layer, xd, ws, routing=r, logits_in=True)
    torch.cuda.synchronize()
    assert np.array_equal(r.topk_idx.cpu().numpy(), ref["idx"])
    assert np.abs(r.topk_w.cpu().numpy() - ref["w"]).max() <= W_TOL
    err, rms, worst = y_error(host_bits(y2), ref["y_exact"])
    log(f"decode_tokens {name} T={T}: logits err/rms={lerr:.2e}, y err/rms={err:.3e}, rms {rms:.3f}")
    assert lerr <= LOGIT_TOL
    assert worst <= 1.0


def test_decode_tokens_workload(dev):
    # the decode workload's layer 3 on T = 2, 3, 5 and 8 of its step inputs
    w = WORKLOADS["decode"]
    L, _ = make_layer(w, 3)
    xs = decode_inputs(w, 8)
    for T in (2, 3, 5, 8):
        _decode_tokens_case(L, xs[:T], dev, "decode workload")


def test_decode_tokens_small_shapes(dev):
    rng = np.random.default_rng(11)
    for T, d, inter, E, k, bias in ((3, 320, 128, 37, 5, True), (8, 256, 128, 8, 8, False),
                                    (1, 576, 192, 40, 3, True), (6, 512, 64, 16, 1, False),
                                    (8, 8192, 128, 8, 2, False),   # the largest d, 8 tokens
                                    (2, 1024, 2048, 16, 8, True)):  # the largest inter
        L = random_layer(rng, d, inter, E, k, router_bias=bias)
        _decode_tokens_case(L, random_x(rng, T, d), dev, f"d={d} I={inter} E={E} k={k}")


# ------------------------------------------------------------------ edge cases

EDGE = [
    # (T, d, inter, E, k, router_bias, seed)
    (1, 256, 128, 8, 2, False, 1),        # single token
    (33, 576, 192, 40, 3, False, 2),      # K not a multiple of 128, E not of 64, odd k
    (600, 256, 128, 4, 2, False, 3),      # several 128-row tiles per expert, ragged tails
    (70, 256, 128, 8, 8, False, 4),       # k = E: every expert selected
    (100, 256, 128, 256, 8, False, 5),    # most experts empty
    (129, 256, 64, 16, 1, True, 6),       # k = 1, one row past a tile
    (90, 320, 128, 37, 5, True, 7),       # E not a multiple of 4 (router column loads), d = 5 x 64
    (100, 512, 576, 8, 2, False, 8),      # inter > 512 and not a multiple of 512: chunked down GEMM
    (70, 1024, 2048, 8, 2, True, 9),      # the largest inter (chunked down GEMM)
    (40, 8192, 128, 8, 2, False, 10),     # the largest d
    (300, 512, 512, 16, 4, True, 11),     # inter = 512: the resident down GEMM with one scale
                                          # load per unit, several items per expert, ragged tails
    (300, 512, 448, 16, 4, True, 12),     # inter = 448: the resident down GEMM, odd group count
    (257, 64, 512, 8, 3, False, 13),      # the smallest d (router with one K-step per wave)
    (130, 2048, 128, 40, 3, True, 14),    # router staged through LDS: ragged token and
                                          # expert tiles (rows and columns clamped)
]


@pytest.mark.parametrize("T,d,inter,E,k,bias,seed", EDGE)
def test_edge_shapes(T, d, inter, E, k, bias, seed, dev):
    rng = np.random.default_rng(1000 + seed)
    L = random_layer(rng, d, inter, E, k, router_bias=bias)
    x = random_x(rng, T, d)
    run_layer_case(L, x, dev, None, f"edge{seed}")


def test_gate_up_round_robin_schedule(dev):
    # more gate/up work items than the grouped schedule takes at inter = 2048
    # (16 column blocks per item): the kernel falls back to its round-robin
    # unit list; the routed down projection runs chunked
    rng = np.random.default_rng(1013)
    T, d, inter, E, k = 30000, 64, 2048, 32, 8
    L = random_layer(rng, d, inter, E, k)
    x = random_x(rng, T, d)
    ref = oracle.route(oracle.router_logits(x, L["w_router"]), k)
    n_tiles = oracle.block_map(ref["counts"], ref["offsets"], q4.TILE_ROWS)[1]
    n_items = n_tiles + (T + 63) // 64
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    n_cb = inter // 128
    grouped_bound = 512 * 8 * ((cus // 8) // n_cb) // 4
    assert n_items > grouped_bound, (n_items, grouped_bound)
    run_layer_case(L, x, dev, "items", "round-robin gate/up", items=300)


@pytest.mark.parametrize("T,d,inter,E,k,bias,seed", [
    (600, 256, 128, 4, 2, False, 3),     # several 128-row tiles per expert, ragged tails
    (300, 512, 512, 16, 4, True, 11),    # the resident down GEMM after gate/up
    (100, 256, 128, 256, 8, False, 5),   # most experts empty: most parts of tiles empty
    (20000, 64, 512, 256, 8, True, 14),  # at 32-row items more items than the grouped
                                         # schedule takes: the round-robin unit list
])
def test_item_rows_variants(T, d, inter, E, k, bias, seed, dev):
    # the gate/up work item at 64, 32 and 16 rows: every row's products are
    # accumulated in the same order as at 128 rows, so y is bit-identical; the
    # 32-row run is also compared with the oracle
    rng = np.random.default_rng(2000 + seed)
    L = random_layer(rng, d, inter, E, k, router_bias=bias)
    x = random_x(rng, T, d)
    layer = q4.DeviceLayer.from_host(L, dev)
    xd = xdev(x, dev)
    l_ref = oracle.router_logits(x, L["w_router"], L.get("router_bias"))
    ref, bm, tm = oracle_routing(l_ref, k)
    r = q4.DeviceRouting(T, E, k, dev)
    r.logits.copy_(torch.from_numpy(l_ref))
    q4.route(layer, xd, routing=r, logits_in=True)
    compare_routing(r, ref, T, E, k, bm, tm)
    n_items32 = 4 * int(r.n_tiles.cpu()[0]) + (T + 63) // 64
    ws = q4.workspace(layer, T, dev)
    ys = {m: host_bits(q4.prefill(layer, xd, r, ws, item_rows=m)) for m in (128, 64, 32, 16)}
    torch.cuda.synchronize()
    for m in (64, 32, 16):
        assert np.array_equal(ys[m], ys[128]), f"item_rows={m} differs from 128"
    tokens = np.arange(T, dtype=np.int32) if T <= 600 else item_tokens(ref, T, k)
    y_exact, _ = oracle.layer_tokens(L, x, tokens, ref["idx"], ref["w"])
    err, rms, worst = y_error(ys[32][tokens], y_exact)
    log(f"item rows T={T} E={E} k={k}: 32-row items ({n_items32} gate/up items), y max "
        f"err/rms={err:.3e}, worst err/allowed={worst:.3f} ({len(tokens)} tokens)")
    assert worst <= 1.0
    with pytest.raises(ValueError):
        q4.prefill(layer, xd, r, ws, item_rows=48)


def test_prefill_at_the_token_limit(dev):
    # T = 32768 (the limit): more gate/up items than one thread of the
    # schedule's 512 covers five at a time; every work item compared
    rng = np.random.default_rng(1014)
    T, d, inter, E, k = 32768, 64, 512, 256, 8
    L = random_layer(rng, d, inter, E, k, router_bias=True)
    x = random_x(rng, T, d)
    run_layer_case(L, x, dev, "items", "T=32768")


def test_large_magnitudes(dev):
    # x scaled by 1024 (exact in bf16): the routed experts' outputs reach far
    # past fp16's largest finite value (65504); the staged partials must keep
    # them
    rng = np.random.default_rng(1015)
    T, d, inter, E, k = 96, 512, 128, 32, 4
    L = random_layer(rng, d, inter, E, k)
    x = bits_to_f32(random_x(rng, T, d)) * np.float32(1024.0)
    from workloads import bf16_bits
    x = bf16_bits(x)
    r = oracle.route(oracle.router_logits(x, L["w_router"]), k)
    big = max(float(np.abs(oracle.expert(L, int(r["idx"][t, 0]), x[t])[1]).max())
              for t in range(4))
    assert big > 65504.0 * 4, big
    err = run_layer_case(L, x, dev, None, "x * 1024")
    log(f"large magnitudes: largest routed output {big:.3e}, y err/rms {err:.3e}")


def test_all_tokens_pick_the_same_experts(dev):
    # a dominant router bias sends every token to experts 5, 2, 9, 0: four
    # experts with T rows each (several tiles), every other expert empty
    rng = np.random.default_rng(77)
    T, E, k = 300, 32, 4
    L = random_layer(rng, 256, 128, E, k, router_bias=True)
    L["router_bias"] = np.zeros(E, np.float32)
    L["router_bias"][[5, 2, 9, 0]] = [40.0, 30.0, 20.0, 10.0]
    x = random_x(rng, T, 256)
    run_layer_case(L, x, dev, None, "one-hot")


def test_routing_ties_and_signed_zeros(dev):
    # coarse logits with many exact ties (and -0.0 vs +0.0) given to the GPU
    rng = np.random.default_rng(8)
    T, E, k = 257, 64, 8
    L = random_layer(rng, 128, 64, E, k)
    l = (np.round(rng.standard_normal((T, E)) * 2) / 2).astype(np.float32)
    l[l == 0] = np.where(rng.random(int((l == 0).sum())) < 0.5, -0.0, 0.0)
    layer = q4.DeviceLayer.from_host(L, dev)
    ref, bm, tm = oracle_routing(l, k)
    r = q4.DeviceRouting(T, E, k, dev)
    r.logits.copy_(torch.from_numpy(l))
    q4.route(layer, xdev(random_x(rng, T, 128), dev), routing=r, logits_in=True)
    compare_routing(r, ref, T, E, k, bm, tm)


def test_routing_at_the_token_limit(dev):
    rng = np.random.default_rng(9)
    T, E, k = 32768, 256, 8
    L = random_layer(rng, 64, 64, E, k)
    l = rng.standard_normal((T, E)).astype(np.float32)
    l[:, 17] += 2.5  # one hot expert with ~T rows
    layer = q4.DeviceLayer.from_host(L, dev)
    ref, bm, tm = oracle_routing(l, k)
    r = q4.DeviceRouting(T, E, k, dev)
    r.logits.copy_(torch.from_numpy(l))
    q4.route(layer, xdev(np.zeros((T, 64), np.uint16), dev), routing=r, logits_in=True)
    compare_routing(r, ref, T, E, k, bm, tm)
    log(f"routing T={T}: n_blocks={bm[1]} n_tiles={tm[1]} max count={ref['counts'].max()}")


def test_small_decode_shapes(dev):
    rng = np.random.default_rng(10)
    for d, inter, E, k, bias in ((576, 192, 40, 3, True), (256, 128, 8, 8, False),
                                 (320, 128, 37, 5, True)):
        L = random_layer(rng, d, inter, E, k, router_bias=bias)
        layer = q4.DeviceLayer.from_host(L, dev)
        ws = q4.workspace(layer, 1, dev)
        x = random_x(rng, 1, d)
        ref = oracle.layer(L, x)
        r = q4.DeviceRouting(1, E, k, dev)
        q4.decode(layer, xdev(x, dev), ws, routing=r)  # the decode path's own router
        torch.cuda.synchronize()
        lrms = float(np.sqrt(np.mean(ref["logits"].astype(np.float64) ** 2)))
        lerr = float(np.abs(r.logits.cpu().numpy() - ref["logits"]).max()) / lrms
        log(f"decode d={d} E={E}: logits err/rms={lerr:.3e}")
        assert lerr <= LOGIT_TOL
        r.logits.copy_(torch.from_numpy(ref["logits"]))
        y = q4.decode(layer, xdev(x, dev), ws, routing=r, logits_in=True)
        torch.cuda.synchronize()
        assert np.array_equal(r.topk_idx.cpu().numpy(), ref["idx"])
        err, _, worst = y_error(host_bits(y), ref["y_exact"])
        log(f"decode d={d} I={inter} E={E} k={k}: y err/rms={err:.3e}")
        assert worst <= 1.0


# ------------------------------------------------------------------ graph capture

def test_graph_replays_match_eager(dev):
    # One prefill layer call (route + prefill) and one few-token decode call
    # captured in a HIP graph; every replay, with eager calls on other inputs
    # in between, must reproduce the eager outputs bit for bit.
    rng = np.random.default_rng(21)
    T, d, inter, E, k = 300, 256, 128, 32, 4
    L = random_layer(rng, d, inter, E, k, router_bias=True)
    layer = q4.DeviceLayer.from_host(L, dev)
    xa, xb = xdev(random_x(rng, T, d), dev), xdev(random_x(rng, T, d), dev)
    r = q4.DeviceRouting(T, E, k, dev)
    ws = q4.workspace(layer, T, dev)
    y = torch.empty((T, d), dtype=torch.bfloat16, device=dev)
    yd = torch.empty((5, d), dtype=torch.bfloat16, device=dev)
    gx = xa.clone()

    def calls(x_in):
        q4.route(layer, x_in, routing=r)
        q4.prefill(layer, x_in, r, ws, y)
        q4.decode_tokens(layer, x_in[:5], ws, yd)

    calls(gx)
    torch.cuda.synchronize()
    y_ref, yd_ref = host_bits(y), host_bits(yd)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls(gx)
    torch.cuda.synchronize()
    for rep in range(3):
        calls(xb)  # eager work on other inputs between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(y), y_ref), f"prefill replay {rep}"
        assert np.array_equal(host_bits(yd), yd_ref), f"decode replay {rep}"
    log("graph replays: prefill and few-token decode equal to eager on 3 replays")
