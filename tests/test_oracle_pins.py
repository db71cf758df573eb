"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test fixes a part of the oracle with something independent of it: values
derived by hand from the definitions (tests/golden/closed_form.json), numbers
the pages print (tests/golden/page_numbers.json), library routines that a
special case reduces to (numpy matmul, numpy stable argsort, scipy softmax,
torch's bf16 conversion, Python's sorted), closed forms and invariants.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from workloads import bits_to_f32, random_layer, random_x, WORKLOADS, make_layer

GOLD = os.path.join(os.path.dirname(__file__), "golden")
CF = json.load(open(os.path.join(GOLD, "closed_form.json")))
PAGE = json.load(open(os.path.join(GOLD, "page_numbers.json")))


def _hex(s):
    return int(s, 16)


def _word(codes):
    return sum(int(c) << (4 * i) for i, c in enumerate(codes))


def _torch_bf16(v):
    return torch.from_numpy(np.asarray(v, np.float32)).to(torch.bfloat16).view(torch.int16) \
        .numpy().view(np.uint16)


def const_q4(n_mat, N, K, code, scale_bits, bias_bits):
    q = np.full((n_mat, N, K // 8), _word([code] * 8), np.uint32)
    s = np.full((n_mat, N, K // 64), scale_bits, np.uint16)
    b = np.full((n_mat, N, K // 64), bias_bits, np.uint16)
    return q, s, b


def set_mat(L, name, qsb):
    L[name + "_q"], L[name + "_s"], L[name + "_b"] = qsb


def zero_mat(L, name):
    """Exactly-zero weights: code 8, scale 2^-7, bias -8 * 2^-7."""
    q = L[name + "_q"]
    set_mat(L, name, const_q4(q.shape[0], q.shape[1], q.shape[2] * 8, 8, 0x3C00, 0xBD80))


# ---------------------------------------------------------------- dequantisation

def test_dequant_nibble_order_from_hand_built_words():
    # scale 2^-7, bias -2^-4: w = (q - 8)/128 is exact, so w identifies q
    tab = CF["dequant_exact"]["w_for_codes_0_to_15"]
    for case in CF["dequant_words"]:
        q = np.array([[_hex(case["word"])] * 8], np.uint32)  # one row, K = 64
        s = np.array([[_hex(CF["dequant_exact"]["scale_bits"])]], np.uint16)
        b = np.array([[_hex(CF["dequant_exact"]["bias_bits"])]], np.uint16)
        w = bits_to_f32(oracle.dequant(q, s, b))[0]
        expect = [tab[c] for c in case["codes"]] * 8
        assert w.tolist() == expect


def test_dequant_exact_values_and_zero_point():
    c = CF["dequant_exact"]
    q = np.array([[_word(range(8)), _word(range(8, 16))] * 4], np.uint32)
    s = np.array([[_hex(c["scale_bits"])]], np.uint16)
    b = np.array([[_hex(c["bias_bits"])]], np.uint16)
    w = bits_to_f32(oracle.dequant(q, s, b))[0]
    assert w.tolist() == c["w_for_codes_0_to_15"] * 4
    # q = 8 with bias = -8*scale exactly gives +0.0
    assert oracle.dequant(q, s, b)[0, 8] == 0


def test_dequant_round_to_nearest_even_on_exact_ties():
    c = CF["dequant_ties"]
    q = np.array([[_word(c["codes"])] * 8], np.uint32)
    s = np.array([[_hex(c["scale_bits"])]], np.uint16)
    b = np.array([[_hex(c["bias_bits"])]], np.uint16)
    w = bits_to_f32(oracle.dequant(q, s, b))[0]
    assert w[:8].tolist() == c["w"]


def test_dequant_group_index_follows_k():
    # two groups of 64 along K with different scales: column k uses group k // 64
    q = np.array([[_word([15] * 8)] * 16], np.uint32)  # K = 128, every code 15
    s = np.array([[0x3C00, 0x3C80]], np.uint16)  # 2^-7, 2^-6
    b = np.array([[0x0000, 0x0000]], np.uint16)
    w = bits_to_f32(oracle.dequant(q, s, b))[0]
    assert np.all(w[:64] == 15 * 2.0 ** -7) and np.all(w[64:] == 15 * 2.0 ** -6)
    # and rows use their own groups
    q2 = np.repeat(q, 2, axis=0)
    s2 = np.array([[0x3C00, 0x3C00], [0x3C80, 0x3C80]], np.uint16)
    b2 = np.zeros((2, 2), np.uint16)
    w2 = bits_to_f32(oracle.dequant(q2, s2, b2))
    assert np.all(w2[0] == 15 * 2.0 ** -7) and np.all(w2[1] == 15 * 2.0 ** -6)


def test_dequant_matches_library_rounding_on_random_groups():
    # q*scale+bias is exact in float64 and (for these distributions) in float32;
    # torch's float32 -> bf16 conversion is round-to-nearest-even
    rng = np.random.default_rng(11)
    L = random_layer(rng, d=256, inter=64, E=2, k=1)
    q, s, b = L["gate_q"][1], L["gate_s"][1], L["gate_b"][1]
    codes = ((q[:, :, None] >> (4 * np.arange(8, dtype=np.uint32))) & 15).reshape(64, 256)
    exact = codes * np.repeat(bits_to_f32(s).astype(np.float64), 64, 1) \
        + np.repeat(bits_to_f32(b).astype(np.float64), 64, 1)
    assert np.all(exact.astype(np.float32).astype(np.float64) == exact)
    assert np.array_equal(oracle.dequant(q, s, b), _torch_bf16(exact.astype(np.float32)))


def test_bf16_round_matches_library_on_float32_values():
    rng = np.random.default_rng(5)
    v = np.concatenate([rng.standard_normal(20000).astype(np.float32) * 10.0 ** rng.integers(-40, 30, 20000),
                        # exact ties: bf16 value + half spacing
                        (bits_to_f32(rng.integers(0, 0x7F00, 5000).astype(np.uint16))
                         * np.float32(1 + 2.0 ** -8)).astype(np.float32),
                        np.float32([1e-40, -3e-39, 0.0, -0.0])]).astype(np.float32)
    v = v[np.isfinite(v) & (np.abs(v) < 3.3e38)]
    assert np.array_equal(oracle.bf16_round(v.astype(np.float64)), _torch_bf16(v))


# ---------------------------------------------------------------- router logits

def test_router_logits_match_float64_matmul():
    rng = np.random.default_rng(1)
    T, d, E = 7, 192, 24  # d != E catches a transposed router
    x = random_x(rng, T, d)
    W = (rng.standard_normal((d, E)) / math.sqrt(d)).astype(np.float32)
    bvec = rng.standard_normal(E).astype(np.float32)
    ref = bits_to_f32(x).astype(np.float64) @ W.astype(np.float64)
    got = oracle.router_logits(x, W)
    assert np.array_equal(got, ref.astype(np.float32)) or \
        np.max(np.abs(got - ref) / np.abs(ref)) < 2 ** -23
    got_b = oracle.router_logits(x, W, bvec)
    ref_b = ref + bvec.astype(np.float64)
    assert np.max(np.abs(got_b - ref_b) / np.abs(ref_b)) < 2 ** -23


# ---------------------------------------------------------------- routing

def _logits(rng, T, E, ties=False):
    l = rng.standard_normal((T, E)).astype(np.float32)
    if ties:  # coarse values force many equal logits, including -0.0 vs +0.0
        l = np.round(l * 2).astype(np.float32) / 2
        l[l == 0] = np.where(rng.random(np.count_nonzero(l == 0)) < 0.5, -0.0, 0.0)
    return l


@pytest.mark.parametrize("T,E,k,ties", [(64, 32, 4, False), (50, 8, 2, True), (33, 256, 8, True),
                                        (5, 4, 4, False), (17, 16, 1, True)])
def test_selection_is_stable_descending_sort(T, E, k, ties):
    rng = np.random.default_rng(T * 1000 + E)
    l = _logits(rng, T, E, ties)
    r = oracle.route(l, k)
    ref = np.argsort(-l, axis=1, kind="stable")[:, :k]
    assert np.array_equal(r["idx"], ref)
    for t in range(T):
        assert len(set(r["idx"][t].tolist())) == k


@pytest.mark.parametrize("T,E,k", [(40, 32, 4), (9, 256, 8), (12, 6, 3)])
def test_scores_closed_form(T, E, k):
    rng = np.random.default_rng(E)
    l = _logits(rng, T, E)
    r = oracle.route(l, k)
    w, idx = r["w"], r["idx"]
    assert np.allclose(w.sum(1), 1.0, atol=1e-14, rtol=0)
    assert np.all(w > 0) and np.all(np.diff(w, axis=1) <= 0)
    sel = np.take_along_axis(l, idx, 1).astype(np.float64)
    # ratios do not depend on the normaliser: w_s / w_0 = exp(l_s - l_0)
    assert np.allclose(w / w[:, :1], np.exp(sel - sel[:, :1]), rtol=1e-13, atol=0)


def test_scores_with_all_experts_selected_are_the_softmax():
    rng = np.random.default_rng(3)
    l = _logits(rng, 20, 8)
    r = oracle.route(l, 8)
    sm = scipy.special.softmax(l.astype(np.float64), axis=1)
    assert np.allclose(r["w"], np.take_along_axis(sm, r["idx"], 1), rtol=1e-13, atol=0)


def test_routing_closed_form_when_all_logits_tie():
    T, E, k = 70, 16, 4
    r = oracle.route(np.zeros((T, E), np.float32), k)
    assert np.array_equal(r["idx"], np.tile(np.arange(k, dtype=np.int32), (T, 1)))
    assert np.allclose(r["w"], 1.0 / k, rtol=1e-15, atol=0)
    assert r["counts"].tolist() == [T] * k + [0] * (E - k)
    assert r["offsets"].tolist() == [min(e, k) * T for e in range(E + 1)]
    exp_perm = np.array([t * k + e for e in range(k) for t in range(T)], np.int32)
    assert np.array_equal(r["perm"], exp_perm)
    bmap, n = oracle.block_map(r["counts"], r["offsets"], 32)
    tiles = math.ceil(T / 32)
    assert n == k * tiles
    assert bmap.tolist() == [[e, e * T + 32 * j] for e in range(k) for j in range(tiles)]


def _check_sorted_order(idx, r, E):
    k = idx.shape[1]
    flat = idx.reshape(-1)
    A = flat.size
    assert np.array_equal(r["counts"], np.bincount(flat, minlength=E))
    assert r["offsets"][0] == 0 and np.array_equal(np.diff(r["offsets"]), r["counts"])
    assert r["offsets"][-1] == A
    assert r["perm"].tolist() == sorted(range(A), key=lambda a: (flat[a], a))
    assert np.array_equal(r["inv_perm"][r["perm"]], np.arange(A))


@pytest.mark.parametrize("T,E,k", [(64, 32, 4), (100, 8, 2), (31, 256, 8), (3, 4, 4)])
def test_histogram_scan_scatter_against_library_sort(T, E, k):
    rng = np.random.default_rng(T + E + k)
    r = oracle.route(_logits(rng, T, E, ties=True), k)
    _check_sorted_order(r["idx"], r, E)


@pytest.mark.parametrize("bm", [32, 128, 1, 7])
def test_block_map_tiles_every_row_once(bm):
    rng = np.random.default_rng(bm)
    T, E, k = 300, 32, 4
    l = _logits(rng, T, E)
    l[:, 3] += 3.0  # one hot expert, some empty ones
    r = oracle.route(l, k)
    bmap, n = oracle.block_map(r["counts"], r["offsets"], bm)
    counts, offs = r["counts"], r["offsets"]
    assert n == sum(math.ceil(c / bm) for c in counts)
    covered = []
    for e, start in bmap:
        assert offs[e] <= start < offs[e + 1] and (start - offs[e]) % bm == 0
        covered.extend(range(start, min(start + bm, offs[e + 1])))
    assert covered == list(range(T * k))  # in order, each row once
    assert list(bmap[:, 0]) == sorted(bmap[:, 0])


def test_page_assignment_count_at_2k_tokens():
    # a 2K-token chunk with top-8 of 256 experts: 16,384 assignments, mean 64 rows per expert
    T, E, k = PAGE["prompt_tokens"], PAGE["n_experts"], PAGE["top_k"]
    rng = np.random.default_rng(2048)
    r = oracle.route(rng.standard_normal((T, E)).astype(np.float32), k)
    assert int(r["counts"].sum()) == PAGE["assignments"]
    assert r["counts"].mean() == PAGE["mean_rows_per_expert"]
    bmap, n = oracle.block_map(r["counts"], r["offsets"], PAGE["tile_rows"])
    assert n >= PAGE["assignments"] // PAGE["tile_rows"]


def test_workload_shapes_follow_the_page():
    w = WORKLOADS["prefill2048"]
    assert (w.n_experts, w.top_k, w.T) == (PAGE["n_experts"], PAGE["top_k"], PAGE["prompt_tokens"])


# ---------------------------------------------------------------- experts and layer

def _unit_layer(d, inter, E, k, gate_code=9, up_code=9, down_code=9):
    # scale 2^-6 (0x3C80), bias -8*2^-6 (0xBE00): w = (code - 8) * 2^-6
    L = {"d": d, "inter": inter, "n_experts": E, "top_k": k,
         "w_router": np.zeros((d, E), np.float32), "router_bias": None}
    set_mat(L, "gate", const_q4(E, inter, d, gate_code, 0x3C80, 0xBE00))
    set_mat(L, "up", const_q4(E, inter, d, up_code, 0x3C80, 0xBE00))
    set_mat(L, "down", const_q4(E, d, inter, down_code, 0x3C80, 0xBE00))
    for m, N, K in (("sh_gate", inter, d), ("sh_up", inter, d), ("sh_down", d, inter)):
        set_mat(L, m, const_q4(1, N, K, 8, 0x3C00, 0xBD80))
    return L


@pytest.mark.parametrize("case", ["expert_unit", "expert_unit_x2", "expert_unit_negative_up"])
def test_expert_closed_form(case):
    c = CF[case]
    base = CF["expert_unit"]
    d, inter = base["d"], base["inter"]
    L = _unit_layer(d, inter, E=2, k=1, gate_code=c.get("gate_code", 9),
                    up_code=c.get("up_code", 9))
    x = np.full((1, d), _torch_bf16([c["x"]])[0], np.uint16)
    h, P = oracle.expert(L, 1, x[0])
    assert np.all(bits_to_f32(h) == c["h"])
    assert np.all(P == c["y"])
    out = oracle.layer(L, x)  # all logits 0: expert 0 selected with weight 1; shared is zero
    assert out["idx"].tolist() == [[0]] and out["w"].tolist() == [[1.0]]
    assert np.all(out["y_exact"] == c["y"])
    if case == "expert_unit":
        assert np.all(out["y"] == _hex(c["y_bits"]))


def _dense_ffn(L, e, x_t):
    """Textbook SwiGLU FFN of expert e on one token: numpy float64 matmuls on the
    dequantised weights, SiLU from scipy, h rounded by torch's bf16 conversion."""
    pre = "sh_" if e < 0 else ""
    ee = 0 if e < 0 else e
    Wg = bits_to_f32(oracle.dequant(L[pre + "gate_q"][ee], L[pre + "gate_s"][ee],
                                    L[pre + "gate_b"][ee])).astype(np.float64)
    Wu = bits_to_f32(oracle.dequant(L[pre + "up_q"][ee], L[pre + "up_s"][ee],
                                    L[pre + "up_b"][ee])).astype(np.float64)
    Wd = bits_to_f32(oracle.dequant(L[pre + "down_q"][ee], L[pre + "down_s"][ee],
                                    L[pre + "down_b"][ee])).astype(np.float64)
    xv = bits_to_f32(x_t).astype(np.float64)
    g, u = Wg @ xv, Wu @ xv
    h = bits_to_f32(_torch_bf16((g * scipy.special.expit(g) * u).astype(np.float32)))
    return Wd @ h.astype(np.float64)


def _close(a, b, rel=1e-12):
    return np.max(np.abs(a - b)) <= rel * np.sqrt(np.mean(b ** 2))


def test_single_expert_layer_is_a_dense_swiglu_ffn():
    rng = np.random.default_rng(21)
    L = random_layer(rng, d=128, inter=64, E=1, k=1)
    for m in ("sh_gate", "sh_up", "sh_down"):
        zero_mat(L, m)
    x = random_x(rng, 6, 128)
    out = oracle.layer(L, x)
    assert np.all(out["w"] == 1.0)
    for t in range(6):
        assert _close(out["y_exact"][t], _dense_ffn(L, 0, x[t]))


def test_shared_expert_alone_when_routed_experts_are_zero():
    rng = np.random.default_rng(22)
    L = random_layer(rng, d=128, inter=64, E=4, k=2)
    for m in ("gate", "up", "down"):
        zero_mat(L, m)
    x = random_x(rng, 5, 128)
    out = oracle.layer(L, x)
    for t in range(5):
        assert _close(out["y_exact"][t], _dense_ffn(L, -1, x[t]))


def test_all_experts_selected_is_a_softmax_weighted_sum():
    rng = np.random.default_rng(23)
    E = 4
    L = random_layer(rng, d=64, inter=64, E=E, k=E, router_bias=True)
    x = random_x(rng, 4, 64)
    out = oracle.layer(L, x)
    sm = scipy.special.softmax(out["logits"].astype(np.float64), axis=1)
    for t in range(4):
        ref = sum(sm[t, e] * _dense_ffn(L, e, x[t]) for e in range(E)) + _dense_ffn(L, -1, x[t])
        assert _close(out["y_exact"][t], ref)


def test_identical_experts_need_renormalised_scores():
    # every routed expert equal: the selected scores sum to 1, so y = FFN(x) + shared(x)
    rng = np.random.default_rng(24)
    E = 8
    L = random_layer(rng, d=64, inter=64, E=E, k=2)
    for m in ("gate", "up", "down"):
        for suf in ("_q", "_s", "_b"):
            L[m + suf] = np.repeat(L[m + suf][:1], E, axis=0)
    x = random_x(rng, 6, 64)
    out = oracle.layer(L, x)
    for t in range(6):
        ref = _dense_ffn(L, 0, x[t]) + _dense_ffn(L, -1, x[t])
        assert _close(out["y_exact"][t], ref, rel=1e-12)


def test_outputs_are_bf16_of_the_exact_sum():
    rng = np.random.default_rng(25)
    L = random_layer(rng, d=64, inter=64, E=6, k=3)
    x = random_x(rng, 8, 64)
    out = oracle.layer(L, x)
    ye = out["y_exact"].astype(np.float32)
    # away from exact ties the library rounding of float32(y_exact) agrees
    assert np.mean(out["y"] == _torch_bf16(ye)) > 0.999


def test_output_bar_half_ulp_is_the_bf16_rounding_bound():
    # The GPU parity bar lets an output element be off by half a bf16 ulp of
    # the exact value (+ a small slack) where that exceeds 2e-2 * RMS.  The
    # helper's half ulp must bound the correct rounding's error everywhere and
    # be attained at midpoints: checked against the oracle's rounding.
    import test_gpu_parity as tgp
    rng = np.random.default_rng(26)
    v = rng.standard_normal(20000) * np.exp(rng.uniform(-20, 20, 20000))
    err = np.abs(bits_to_f32(oracle.bf16_round(v)).astype(np.float64) - v)
    assert (err <= tgp.bf16_half_ulp(v)).all()
    # midpoints between consecutive bf16 numbers: the error is exactly half an ulp
    lo = bits_to_f32(np.arange(0x3F80, 0x3FFF, dtype=np.uint16)).astype(np.float64)
    mid = (lo + bits_to_f32(np.arange(0x3F81, 0x4000, dtype=np.uint16))) / 2
    err = np.abs(bits_to_f32(oracle.bf16_round(mid)).astype(np.float64) - mid)
    assert np.array_equal(err, tgp.bf16_half_ulp(mid))
    assert tgp.bf16_half_ulp(np.array([0.0]))[0] == 0.0


def test_tiny_workload_layer_runs_and_is_deterministic():
    w = WORKLOADS["tiny"]
    L, x = make_layer(w)
    a = oracle.layer(L, x)
    b = oracle.layer(L, x, tokens=np.array([5, 0, 31], np.int32))
    assert a["y_exact"].shape == (w.T, w.d)
    assert np.array_equal(a["y_exact"][[5, 0, 31]], b["y_exact"])
    _check_sorted_order(a["idx"], a, w.n_experts)
    rms = np.sqrt(np.mean(a["y_exact"] ** 2))
    assert 0.05 < rms < 50


# ---------------------------------------------------------------- token hand-off

def test_lm_logits_match_float64_matmul():
    rng = np.random.default_rng(7)
    V, d = 37, 192  # V != d catches a transposed head
    from workloads import random_lm
    x, head, _ = random_lm(rng, V, d)
    W = bits_to_f32(oracle.dequant(head["q"], head["scale"], head["bias"])).astype(np.float64)
    ref = W @ bits_to_f32(x).astype(np.float64)
    got = oracle.lm_logits(x, head["q"], head["scale"], head["bias"])
    assert got.shape == (V,) and got.dtype == np.float32
    assert np.all(np.abs(got - ref) <= 2 ** -23 * np.abs(ref) + 1e-30)


def test_lm_logits_closed_form_per_row():
    # row v: every code c_v = v % 16, scale 2^-7, bias -8 * 2^-7, so every weight is
    # (c_v - 8) / 128 exactly; with x = 1 the logit is d * (c_v - 8) / 128.
    V, d = 40, 256
    codes = np.arange(V) % 16
    q = np.stack([np.full(d // 8, _word([c] * 8), np.uint32) for c in codes])
    s = np.full((V, d // 64), 0x3C00, np.uint16)
    b = np.full((V, d // 64), 0xBD80, np.uint16)
    x = np.full(d, 0x3F80, np.uint16)  # bf16 1.0
    got = oracle.lm_logits(x, q, s, b)
    assert np.array_equal(got, (d * (codes - 8) / 128).astype(np.float32))
    # greedy token: code 15 first appears at v = 15; the next input is its row
    lg, tok, nxt = oracle.lm_step({"q": q, "scale": s, "bias": b}, {"q": q, "scale": s, "bias": b}, x)
    assert tok == 15
    assert np.all(bits_to_f32(nxt) == np.float32(7 / 128))


@pytest.mark.parametrize("vals,want", [
    ([1, 3, 3, 2], 1),                          # equal maxima: the lower index
    ([float("nan"), -1, -2], 1),                # NaN counts as -inf
    ([float("nan")] * 5, 0),                    # all NaN: token 0
    ([-math.inf] * 3, 0),
    ([-math.inf, float("nan"), -5], 2),
    ([-0.0, 0.0], 0),                           # signed zeros are equal
    ([0.0, -0.0, 1e-45], 2),                    # the smallest subnormal beats zero
    ([2, float("nan"), 2], 0),
    ([5], 0),
    ([3.4e38, math.inf, 1], 1),
])
def test_argmax_hand_cases(vals, want):
    assert oracle.argmax(np.array(vals, np.float32)) == want


def test_argmax_matches_numpy_first_occurrence():
    rng = np.random.default_rng(3)
    for V in (1, 2, 1000, 100003):
        l = np.round(rng.standard_normal(V) * 4).astype(np.float32)  # many ties
        assert oracle.argmax(l) == int(np.argmax(l))
