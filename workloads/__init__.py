"""Seeded synthetic inputs for the routed-MoE Q4 FFN layer.

This module only draws random numbers and stores them in the layer's storage
formats.  It computes nothing the layer computes: no dequantisation, no
routing, no contraction.  Both the HIP path and the CPU oracle read the arrays
it returns, so it is the one piece of code the two sides share.

The layer shape is that of Qwen3.6-35B-A3B's MoE FFN as the page "Perplexity's
Lily beats MLX-LM on MacBook M5 because it only runs one model" describes it
(section "Why Qwen3.6-35B-A3B is a weird workload": 8 of 256 routed experts
per token plus 1 always-on shared expert), with the group-64 affine 4-bit
weight format of its section "Prefill: keep routing on the GPU, dequantize in
flight" (a bf16 scale and a bf16 bias per group of 64 weights).

Storage formats (all arrays are C-contiguous numpy arrays):
  x            uint16 [T, d]            bf16 bit patterns, x ~ N(0, 1)
  w_router     float32 [d, E]           W_r ~ N(0, 1/d)
  router_bias  float32 [E] or None      only for the skewed workload
  <m>_q        uint32 [n_mat, N, K/8]   eight 4-bit codes per word along K,
                                        lowest nibble = lowest k; codes ~ U{0..15}
  <m>_s        uint16 [n_mat, N, K/64]  bf16 scale ~ U(0.005, 0.015)
  <m>_b        uint16 [n_mat, N, K/64]  bf16 bias = -8*scale + U(-0.001, 0.001)
with <m> in gate, up (N = inter, K = d), down (N = d, K = inter) for the E
routed experts and sh_gate, sh_up, sh_down for the one shared expert.

Draw order for a one-layer workload, from numpy PCG64(seed):
  x, w_router, then gate, up, down of the routed experts (each: codes,
  scales, bias noise), then sh_gate, sh_up, sh_down, then (skewed workload
  only) the expert rank permutation.
The decode workload draws layer l from PCG64(SeedSequence([seed, l])) in the
same order without x, and the per-step inputs from
PCG64(SeedSequence([seed, n_layers])).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

GROUP = 64

MATS = ("gate", "up", "down", "sh_gate", "sh_up", "sh_down")


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    d: int
    inter: int
    n_experts: int
    top_k: int
    seed: int
    skew: bool = False
    n_layers: int = 1
    n_steps: int = 1
    note: str = ""


WORKLOADS = {
    "tiny": Workload("tiny", T=32, d=512, inter=128, n_experts=32, top_k=4, seed=0,
                     note="tiny MoE layer, checkable on the CPU in seconds"),
    "decode": Workload("decode", T=1, d=2048, inter=512, n_experts=256, top_k=8, seed=1,
                       n_layers=40, n_steps=256,
                       note="batch-1 decode, 40 distinct layers cycled, fresh x per step"),
    "prefill512": Workload("prefill512", T=512, d=2048, inter=512, n_experts=256, top_k=8,
                           seed=2, note="prefill chunk, near-uniform expert load"),
    "prefill2048": Workload("prefill2048", T=2048, d=2048, inter=512, n_experts=256, top_k=8,
                            seed=3, note="prefill chunk, ~64 rows per expert"),
    "skew4096": Workload("skew4096", T=4096, d=2048, inter=512, n_experts=256, top_k=8,
                         seed=4, skew=True,
                         note="prefill chunk, Zipf-like expert load from a per-expert router bias"),
}


def bf16_bits(a) -> np.ndarray:
    """Store float32 values as bf16 bit patterns (round to nearest even, via torch)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def bits_to_f32(b) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def q4_matrix(rng: np.random.Generator, n_mat: int, N: int, K: int):
    """Random group-64 affine 4-bit matrices: codes, bf16 scales, bf16 biases."""
    assert K % GROUP == 0
    q = rng.integers(0, 1 << 32, size=(n_mat, N, K // 8), dtype=np.uint32)
    scale = bf16_bits(rng.uniform(0.005, 0.015, size=(n_mat, N, K // GROUP)).astype(np.float32))
    noise = rng.uniform(-0.001, 0.001, size=(n_mat, N, K // GROUP)).astype(np.float32)
    bias = bf16_bits(np.float32(-8.0) * bits_to_f32(scale) + noise)
    return q, scale, bias


def _experts(rng, E, d, inter):
    out = {}
    for name, n_mat, N, K in (("gate", E, inter, d), ("up", E, inter, d), ("down", E, d, inter),
                              ("sh_gate", 1, inter, d), ("sh_up", 1, inter, d),
                              ("sh_down", 1, d, inter)):
        q, s, b = q4_matrix(rng, n_mat, N, K)
        out[name + "_q"], out[name + "_s"], out[name + "_b"] = q, s, b
    return out


def make_layer(w: Workload, layer: int = 0):
    """One layer's weights (dict of numpy arrays) and, for one-layer workloads, x.

    Returns (layer_dict, x) where x is uint16 [T, d] bf16 bits, or None for the
    decode workload (use `decode_inputs`)."""
    if w.n_layers == 1:
        assert layer == 0
        rng = np.random.Generator(np.random.PCG64(w.seed))
        x = bf16_bits(rng.standard_normal((w.T, w.d), dtype=np.float32))
    else:
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.seed, layer])))
        x = None
    L = {"d": w.d, "inter": w.inter, "n_experts": w.n_experts, "top_k": w.top_k}
    L["w_router"] = (rng.standard_normal((w.d, w.n_experts), dtype=np.float32)
                     * np.float32(1.0 / np.sqrt(w.d))).astype(np.float32)
    L.update(_experts(rng, w.n_experts, w.d, w.inter))
    L["router_bias"] = skew_bias(rng, w.n_experts) if w.skew else None
    return L, x


def skew_bias(rng: np.random.Generator, E: int) -> np.ndarray:
    """The skewed workload's router bias: b_e = 3 * ln(1 / rank_e^1.1) with rank a
    seeded permutation of 1..E (a fixed per-expert preference, Zipf-like load)."""
    rank = rng.permutation(E).astype(np.float64) + 1.0
    return (3.0 * np.log(1.0 / rank ** 1.1)).astype(np.float32)


def decode_inputs(w: Workload, n_steps: int | None = None):
    """Per-step decode inputs: uint16 [n_steps, d] bf16 bits, x ~ N(0, 1)."""
    n = w.n_steps if n_steps is None else n_steps
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.seed, w.n_layers])))
    return bf16_bits(rng.standard_normal((w.n_steps, w.d), dtype=np.float32))[:n].copy()


def random_layer(rng: np.random.Generator, d: int, inter: int, E: int, k: int,
                 router_bias: bool = False):
    """A random layer of any shape with the same value distributions (for edge cases)."""
    L = {"d": d, "inter": inter, "n_experts": E, "top_k": k}
    L["w_router"] = (rng.standard_normal((d, E), dtype=np.float32)
                     * np.float32(1.0 / np.sqrt(d))).astype(np.float32)
    L.update(_experts(rng, E, d, inter))
    L["router_bias"] = (rng.standard_normal(E).astype(np.float32) if router_bias else None)
    return L


def random_x(rng: np.random.Generator, T: int, d: int) -> np.ndarray:
    return bf16_bits(rng.standard_normal((T, d), dtype=np.float32))


# ---- the greedy token hand-off (section "Decode: minimize bytes per token":
# the chosen token stays on the device, from the largest output logit into the
# following step's input).  The pages give neither the vocabulary size nor
# the format of the output head and the embedding table; both are taken as
# V x d matrices in the experts' Q4 format, with the experts' value
# distributions.  Draw order from PCG64(seed): x, head, embedding table.

@dataclass(frozen=True)
class LmWorkload:
    name: str
    V: int
    d: int
    seed: int
    note: str = ""


LM_WORKLOADS = {
    "lm_tiny": LmWorkload("lm_tiny", V=3000, d=512, seed=20,
                          note="small head, checkable on the CPU in well under a second"),
    "lm_head": LmWorkload("lm_head", V=248320, d=2048, seed=21,
                          note="the layer's hidden size and a vocabulary of 248,320 rows"),
}


def random_lm(rng: np.random.Generator, V: int, d: int, with_embed: bool = True):
    """(x bf16 [d], head, embed) with head / embed dicts of q [V, d/8], scale, bias
    (embed None without with_embed; x and head are the same either way)."""
    x = bf16_bits(rng.standard_normal(d, dtype=np.float32))
    out = [None, None]
    for i in range(2 if with_embed else 1):
        q, s, b = q4_matrix(rng, 1, V, d)
        out[i] = {"q": q[0], "scale": s[0], "bias": b[0]}
    return x, out[0], out[1]


def make_lm(w: LmWorkload, with_embed: bool = True):
    return random_lm(np.random.Generator(np.random.PCG64(w.seed)), w.V, w.d, with_embed)
