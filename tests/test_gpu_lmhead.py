"""Parity of the greedy token hand-off (moe_lm_argmax, through the C ABI) with
the CPU oracle.

Bars:
  - logits: max |err| <= 1e-3 * RMS(oracle logits) (fp32 sums in another order
    than the oracle's fp64 ones);
  - token: bit-exact against the argmax of the kernel's own fp32 logits (the
    decision taken in the kernel's precision), and equal to the oracle's token
    wherever the oracle's two largest logits are further apart than twice the
    logit bound (else the oracle's logit at the kernel's token is within that
    bound of the maximum);
  - with given fp32 logits (MOE_LOGITS_IN): the token bit-exact against the oracle;
  - the next input: bit-exact against the oracle's dequantised embedding row.
"""
import numpy as np
import pytest
import torch

import oracle
import q4_routed_expert_amd as q4
from workloads import LM_WORKLOADS, make_lm, random_lm

pytestmark = pytest.mark.gpu

LOGIT_TOL = 1e-3


def log(msg):
    print(f"[lmhead] {msg}", flush=True)


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def xdev(x, dev):
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(dev).view(torch.bfloat16)


def host_bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def check_step(lm, head, embed, x_bits, logits, token, x_next):
    """Compare one GPU hand-off with the oracle; returns the GPU's token."""
    torch.cuda.synchronize()
    lg = logits.cpu().numpy()
    tok = int(token.cpu().numpy()[0])
    ref = oracle.lm_logits(x_bits, head["q"], head["scale"], head["bias"])
    rms = float(np.sqrt(np.mean(ref.astype(np.float64) ** 2)))
    bound = LOGIT_TOL * max(rms, 1e-30)
    err = float(np.abs(lg.astype(np.float64) - ref).max())
    assert err <= bound, (err, bound)
    # the decision in the kernel's precision: its own logits
    assert tok == oracle.argmax(lg)
    ref_tok = oracle.argmax(ref)
    top2 = np.sort(ref)[-2:] if ref.size > 1 else np.array([-np.inf, ref[0]])
    if top2[1] - top2[0] > 2 * bound:
        assert tok == ref_tok
    else:
        assert ref[tok] >= ref[ref_tok] - 2 * bound
    if x_next is not None:
        want = oracle.embed_row(embed["q"], embed["scale"], embed["bias"], tok)
        assert np.array_equal(host_bits(x_next), want)
    return tok


def run_case(dev, x, head, embed, alias=False):
    lm = q4.DeviceLmHead.from_host(head, embed, dev)
    ws = q4.lm_workspace(lm, dev)
    xd = xdev(x, dev)
    x_next = xd if alias else torch.empty_like(xd)
    logits, token, _ = q4.lm_argmax(lm, xd, ws, x_next=x_next)
    return check_step(lm, head, embed, x, logits, token, x_next)


@pytest.mark.parametrize("V,d,seed", [(1, 64, 0), (33, 192, 1), (2049, 2048, 2), (1000, 4160, 3),
                                      (65, 8192, 4), (31, 512, 5), (4097, 1024, 6),
                                      (q4._abi.MOE_MAX_VOCAB, 64, 7)])
def test_small_heads(dev, V, d, seed):
    log(f"V={V} d={d} seed={seed}")
    x, head, embed = random_lm(np.random.default_rng(seed), V, d)
    run_case(dev, x, head, embed)


def test_tiny_workload_with_aliased_next_input(dev):
    w = LM_WORKLOADS["lm_tiny"]
    log(f"{w.name} V={w.V} d={w.d}")
    x, head, embed = make_lm(w)
    run_case(dev, x, head, embed, alias=True)


def test_equal_logits_pick_the_lower_row(dev):
    # a copy of the winning row at a lower and at a higher index: identical rows
    # give identical logits on both sides, so the lowest copy must win
    V, d = 5000, 1024
    x, head, embed = random_lm(np.random.default_rng(11), V, d)
    j = oracle.argmax(oracle.lm_logits(x, head["q"], head["scale"], head["bias"]))
    for i in sorted({min(j + 37, V - 1), j // 3, V - 1}):
        if i == j:
            continue
        h = {k: v.copy() for k, v in head.items()}
        for k in h:
            h[k][i] = head[k][j]
        log(f"copy of row {j} at {i}")
        tok = run_case(dev, x, h, embed)
        assert tok == min(i, j)


def test_full_size_head(dev):
    w = LM_WORKLOADS["lm_head"]
    log(f"{w.name} V={w.V} d={w.d}: generating")
    x, head, embed = make_lm(w)
    log("running")
    tok = run_case(dev, x, head, embed)
    log(f"token {tok}")


def test_two_slot_chain_matches_the_oracle(dev):
    # three greedy steps, the token alternating between two slots of one array and
    # each step's input the previous step's embedding row, all on the device
    V, d = 3000, 512
    x0, head, embed = random_lm(np.random.default_rng(12), V, d)
    lm = q4.DeviceLmHead.from_host(head, embed, dev)
    ws = q4.lm_workspace(lm, dev)
    slots = torch.full((2,), -1, dtype=torch.int32, device=dev)
    xs = [xdev(x0, dev), torch.empty(d, dtype=torch.bfloat16, device=dev)]
    logits = torch.empty(V, dtype=torch.float32, device=dev)
    for step in range(3):
        q4.lm_argmax(lm, xs[step % 2], ws, logits=logits, token=slots[step % 2:step % 2 + 1],
                     x_next=xs[(step + 1) % 2])
    torch.cuda.synchronize()
    got = slots.cpu().numpy()
    x = x0
    toks = []
    for step in range(3):
        _, t, x = oracle.lm_step(head, embed, x)
        toks.append(t)
    log(f"oracle chain {toks}, slots {got.tolist()}")
    assert got[0] == toks[2] and got[1] == toks[1]
    assert np.array_equal(host_bits(xs[1]), x)


def _given(dev, lg):
    V = lg.size
    lm = q4.DeviceLmHead(V, 64, None, None)
    ws = q4.lm_workspace(lm, dev)
    logits = torch.from_numpy(np.ascontiguousarray(lg, np.float32)).to(dev)
    _, token, _ = q4.lm_argmax(lm, None, ws, logits=logits, logits_in=True)
    torch.cuda.synchronize()
    return int(token.cpu().numpy()[0])


def _given_cases():
    rng = np.random.default_rng(5)
    nan, inf = np.float32(np.nan), np.float32(np.inf)
    cases = []
    for V in (1, 2, 7, 2047, 2048, 2049, 248320):
        cases.append(("coarse", np.round(rng.standard_normal(V) * 3).astype(np.float32)))
    l = rng.standard_normal(5000).astype(np.float32)
    l[rng.random(5000) < 0.3] = nan
    cases.append(("nan", l))
    cases.append(("all-nan", np.full(3000, nan, np.float32)))
    cases.append(("all-neg-inf", np.full(4100, -inf, np.float32)))
    l = np.zeros(6000, np.float32)
    l[2047] = l[2048] = 1.0  # tie across two work groups' ranges
    cases.append(("boundary-tie", l))
    l = np.full(9000, -0.0, np.float32)
    l[::2] = 0.0  # signed zeros are equal
    cases.append(("signed-zero", l))
    l = rng.standard_normal(q4._abi.MOE_MAX_VOCAB).astype(np.float32)
    l[-1] = l[17] = 10.0
    cases.append(("max-vocab", l))
    l = rng.standard_normal(100).astype(np.float32)
    l[40] = inf
    cases.append(("inf", l))
    return cases


@pytest.mark.parametrize("name,lg", _given_cases(), ids=lambda v: v if isinstance(v, str) else "")
def test_given_logits_token_is_exact(dev, name, lg):
    log(f"given logits {name} V={lg.size}")
    assert _given(dev, lg) == oracle.argmax(lg)


def test_graph_replays_of_the_chain_match_eager(dev):
    # two hand-off steps captured once; each replay continues the chain from where
    # the previous one left it, and must match the same steps run eagerly
    V, d = 3000, 512
    x0, head, embed = random_lm(np.random.default_rng(13), V, d)
    lm = q4.DeviceLmHead.from_host(head, embed, dev)
    ws = q4.lm_workspace(lm, dev)
    logits = torch.empty(V, dtype=torch.float32, device=dev)

    def chain(xs, slots, n, stream=None):
        for step in range(n):
            q4.lm_argmax(lm, xs[step % 2], ws, logits=logits,
                         token=slots[step % 2:step % 2 + 1], x_next=xs[(step + 1) % 2],
                         stream=stream)

    xs_e = [xdev(x0, dev), torch.empty(d, dtype=torch.bfloat16, device=dev)]
    slots_e = torch.full((2,), -1, dtype=torch.int32, device=dev)
    want = []
    for rep in range(4):
        chain(xs_e, slots_e, 2)
        torch.cuda.synchronize()
        want.append((slots_e.cpu().numpy().copy(), host_bits(xs_e[0]).copy()))
    xs = [xdev(x0, dev), torch.empty(d, dtype=torch.bfloat16, device=dev)]
    slots = torch.full((2,), -1, dtype=torch.int32, device=dev)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        chain([xs[0].clone(), xs[1].clone()], slots.clone(), 2)  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        chain(xs, slots, 2)
    xs[0].copy_(xdev(x0, dev))
    slots.fill_(-1)
    torch.cuda.synchronize()
    for rep in range(4):
        g.replay()
        torch.cuda.synchronize()
        _ = torch.zeros(16, device=dev).sum()  # eager work between replays
        log(f"replay {rep}: slots {slots.cpu().numpy().tolist()} want {want[rep][0].tolist()}")
        assert np.array_equal(slots.cpu().numpy(), want[rep][0])
        assert np.array_equal(host_bits(xs[0]), want[rep][1])
