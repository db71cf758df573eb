#!/usr/bin/env python3
"""Benchmark of the routed-MoE Q4 FFN layer on one MI355X.

One step = one prefill layer call on the T=2048 chunk (moe_route + moe_prefill:
router logits, top-8, histogram/scan/scatter/block maps, gate/up grouped GEMM
with SiLU*up, routed down GEMM, shared down GEMM with the fixed-order combine
in its epilogue), inputs
resident in HBM, two distinct weight sets alternated so the weights stream
from HBM; only two events bracket the timed steps, and the per-kernel split
comes from separate steps with an event after every kernel.  The same steps
are also captured in a HIP graph (two layer calls, one per weight set) and
replayed as a cross-check (`graph`: time and bit-equality with the eager
output).  After the timed prefill steps the batch-1 decode layer is measured
on 40 distinct layers cycled for `--decode-steps` steps (one moe_decode call
per layer, every call on one stream), and the CPU oracle is timed on a bounded
sample of the prefill workload.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import ctypes as C
import dataclasses
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 matrix-core peak (published)
PEAK_HBM_GBPS = 8000.0     # MI355X HBM3E peak (published)
METRIC = "prefill MoE-layer tok/s @T=2048 (%MFMA peak); decode GB/s per layer (%HBM peak)"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def q4_bytes(N, K):
    """Bytes of one N x K group-64 affine 4-bit matrix: codes + bf16 scale + bf16 bias."""
    return N * K // 2 + N * (K // 64) * 4


class HipEvents:
    """HIP events through the process's (torch's) HIP runtime."""

    def __init__(self):
        with open("/proc/self/maps") as f:
            path = sorted({ln.split()[-1] for ln in f if "libamdhip64" in ln})[0]
        self.rt = C.CDLL(path)
        self.rt.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
        self.rt.hipEventRecord.argtypes = [C.c_void_p, C.c_void_p]
        self.rt.hipEventSynchronize.argtypes = [C.c_void_p]
        self.rt.hipEventDestroy.argtypes = [C.c_void_p]
        self.pool = []

    def make(self, n):
        arr = (C.c_void_p * n)()
        for i in range(n):
            if self.rt.hipEventCreate(C.byref(arr, i * C.sizeof(C.c_void_p))) != 0:
                raise RuntimeError("hipEventCreate failed")
        self.pool.append(arr)
        return arr

    def record(self, ev, stream):
        self.rt.hipEventRecord(ev, stream)

    def ms(self, a, b):
        out = C.c_float()
        if self.rt.hipEventElapsedTime(C.byref(out), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(out.value)

    def close(self):
        for arr in self.pool:
            for e in arr:
                self.rt.hipEventDestroy(e)
        self.pool = []


def prefill_work(T, d, I, E, k, counts):
    """Algorithmic flops and bytes of one prefill layer call, per kernel and total."""
    touched = int((counts > 0).sum())
    gu_w = (touched + 1) * 2 * q4_bytes(I, d)
    dn_w = (touched + 1) * q4_bytes(d, I)
    f_gu = 4 * T * k * d * I + 4 * T * d * I
    f_dn_routed = 2 * T * k * I * d
    f_dn_shared = 2 * T * I * d
    x_b, y_b, h_b, hs_b = 2 * T * d, 2 * T * d, 2 * T * k * I, 2 * T * I
    return {
        "touched_experts": touched,
        "flops": f_gu + f_dn_routed + f_dn_shared,
        "bytes": gu_w + dn_w + 4 * d * E + x_b + y_b,
        "gate_up": {"flops": f_gu, "bytes": gu_w + x_b + h_b + hs_b},
        # routed rows -> fp16 staging rows (+ one exponent byte per 32 columns)
        "down": {"flops": f_dn_routed,
                 "bytes": touched * q4_bytes(d, I) + h_b + 2 * T * k * d + T * k * d // 32},
        # shared expert's down GEMM, the staged rows read back, scores, y
        "shared_down_combine": {"flops": f_dn_shared + 2 * T * k * d + T * d,
                                "bytes": q4_bytes(d, I) + hs_b + 2 * T * k * d + T * k * d // 32
                                + 4 * T * k + y_b},
    }


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_moe_layer_T2048_decode.md")
KERNEL_SOURCES = ("q4_routed_expert_amd/csrc/prefill.hip", "q4_routed_expert_amd/csrc/decode.hip",
                  "q4_routed_expert_amd/csrc/q4moe_dev.h", "q4_routed_expert_amd/csrc/internal.h")
LM_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_lm_head_V248320.md")
LM_SOURCES = ("q4_routed_expert_amd/csrc/lmhead.hip", "q4_routed_expert_amd/csrc/lmhead.h",
              "q4_routed_expert_amd/csrc/q4moe_dev.h", "q4_routed_expert_amd/csrc/internal.h")


def kernel_source_hash(sources=KERNEL_SOURCES):
    import hashlib
    h = hashlib.sha256()
    for rel in sources:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(key, path=None, sources=KERNEL_SOURCES):
    """HBM bytes per launch from a committed rocprofv3 FETCH_SIZE/WRITE_SIZE summary, or None
    when the summary is missing or the kernel sources have changed since it was taken."""
    try:
        with open(path or TRAFFIC_FILE) as f:
            for line in f:
                if line.startswith("traffic-json: "):
                    rec = json.loads(line[len("traffic-json: "):])
                    if rec.get("source_hash") == kernel_source_hash(sources) and key in rec:
                        return rec[key]
    except OSError:
        pass
    return None


def copy_calibration(torch):
    """A plain copy of known size for calibrating the HBM byte counters: reads and writes
    256 MiB once per call (an elementwise negation, one kernel)."""
    n = 64 * 1024 * 1024
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    log(f"copy calibration: 3 x elementwise negation of {4 * n} bytes")
    del src, dst


def roofline(flops, nbytes, seconds):
    t_mfma = flops / (PEAK_BF16_TFLOPS * 1e12)
    t_hbm = nbytes / (PEAK_HBM_GBPS * 1e9)
    if t_mfma >= t_hbm:
        a = flops / seconds / 1e12
        return {"bound": "mfma", "achieved": round(a, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(a / PEAK_BF16_TFLOPS, 4), "traffic": None}
    a = nbytes / seconds / 1e9
    return {"bound": "hbm", "achieved": round(a, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "frac": round(a / PEAK_HBM_GBPS, 4), "traffic": None}


GRAPH_LAYERS = 8  # prefill layer steps per HIP-graph replay


def bench_prefill(args, q4, torch, ev, stream):
    from workloads import WORKLOADS, make_layer
    w = WORKLOADS["prefill2048"]
    log(f"generating two weight sets for {w.name} (T={w.T}, d={w.d}, I={w.inter}, E={w.n_experts}, k={w.top_k})")
    L0, x = make_layer(w)
    L1, _ = make_layer(dataclasses.replace(w, seed=w.seed + 100))
    dev = torch.device("cuda:0")
    layers = [q4.DeviceLayer.from_host(L, dev) for L in (L0, L1)]
    del L0, L1
    xd = torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
    r = q4.DeviceRouting(w.T, w.n_experts, w.top_k, dev)
    ws = q4.workspace(layers[0], w.T, dev)
    y = torch.empty((w.T, w.d), dtype=torch.bfloat16, device=dev)
    lib = q4._abi.lib()

    def step(i, trace_route=None, trace_pre=None):
        if trace_route is not None:
            lib.moe_trace_events(C.cast(trace_route, C.c_void_p), 4)
        q4.route(layers[i % 2], xd, routing=r)
        if trace_pre is not None:
            lib.moe_trace_events(C.cast(trace_pre, C.c_void_p), 4)
        q4.prefill(layers[i % 2], xd, r, ws, y)
        lib.moe_trace_events(None, 0)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # clocks under load: sysfs read a few times while a queue of untimed steps runs
    pci = gpu_pci(torch)
    n_load = max(64, int(0.15e6 / 250))
    for i in range(n_load):
        step(i)
    under_load = []
    for _ in range(4):
        time.sleep(0.02)
        under_load.append(gpu_clocks(pci))
    torch.cuda.synchronize()
    # timed steps: only two events around the whole loop
    K = args.steps
    t = ev.make(2)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ev.record(t[0], stream)
    for i in range(K):
        step(args.warmup + i)
    ev.record(t[1], stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = ev.ms(t[0], t[1]) / K
    # per-kernel split from separate steps with an event after every kernel
    # (each event adds a little to the kernel it follows)
    Kt = min(K, 20)
    ev_r = [ev.make(4) for _ in range(Kt)]
    ev_p = [ev.make(4) for _ in range(Kt)]
    for i in range(Kt):
        step(args.warmup + K + i, ev_r[i], ev_p[i])
    torch.cuda.synchronize()
    names_r = ["router_logits", "topk_histogram", "route_scatter"]
    names_p = ["gate_up", "down", "shared_down_combine"]
    per = {n: 0.0 for n in names_r + names_p}
    for i in range(Kt):
        for j, n in enumerate(names_r):
            per[n] += ev.ms(ev_r[i][j], ev_r[i][j + 1]) / Kt
        for j, n in enumerate(names_p):
            per[n] += ev.ms(ev_p[i][j], ev_p[i][j + 1]) / Kt
    counts = r.counts.cpu().numpy()
    work = prefill_work(w.T, w.d, w.inter, w.n_experts, w.top_k, counts)
    sec = ms_step / 1e3
    tflops = work["flops"] / sec / 1e12
    log(f"prefill: {ms_step * 1e3:.1f} us/layer ({wall / K * 1e6:.1f} us wall), "
        f"{tflops:.1f} TFLOP/s, per kernel (us): " +
        ", ".join(f"{n}={v * 1e3:.1f}" for n, v in per.items()))
    out = {
        "workload": w, "ms_per_step": ms_step, "wall_ms_per_step": wall / K * 1e3,
        "tok_s": w.T / sec, "tflops": tflops, "mfma_frac": tflops / PEAK_BF16_TFLOPS,
        "gbps": work["bytes"] / sec / 1e9, "work": work, "kernel_us": {n: v * 1e3 for n, v in per.items()},
        "clocks_under_load": under_load,
    }
    # GRAPH_LAYERS layer steps (route + prefill, alternating the weight sets)
    # captured once in a HIP graph and replayed; the output must equal the
    # eager output.  The first rounds of replays after a process's first
    # capture run slower (about 10 % here, once), so the timed replays follow
    # untimed ones.
    if not args.no_graph:
        for i in range(GRAPH_LAYERS):
            step(i)
        torch.cuda.synchronize()
        y_eager = y.clone()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(GRAPH_LAYERS):
                step(i)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        same = bool(torch.equal(y, y_eager))
        reps = max(1, K // GRAPH_LAYERS)
        for _ in range(2 * reps):
            g.replay()
        torch.cuda.synchronize()
        t2 = ev.make(2)
        gs = int(torch.cuda.current_stream().cuda_stream)
        ev.record(t2[0], gs)
        for _ in range(reps):
            g.replay()
        ev.record(t2[1], gs)
        torch.cuda.synchronize()
        us_g = ev.ms(t2[0], t2[1]) * 1e3 / (GRAPH_LAYERS * reps)
        out["graph"] = {"us_per_layer": us_g, "tok_s": w.T / (us_g * 1e-6),
                        "mfma_frac": work["flops"] / (us_g * 1e-6) / 1e12 / PEAK_BF16_TFLOPS,
                        "replays": reps, "layers_per_replay": GRAPH_LAYERS, "matches_eager": same}
        log(f"prefill graph: {us_g:.1f} us/layer, output equal to eager: {same}")
        del g
    gu_sec = per["gate_up"] / 1e3
    out["roofline"] = roofline(work["gate_up"]["flops"], work["gate_up"]["bytes"], gu_sec)
    out["roofline"]["kernel"] = "gate_up_kernel (grouped gate/up GEMM + SiLU*up)"
    out["roofline"]["traffic"] = measured_traffic("gate_up_bytes")
    out["roofline"]["mfma_frac"] = round(work["gate_up"]["flops"] / gu_sec / 1e12 / PEAK_BF16_TFLOPS, 4)
    del layers, ws
    torch.cuda.empty_cache()
    return out


def bench_config(name, args, q4, torch, ev, stream):
    """route + prefill on one of the other prefill workloads (its own seed and, for
    the skewed one, its router bias), two weight sets alternated (the second drawn
    with seed + 100), timed like the headline."""
    from workloads import WORKLOADS, make_layer
    w = WORKLOADS[name]
    log(f"config {name}: generating two weight sets (T={w.T}, d={w.d}, I={w.inter}, "
        f"E={w.n_experts}, k={w.top_k}, seed {w.seed})")
    L0, x = make_layer(w)
    L1, _ = make_layer(dataclasses.replace(w, seed=w.seed + 100))
    if w.skew:  # the same per-expert preference on both sets
        L1["router_bias"] = L0["router_bias"]
    dev = torch.device("cuda:0")
    layers = [q4.DeviceLayer.from_host(L, dev) for L in (L0, L1)]
    del L0, L1
    xd = torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
    r = q4.DeviceRouting(w.T, w.n_experts, w.top_k, dev)
    ws = q4.workspace(layers[0], w.T, dev)
    y = torch.empty((w.T, w.d), dtype=torch.bfloat16, device=dev)

    def step(i):
        q4.route(layers[i % 2], xd, routing=r)
        q4.prefill(layers[i % 2], xd, r, ws, y)

    for i in range(max(20, args.warmup // 4)):
        step(i)
    torch.cuda.synchronize()
    n = max(10, args.steps)
    t = ev.make(2)
    ev.record(t[0], stream)
    for i in range(n):
        step(i)
    ev.record(t[1], stream)
    torch.cuda.synchronize()
    us = ev.ms(t[0], t[1]) * 1e3 / n
    work = prefill_work(w.T, w.d, w.inter, w.n_experts, w.top_k, r.counts.cpu().numpy())
    sec = us * 1e-6
    rec = {"T": w.T, "d": w.d, "inter": w.inter, "n_experts": w.n_experts, "top_k": w.top_k,
           "seed": w.seed, "skewed_router": w.skew, "steps": n, "us_per_layer": round(us, 2),
           "tok_s": round(w.T / sec, 1), "tflops": round(work["flops"] / sec / 1e12, 2),
           "mfma_frac": round(work["flops"] / sec / 1e12 / PEAK_BF16_TFLOPS, 4),
           "gbps": round(work["bytes"] / sec / 1e9, 1),
           "hbm_frac": round(work["bytes"] / sec / 1e9 / PEAK_HBM_GBPS, 4),
           "touched_experts": work["touched_experts"],
           "algorithmic": {"flops": work["flops"], "bytes": work["bytes"]}}
    log(f"config {name}: {us:.1f} us/layer, {rec['tok_s']:.0f} tok/s, MFMA {rec['mfma_frac']:.3f}, "
        f"HBM {rec['hbm_frac']:.3f}, {rec['touched_experts']} experts touched")
    del layers, ws, r, y
    torch.cuda.empty_cache()
    return rec


def host_info():
    """The host CPU model and thread counts (for the oracle's timing), from /proc
    (no child process: the bench must not start programs once the GPU is in use)."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = None
    return {"cpu_model": model, "logical_cpus": os.cpu_count(), "usable_cpus": usable}


def gpu_clocks(pci=None):
    """The current shader and memory clock levels (the line marked '*' of
    pp_dpm_sclk / pp_dpm_mclk in sysfs) of the GPU at PCI address prefix `pci`
    ("dddd:bb:dd."), or of every GPU the kernel driver lists when it is None."""
    import glob
    cards = {}
    for dev in sorted(glob.glob("/sys/class/drm/card*/device")):
        addr = os.path.basename(os.path.realpath(dev))
        if pci is not None and not addr.startswith(pci):
            continue
        rec = {}
        for name in ("pp_dpm_sclk", "pp_dpm_mclk"):
            try:
                with open(os.path.join(dev, name)) as f:
                    cur = [ln.split(":", 1)[1].strip(" *\n") for ln in f if ln.rstrip().endswith("*")]
                rec[name[7:]] = cur[0] if cur else None
            except OSError:
                pass
        if rec:
            cards[addr] = rec
    return cards or {"error": "no pp_dpm_sclk in sysfs"}


def gpu_pci(torch):
    """PCI address prefix of cuda:0 as sysfs names it."""
    p = torch.cuda.get_device_properties(0)
    return f"{p.pci_domain_id:04x}:{p.pci_bus_id:02x}:{p.pci_device_id:02x}."


def bench_decode(args, q4, torch, ev, stream):
    from workloads import WORKLOADS, decode_inputs, make_layer
    w = WORKLOADS["decode"]
    n_layers, n_steps = args.decode_layers, args.decode_steps
    dev = torch.device("cuda:0")
    log(f"generating {n_layers} decode layers (d={w.d}, I={w.inter}, E={w.n_experts}, k={w.top_k})")
    layers = []
    for li in range(n_layers):
        L, _ = make_layer(w, li)
        layers.append(q4.DeviceLayer.from_host(L, dev))
        del L
    xs = torch.from_numpy(decode_inputs(w, n_steps).view(np.int16)).to(dev).view(torch.bfloat16)
    ws = q4.workspace(layers[0], 1, dev)
    y = torch.empty((1, w.d), dtype=torch.bfloat16, device=dev)
    lib = q4._abi.lib()
    for st in range(max(1, args.decode_warmup)):  # warm-up passes over all layers
        for li in range(n_layers):
            q4.decode(layers[li], xs[st % n_steps:st % n_steps + 1], ws, y)
    torch.cuda.synchronize()
    mid = n_steps // 2
    ev_d = [ev.make(4) for _ in range(n_layers)]
    # The timed loop calls the C entry point with prebuilt arguments: the
    # binding's per-call tensor checks (used above) would otherwise pace the
    # GPU, a layer call taking about as long on the host as on the device.
    dec = lib.moe_decode
    l_ptr = [C.addressof(L.struct) for L in layers]
    x0, row_b = xs.data_ptr(), 2 * w.d
    ws_p, ws_n, y_p = ws.data_ptr(), ws.numel(), y.data_ptr()
    t = ev.make(2)
    ev.record(t[0], stream)
    for st in range(n_steps):
        xp = x0 + st * row_b
        for li in range(n_layers):
            if st == mid:
                lib.moe_trace_events(C.cast(ev_d[li], C.c_void_p), 4)
            if dec(l_ptr[li], xp, 0, None, ws_p, ws_n, y_p, stream):
                raise RuntimeError(lib.moe_last_error().decode())
            if st == mid:
                lib.moe_trace_events(None, 0)
    ev.record(t[1], stream)
    torch.cuda.synchronize()
    calls = n_steps * n_layers
    us_layer = ev.ms(t[0], t[1]) * 1e3 / calls
    names = ["router_shared_gate_up", "topk_gate_up", "down_combine"]
    per = {n: sum(ev.ms(ev_d[li][j], ev_d[li][j + 1]) for li in range(n_layers)) * 1e3 / n_layers
           for j, n in enumerate(names)}
    expert_bytes = (w.top_k + 1) * (2 * q4_bytes(w.inter, w.d) + q4_bytes(w.d, w.inter))
    router_bytes = 4 * w.d * w.n_experts
    gbps = expert_bytes / (us_layer * 1e-6) / 1e9
    log(f"decode eager: {us_layer:.2f} us/layer, {gbps:.0f} GB/s on the 9 experts' bytes, "
        f"per kernel (us): " + ", ".join(f"{n}={v:.2f}" for n, v in per.items()))
    out = {"us_per_layer": us_layer, "gbps": gbps, "hbm_frac": gbps / PEAK_HBM_GBPS,
           "gbps_incl_router": (expert_bytes + router_bytes) / (us_layer * 1e-6) / 1e9,
           "expert_bytes_per_layer": expert_bytes, "kernel_us": per,
           "layers": n_layers, "steps": n_steps, "calls": calls}
    # the same 40-layer step captured once in a HIP graph and replayed
    if not args.no_graph:
        y_eager = y.clone()
        g = torch.cuda.CUDAGraph()
        gx = xs[n_steps - 1:n_steps].clone()
        with torch.cuda.graph(g):
            for li in range(n_layers):
                q4.decode(layers[li], gx, ws, y)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        same = bool(torch.equal(y, y_eager))
        reps = max(1, n_steps // 4)
        t2 = ev.make(2)
        gs = torch.cuda.current_stream()
        ev.record(t2[0], int(gs.cuda_stream))
        for _ in range(reps):
            g.replay()
        ev.record(t2[1], int(gs.cuda_stream))
        torch.cuda.synchronize()
        us_g = ev.ms(t2[0], t2[1]) * 1e3 / (reps * n_layers)
        out["graph"] = {"us_per_layer": us_g, "gbps": expert_bytes / (us_g * 1e-6) / 1e9,
                        "hbm_frac": expert_bytes / (us_g * 1e-6) / 1e9 / PEAK_HBM_GBPS,
                        "replays": reps, "matches_eager": same}
        log(f"decode graph: {us_g:.2f} us/layer ({out['graph']['gbps']:.0f} GB/s), "
            f"output equal to eager: {same}")
        del g
    # the few-token decode shape: moe_decode_tokens on T tokens per call
    out["tokens"] = []
    for T in (2, 4, 8):
        if args.decode_steps < 4 or args.no_decode_tokens:
            break
        xt = torch.from_numpy(decode_inputs(w, 8 * 32).view(np.int16)).to(dev).view(torch.bfloat16)
        n_st = max(2, n_steps // 4)
        yT = torch.empty((T, w.d), dtype=torch.bfloat16, device=dev)
        for li in range(n_layers):
            q4.decode_tokens(layers[li], xt[0:T], ws, yT)
        torch.cuda.synchronize()
        tT = ev.make(2)
        dect, xt0, yT_p = lib.moe_decode_tokens, xt.data_ptr(), yT.data_ptr()
        ev.record(tT[0], stream)
        for st in range(n_st):
            xp = xt0 + ((st * T) % (xt.shape[0] - T + 1)) * row_b
            for li in range(n_layers):
                if dect(l_ptr[li], xp, T, 0, None, ws_p, ws_n, yT_p, stream):
                    raise RuntimeError(lib.moe_last_error().decode())
        ev.record(tT[1], stream)
        torch.cuda.synchronize()
        usT = ev.ms(tT[0], tT[1]) * 1e3 / (n_st * n_layers)
        # per-kernel split over one more pass of the layers
        evT = [ev.make(4) for _ in range(n_layers)]
        for li in range(n_layers):
            lib.moe_trace_events(C.cast(evT[li], C.c_void_p), 4)
            q4.decode_tokens(layers[li], xt[0:T], ws, yT)
            lib.moe_trace_events(None, 0)
        torch.cuda.synchronize()
        perT = [sum(ev.ms(evT[li][j], evT[li][j + 1]) for li in range(n_layers)) * 1e3 / n_layers
                for j in range(3)]
        # distinct experts the T tokens select, over one pass of the layers
        rT = q4.DeviceRouting(T, w.n_experts, w.top_k, dev)
        uni = []
        for li in range(n_layers):
            q4.decode_tokens(layers[li], xt[0:T], ws, yT, routing=rT)
            uni.append(len(np.unique(rT.topk_idx.cpu().numpy())))
        n_uni = float(np.mean(uni))
        per_expert = expert_bytes // (w.top_k + 1)
        bytesT = (n_uni + 1) * per_expert
        rec = {"T": T, "us_per_layer": round(usT, 3), "us_per_token": round(usT / T, 3),
               "distinct_experts": round(n_uni, 2), "expert_bytes_per_layer": int(bytesT),
               "gbps": round(bytesT / (usT * 1e-6) / 1e9, 1),
               "hbm_frac": round(bytesT / (usT * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4),
               "bytes_per_token": int(bytesT / T),
               "kernel_us": {n: round(v, 3) for n, v in zip(names, perT)}}
        out["tokens"].append(rec)
        log(f"decode T={T}: {usT:.2f} us/layer ({usT / T:.2f} us/token), {n_uni:.1f} distinct "
            f"experts, {rec['gbps']:.0f} GB/s on their bytes, per kernel (us): " +
            ", ".join(f"{n}={v:.2f}" for n, v in zip(names, perT)))
        del rT
    # priced on the measured layer time (the three kernels back to back, launch
    # gaps included), the same time as us_per_layer
    out["roofline"] = {"bound": "hbm", "achieved": round(gbps, 1),
                       "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                       "frac": round(gbps / PEAK_HBM_GBPS, 4),
                       "traffic": measured_traffic("decode_bytes_per_layer"),
                       "kernels": "decode router partials + shared gate/up, top-k + routed gate/up, "
                                  "down/combine (one layer call)"}
    del layers, ws
    torch.cuda.empty_cache()
    return out


def bench_handoff(args, q4, torch, ev, stream):
    """Greedy token hand-off (moe_lm_argmax) at V = 248,320, d = 2048: a chain of
    steps, each reading the previous step's embedding row as its input and
    writing its token into one of two slots, with no host synchronisation."""
    from workloads import LM_WORKLOADS, make_lm
    w = LM_WORKLOADS["lm_head"]
    log(f"hand-off: generating the output head and embedding table (V={w.V}, d={w.d})")
    x, head, embed = make_lm(w)
    dev = torch.device("cuda:0")
    lm = q4.DeviceLmHead.from_host(head, embed, dev)
    del head, embed
    ws = q4.lm_workspace(lm, dev)
    xs = [torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16),
          torch.empty(w.d, dtype=torch.bfloat16, device=dev)]
    logits = torch.empty(w.V, dtype=torch.float32, device=dev)
    slots = torch.zeros(2, dtype=torch.int32, device=dev)
    lib = q4._abi.lib()

    def step(i):
        q4.lm_argmax(lm, xs[i % 2], ws, logits=logits, token=slots[i % 2:i % 2 + 1],
                     x_next=xs[(i + 1) % 2])

    for i in range(20):
        step(i)
    torch.cuda.synchronize()
    n = max(20, args.steps * 4)
    t = ev.make(2)
    ev.record(t[0], stream)
    for i in range(n):
        step(i)
    ev.record(t[1], stream)
    torch.cuda.synchronize()
    us = ev.ms(t[0], t[1]) * 1e3 / n
    n_tr = 20
    evs = [ev.make(3) for _ in range(n_tr)]
    for i in range(n_tr):
        lib.moe_trace_events(C.cast(evs[i], C.c_void_p), 3)
        step(i)
        lib.moe_trace_events(None, 0)
    torch.cuda.synchronize()
    per = {nm: sum(ev.ms(evs[i][j], evs[i][j + 1]) for i in range(n_tr)) * 1e3 / n_tr
           for j, nm in enumerate(("lm_head", "pick_embed"))}
    # the same chain captured in a HIP graph (8 steps) and replayed
    graph = None
    if not getattr(args, "no_graph", False):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(8):
                step(i)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        reps = max(5, n // 8)
        tg = ev.make(2)
        gs = int(torch.cuda.current_stream().cuda_stream)
        ev.record(tg[0], gs)
        for _ in range(reps):
            g.replay()
        ev.record(tg[1], gs)
        torch.cuda.synchronize()
        graph = {"us_per_step": round(ev.ms(tg[0], tg[1]) * 1e3 / (8 * reps), 3),
                 "steps": 8 * reps}
        log(f"hand-off graph: {graph['us_per_step']:.2f} us/step")
        del g
    n_part = -(-w.V // 16)
    # algorithmic bytes of the head kernel: every code, scale and bias once, x,
    # the logits and the partial results written
    head_bytes = q4_bytes(w.V, w.d) + 2 * w.d + 4 * w.V + 8 * n_part
    gbps = head_bytes / (per["lm_head"] * 1e-6) / 1e9
    log(f"hand-off: {us:.2f} us/step, per kernel (us): " +
        ", ".join(f"{k}={v:.2f}" for k, v in per.items()) + f"; head {gbps:.0f} GB/s")
    out = {"V": w.V, "d": w.d, "us_per_step": round(us, 3), "steps": n,
           "kernel_us": {k: round(v, 3) for k, v in per.items()},
           "head_bytes": head_bytes, "graph": graph,
           "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS,
                        "unit": "GB/s", "frac": round(gbps / PEAK_HBM_GBPS, 4),
                        "traffic": measured_traffic("lm_head_bytes", LM_TRAFFIC_FILE, LM_SOURCES),
                        "kernel": "lm_head_kernel (Q4 output-head GEMV + partial argmax)"}}
    del lm, ws, xs, logits
    torch.cuda.empty_cache()
    return out


def bench_sweep(args, q4, torch, ev, stream):
    """Prefill layer time over chunk sizes T (balanced and skewed router), the
    small-T verify shapes (T = 1..8 through the same prefill path) included.
    Weights: two sets alternated, as in the headline; x: the first T rows of one
    seeded draw; the skewed rows add the skewed workload's router bias."""
    from workloads import WORKLOADS, make_layer, skew_bias
    Ts = [int(t) for t in args.sweep.split(",")]
    base = WORKLOADS["prefill2048"]
    w = dataclasses.replace(base, T=max(Ts))
    log(f"sweep: generating two weight sets and x for T up to {w.T}")
    L0, x = make_layer(w)
    L1, _ = make_layer(dataclasses.replace(w, seed=w.seed + 100))
    bias = skew_bias(np.random.Generator(np.random.PCG64(w.seed + 200)), w.n_experts)
    dev = torch.device("cuda:0")
    sets = {False: [q4.DeviceLayer.from_host(L, dev) for L in (L0, L1)],
            True: [q4.DeviceLayer.from_host(dict(L, router_bias=bias), dev) for L in (L0, L1)]}
    del L0, L1
    xd = torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
    ws = q4.workspace(sets[False][0], w.T, dev)
    rows = []
    for skew in (False, True):
        for T in Ts:
            if skew and T < 256:
                continue
            r = q4.DeviceRouting(T, w.n_experts, w.top_k, dev)
            y = torch.empty((T, w.d), dtype=torch.bfloat16, device=dev)
            xs = xd[:T]

            def step(i):
                q4.route(sets[skew][i % 2], xs, routing=r)
                q4.prefill(sets[skew][i % 2], xs, r, ws, y)

            for i in range(3):
                step(i)
            torch.cuda.synchronize()
            n = max(4, min(args.steps, 20))
            t = ev.make(2)
            ev.record(t[0], stream)
            for i in range(n):
                step(i)
            ev.record(t[1], stream)
            torch.cuda.synchronize()
            us = ev.ms(t[0], t[1]) * 1e3 / n
            counts = r.counts.cpu().numpy()
            work = prefill_work(T, w.d, w.inter, w.n_experts, w.top_k, counts)
            sec = us * 1e-6
            row = {"T": T, "skew": skew, "us_per_layer": round(us, 2), "tok_s": round(T / sec, 1),
                   "tflops": round(work["flops"] / sec / 1e12, 2),
                   "mfma_frac": round(work["flops"] / sec / 1e12 / PEAK_BF16_TFLOPS, 4),
                   "gbps": round(work["bytes"] / sec / 1e9, 1),
                   "hbm_frac": round(work["bytes"] / sec / 1e9 / PEAK_HBM_GBPS, 4),
                   "touched_experts": work["touched_experts"],
                   "weight_bytes_per_token": round((work["bytes"] - 4 * T * w.d) / T, 1)}
            rows.append(row)
            log(f"sweep T={T} skew={skew}: {us:.1f} us/layer, {row['tok_s']:.0f} tok/s, "
                f"MFMA {row['mfma_frac']:.3f}, HBM {row['hbm_frac']:.3f}, "
                f"{row['touched_experts']} experts touched")
            del r, y
    del sets, ws
    torch.cuda.empty_cache()
    return rows


def bench_item_rows(args, q4, torch, ev, stream):
    """Gate/up work-item height ablation: route + prefill at item heights 128, 64,
    32 and 16 rows (the rows that share one dequantised weight tile; 16-row items
    fill half of one 32-row MFMA subtile), T = 512, 2048,
    4096, with the balanced router and with the skewed workload's router bias.
    Weights: the T=2048 workload's two sets, alternated; x: the first T rows of one
    seeded draw of 4096 rows; the skewed rows add the skewed workload's bias."""
    from workloads import WORKLOADS, make_layer, skew_bias
    base = WORKLOADS["prefill2048"]
    Ts = (512, 2048, 4096)
    w = dataclasses.replace(base, T=max(Ts))
    log(f"item-height ablation: generating two weight sets and x for T up to {w.T}")
    L0, x = make_layer(w)
    L1, _ = make_layer(dataclasses.replace(w, seed=w.seed + 100))
    bias = skew_bias(np.random.Generator(np.random.PCG64(WORKLOADS["skew4096"].seed)), w.n_experts)
    dev = torch.device("cuda:0")
    sets = {False: [q4.DeviceLayer.from_host(L, dev) for L in (L0, L1)],
            True: [q4.DeviceLayer.from_host(dict(L, router_bias=bias), dev) for L in (L0, L1)]}
    del L0, L1
    xd = torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
    ws = q4.workspace(sets[False][0], w.T, dev)
    lib = q4._abi.lib()
    rows = []
    for skew in (False, True):
        for T in Ts:
            r = q4.DeviceRouting(T, w.n_experts, w.top_k, dev)
            y = torch.empty((T, w.d), dtype=torch.bfloat16, device=dev)
            xs = xd[:T]
            rec = {"T": T, "skew": skew}
            # two passes in opposite orders, the faster kept (clock ramps and
            # order effects cancel)
            for m in (128, 64, 32, 16, 16, 32, 64, 128):
                def step(i, tr=None):
                    q4.route(sets[skew][i % 2], xs, routing=r)
                    if tr is not None:
                        lib.moe_trace_events(C.cast(tr, C.c_void_p), 4)
                    q4.prefill(sets[skew][i % 2], xs, r, ws, y, item_rows=m)
                    lib.moe_trace_events(None, 0)

                for i in range(4):
                    step(i)
                torch.cuda.synchronize()
                n = max(10, min(args.steps, 30))
                t = ev.make(2)
                ev.record(t[0], stream)
                for i in range(n):
                    step(i)
                ev.record(t[1], stream)
                torch.cuda.synchronize()
                us = ev.ms(t[0], t[1]) * 1e3 / n
                trs = [ev.make(4) for _ in range(8)]
                for i, tr in enumerate(trs):
                    step(i, tr)
                torch.cuda.synchronize()
                gu = sum(ev.ms(tr[0], tr[1]) for tr in trs) * 1e3 / len(trs)
                prev = rec.get(f"rows{m}")
                if prev is None or us < prev["us_per_layer"]:
                    rec[f"rows{m}"] = {"us_per_layer": round(us, 2),
                                       "tok_s": round(T / (us * 1e-6), 1), "gate_up_us": round(gu, 2)}
            rec["touched_experts"] = int((r.counts.cpu().numpy() > 0).sum())
            rows.append(rec)
            log(f"item rows T={T} skew={skew}: " + ", ".join(
                f"{m} rows {rec[f'rows{m}']['us_per_layer']:.1f} us/layer "
                f"(gate/up {rec[f'rows{m}']['gate_up_us']:.1f})" for m in (128, 64, 32, 16)))
            del r, y
    del sets, ws
    torch.cuda.empty_cache()
    return rows


def cpu_baseline(n_tokens):
    import oracle
    from workloads import WORKLOADS, make_layer
    w = WORKLOADS["prefill2048"]
    L, x = make_layer(w)
    xs = x[:n_tokens]
    t0 = time.perf_counter()
    logits = oracle.router_logits(xs, L["w_router"], L["router_bias"])
    r = oracle.route(logits, w.top_k)
    oracle.layer_tokens(L, xs, np.arange(n_tokens, dtype=np.int32), r["idx"], r["w"])
    sec = time.perf_counter() - t0
    return {"value": round(n_tokens / sec, 3), "unit": "tok/s", "cores": oracle.threads(),
            "kind": "oracle", "seconds": round(sec, 2), "host": host_info(),
            "sample": f"first {n_tokens} tokens of the prefill T=2048 layer: router logits, "
                      f"routing and all {w.top_k}+1 expert FFNs of those tokens (fp64 oracle)"}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # about 60 ms of untimed layer calls: the first tens of calls run up to 15 %
    # slower (clocks and caches settling), measured over 20 .. 400 warm-up calls
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--decode-steps", type=int, default=256)
    ap.add_argument("--decode-layers", type=int, default=40)
    ap.add_argument("--decode-warmup", type=int, default=1,
                    help="untimed decode passes over the layers before the timed steps")
    ap.add_argument("--cpu-tokens", type=int, default=768)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-handoff", action="store_true",
                    help="skip the greedy token hand-off (output head + argmax) measurement")
    ap.add_argument("--no-decode-tokens", action="store_true",
                    help="skip the few-token decode figures (T = 2, 4, 8)")
    ap.add_argument("--sweep", default=None, metavar="T1,T2,...",
                    help="only the prefill sweep over these chunk sizes (balanced and skewed)")
    ap.add_argument("--no-ablation", action="store_true",
                    help="skip the gate/up item-height ablation (128 / 64 / 32 rows)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other prefill workloads (tiny, T=512, skewed T=4096)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a plain 256 MiB copy (for HBM byte-counter calibration)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: this layer build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE={world}).", file=sys.stderr)
        sys.exit(2)

    import torch
    import q4_routed_expert_amd as q4
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    ev = HipEvents()
    stream = int(torch.cuda.current_stream().cuda_stream)
    if args.copy_calibration:
        copy_calibration(torch)
    if args.sweep:
        rows = bench_sweep(args, q4, torch, ev, stream)
        ev.close()
        print(json.dumps({"metric": "prefill MoE-layer us/layer over chunk sizes T", "unit": "us",
                          "n_gpus": 1, "higher_is_better": False, "data": "synthetic",
                          "config": {"workload": "routed-MoE FFN layer, d=2048, I=512, E=256, "
                                                 "top-8 + 1 shared, Q4 group-64, 2 weight sets"},
                          "sweep": rows}), flush=True)
        return
    pci = gpu_pci(torch)
    clocks_before = gpu_clocks(pci)
    pre = bench_prefill(args, q4, torch, ev, stream)
    configs = {} if args.no_configs else {
        n: bench_config(n, args, q4, torch, ev, stream) for n in ("tiny", "prefill512", "skew4096")}
    abl = None if args.no_ablation else bench_item_rows(args, q4, torch, ev, stream)
    dec = None if args.no_decode else bench_decode(args, q4, torch, ev, stream)
    hand = None if args.no_handoff else bench_handoff(args, q4, torch, ev, stream)
    cpu = None if args.no_cpu_baseline else cpu_baseline(args.cpu_tokens)
    ev.close()
    w = pre["workload"]
    ms_step = pre["ms_per_step"]
    line = {
        "metric": METRIC, "value": round(w.T / (ms_step * 1e-3), 1), "unit": "tok/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"routed-MoE FFN layer, prefill chunk T={w.T}, d={w.d}, "
                               f"I={w.inter}, E={w.n_experts}, top-{w.top_k} + 1 shared expert, "
                               f"Q4 group-64 weights (bf16 scale/bias), 2 weight sets alternated",
                   "T": w.T, "d": w.d, "inter": w.inter, "n_experts": w.n_experts,
                   "top_k": w.top_k, "seed": w.seed},
        "us_per_layer": round(ms_step * 1e3, 2),
        "tflops": round(pre["work"]["flops"] / (ms_step * 1e-3) / 1e12, 2),
        "mfma_frac": round(pre["work"]["flops"] / (ms_step * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "gbps": round(pre["work"]["bytes"] / (ms_step * 1e-3) / 1e9, 1),
        "hbm_frac": round(pre["work"]["bytes"] / (ms_step * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
        "kernel_us": {n: round(v, 2) for n, v in pre["kernel_us"].items()},
        "algorithmic": {"flops": pre["work"]["flops"], "bytes": pre["work"]["bytes"],
                        "touched_experts": pre["work"]["touched_experts"]},
        "roofline": pre["roofline"],
    }
    if "graph" in pre:
        line["graph"] = {k: (round(v, 4) if isinstance(v, float) else v)
                         for k, v in pre["graph"].items()}
    if dec is not None:
        line["decode"] = {k: (round(v, 4) if isinstance(v, float) else v) for k, v in dec.items()
                          if k not in ("roofline", "graph", "kernel_us", "tokens")}
        line["decode"]["kernel_us"] = {n: round(v, 3) for n, v in dec["kernel_us"].items()}
        if "graph" in dec:
            line["decode"]["graph"] = {k: (round(v, 4) if isinstance(v, float) else v)
                                       for k, v in dec["graph"].items()}
        line["decode"]["tokens"] = dec["tokens"]
        line["roofline_decode"] = dec["roofline"]
    if configs:
        line["configs"] = configs
    if abl is not None:
        line["sweep"] = {"gate_up_item_rows": abl}
    if hand is not None:
        line["handoff"] = {k: v for k, v in hand.items() if k != "roofline"}
        line["roofline_handoff"] = hand["roofline"]
    line["clocks"] = {"idle_before": clocks_before, "under_load": pre["clocks_under_load"],
                      "idle_after": gpu_clocks(pci)}
    if cpu is not None:
        line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
