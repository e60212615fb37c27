#!/usr/bin/env python3
"""Benchmark of the quantized MoE layer on one MI355X.

Default run: the Qwen3-30B-A3B-shaped INT4 (block 32) layer, H=2048, I=768,
E=128, top-8, bf16 activations, decoding M=4 tokens per step (the headline
line), plus M=1 decode and the 8192-token packed prefill as extra entries.

Timing. Every timed region is bracketed by torch.cuda.synchronize(). Inside,
a short spin kernel first holds the stream while the host enqueues the K
steps, then HIP events on that stream time exactly the K steps on the GPU, so
host launch overhead is not mistaken for layer time. Decode steps rotate over
NROT independently seeded layer instances (weights, activations, logits)
whose combined active-expert bytes exceed the 256 MB MALL, so the weights
come from HBM as they would in a deep model.

Roofline. A second pass enables the library's stage hook, which records a
HIP event on the stream after each kernel launch; per-kernel durations come
from those events. The fused decode is a single launch per step, so its
duration is the per-step time of the timed region itself. Algorithmic bytes
(decode: active experts' codes and scales, x, logits, out) and FLOPs
(prefill) per launch are counted from the routing the call actually made
(distinct experts per call).

HBM traffic. roofline.traffic is the dominant kernel's HBM bytes per launch
(the fused decode; for the 8K prefill entry, the FC1 GEMM) as rocprofv3
counters measured them (FETCH_SIZE + WRITE_SIZE, each
scaled by what the same counter reads for a plain copy of known size), read
from the committed counter summary under profiles/ only if that summary was
taken on the current kernel source (a digest of the sources is recorded with
it); otherwise null.

CPU baseline. The plain C oracle, timed on a bounded sample of tokens of the
same workload on this host's cores.

Extra entries: M=1 decode and the 8192-token prefill of the same layer; the
INT3 (block 64) layer at M=4 decode and as a 2048-token prefill; one pass over
a stack of 48 independent INT2 (block 32) layers with Zipf routing drawn per
layer, at M=1 decode and as a 32768-token packed prefill; batches of 32 and
64 tokens of the INT4 layer (the small-batch path). Each entry reports the
per-step min / median / max over its timed steps; prefill entries the load
skew of their routing (routes per expert).

`--only <workload>` runs one workload alone (for profiling) and prints its
results instead of the benchmark line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import qmoe_inputs as qi  # noqa: E402
import quantized_mixture_experts_qmoe_amd as q  # noqa: E402

METRIC = "QMoE layer tokens/s: decode M=1..4 (%HBM peak), 8K prefill (%MFMA peak)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
F16_PEAK_TFLOPS = 2500.0       # MI355X dense fp16 (and bf16) MFMA, TFLOP/s
NROT = 24
DEV = torch.device("cuda:0")
_CSRC = "quantized_mixture_experts_qmoe_amd/csrc/"
_COMMON = [_CSRC + "device.h", _CSRC + "internal.h"]
# Committed counter summaries (profiles/) and the sources each was taken on:
# a summary's figures are reported only while the digest recorded in it
# matches the digest of those sources now.
TRAFFIC = {
    "decode4": ("decode_fused_traffic_qwen3_int4_m4.txt", [_CSRC + "decode_fused.hip"] + _COMMON),
    "decode1": ("decode_fused_traffic_qwen3_int4_m1.txt", [_CSRC + "decode_fused.hip"] + _COMMON),
    "int3_decode4": ("decode_fused_traffic_qwen3_int3_m4.txt", [_CSRC + "decode_fused.hip"] + _COMMON),
    "stack_decode1": ("decode_fused_traffic_int2_stack_m1.txt", [_CSRC + "decode_fused.hip"] + _COMMON),
    "prefill": ("prefill_traffic_qwen3_int4_8k.txt", [_CSRC + "prefill.hip"] + _COMMON),
    "small32": ("small_traffic_qwen3_int4_t32.txt", [_CSRC + "small.hip", _CSRC + "route.hip",
                                                     _CSRC + "prefill.hip"] + _COMMON),
}
TRAFFIC_SOURCES = TRAFFIC["decode4"][1]
PREFILL_SOURCES = TRAFFIC["prefill"][1]


def kernel_source_digest(sources=None) -> str:
    h = hashlib.sha256()
    for rel in (TRAFFIC_SOURCES if sources is None else sources):
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload="decode4", key="hbm_bytes_per_launch"):
    """Counter-measured HBM bytes per launch of a workload's dominant kernel
    from its committed counter summary, or None if there is none taken on
    the current kernel sources."""
    name, sources = TRAFFIC[workload]
    try:
        with open(os.path.join(ROOT, "profiles", name)) as f:
            kv = dict(line.split(":", 1) for line in f if ":" in line and not line.startswith(("#", "|", "-")))
    except OSError:
        return None
    kv = {k.strip(): v.strip() for k, v in kv.items()}
    if kv.get("source_digest") != kernel_source_digest(sources):
        return None
    try:
        return float(kv[key])
    except (KeyError, ValueError):
        return None


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# ----------------------------------------------------------------- instances

def make_layer(spec: qi.LayerSpec, w: qi.LayerWeights, max_tokens: int) -> q.QMoELayer:
    cfg = q.LayerConfig(spec.hidden, spec.inter, spec.num_experts, spec.top_k, spec.bits,
                        spec.block_size, spec.zero_point, torch.bfloat16, max_tokens)
    return q.QMoELayer(cfg, torch.from_numpy(w.fc1_codes).to(DEV),
                       torch.from_numpy(w.fc1_scales).to(DEV),
                       torch.from_numpy(w.fc2_codes).to(DEV),
                       torch.from_numpy(w.fc2_scales).to(DEV))


def device_instance(spec: qi.LayerSpec, T: int, seed: int, max_tokens: int, zipf_s=None):
    """A layer instance drawn on the GPU (same distributions as qmoe_inputs;
    with zipf_s, the logits carry that layer's Zipf popularity bias)."""
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    E, H, I, bs, c = spec.num_experts, spec.hidden, spec.inter, spec.block_size, spec.scale_c

    def codes(n, kk):
        return torch.randint(0, 256, (E, n, kk * spec.bits // 8), generator=g, device=DEV,
                             dtype=torch.uint8)

    def scales(n, kk):
        return (torch.randn((E, n, kk // bs), generator=g, device=DEV).abs() * c + 1e-3).half()

    w = (codes(2 * I, H), scales(2 * I, H), codes(H, I), scales(H, I))
    cfg = q.LayerConfig(spec.hidden, spec.inter, spec.num_experts, spec.top_k, spec.bits,
                        spec.block_size, spec.zero_point, torch.bfloat16, max_tokens)
    layer = q.QMoELayer(cfg, *w)
    x = torch.randn((T, H), generator=g, device=DEV).bfloat16()
    logits = torch.randn((T, E), generator=g, device=DEV, dtype=torch.float64)
    if zipf_s is not None:
        bias = qi.zipf_bias(E, zipf_s, np.random.default_rng(seed))
        logits = logits + torch.from_numpy(bias).to(DEV)[None, :]
    return layer, x, logits.bfloat16()


def expert_bytes(spec: qi.LayerSpec):
    H, I, bs, b = spec.hidden, spec.inter, spec.block_size, spec.bits
    fc1 = 2 * I * H * b // 8 + 2 * I * (H // bs) * 2
    fc2 = H * I * b // 8 + H * (I // bs) * 2
    return fc1, fc2


# ----------------------------------------------------------------- timing

_SLEEP_CYCLES = None


def _hold_stream(seconds: float):
    """Enqueue a spin kernel that keeps the stream busy for about `seconds`."""
    global _SLEEP_CYCLES
    if _SLEEP_CYCLES is None:
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        torch.cuda._sleep(1_000_000)
        b.record()
        torch.cuda.synchronize()
        _SLEEP_CYCLES = 1_000_000 / max(a.elapsed_time(b) / 1e3, 1e-6)   # cycles per second
    torch.cuda._sleep(int(_SLEEP_CYCLES * seconds))


def step_spread(step, K: int, hold_s: float):
    """Per-step GPU times (us) of K calls, each bracketed by events on the
    stream while a spin kernel holds it: min, median and max."""
    torch.cuda.synchronize()
    _hold_stream(hold_s)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    evs[0].record()
    for i in range(K):
        step(i)
        evs[i + 1].record()
    torch.cuda.synchronize()
    us = np.array([evs[i].elapsed_time(evs[i + 1]) * 1e3 for i in range(K)])
    return {"min": float(us.min()), "median": float(np.median(us)), "max": float(us.max())}


def time_steps(step, K: int, hold_s: float):
    """GPU time of exactly K calls of step(i), host enqueue hidden behind a spin kernel."""
    torch.cuda.synchronize()
    _hold_stream(hold_s)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for i in range(K):
        step(i)
    end.record()
    enqueue_s = time.perf_counter() - t0
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - t0
    return start.elapsed_time(end) / K, enqueue_s, wall_s


def kernel_times(layers, step, K: int, hold_s: float):
    """Duration (ms) per kernel role: the median over the calls of the
    interval between the events the stage hook records around it. (A host
    stall while the steps are enqueued lands in one interval; the median
    keeps it out.)"""
    marks = []

    def hook(stage, name):
        ev = torch.cuda.Event(enable_timing=True)
        ev.record()
        marks.append((stage, name, ev))

    for L in layers:
        L.set_stage_hook(hook)
    torch.cuda.synchronize()
    _hold_stream(hold_s)
    for i in range(K):
        step(i)
    torch.cuda.synchronize()
    for L in layers:
        L.set_stage_hook(None)
    per = {}
    for a, b in zip(marks, marks[1:]):
        if b[0] == 0:
            continue            # next call starts
        per.setdefault(b[1], []).append(a[2].elapsed_time(b[2]))
    return {k: float(np.median(v)) for k, v in per.items()}


# ----------------------------------------------------------------- workloads

def bench_decode(T: int, steps: int, warmup: int, name: str = "decode"):
    spec = qi.QWEN3_INT4 if name == "decode" else qi.QWEN3_INT3
    log(f"[bench] {name} M={T}: building {NROT} layer instances")
    wl0 = qi.make_workload(name, T=T)
    insts = [(make_layer(spec, wl0.weights, 4), wl0.tokens.x.to(DEV), wl0.tokens.logits.to(DEV))]
    for i in range(1, NROT):
        insts.append(device_instance(spec, T, 1000 * T + i + (0 if name == "decode" else 500), 4))
    ws = insts[0][0].workspace(T)
    out = torch.empty((T, spec.hidden), dtype=torch.bfloat16, device=DEV)

    def step(i):
        L, x, l = insts[i % NROT]
        L.forward(x, l, out=out, workspace=ws)

    # distinct experts of each instance (from the routing the layer computed)
    distinct = []
    for i in range(NROT):
        step(i)
        ids, _ = insts[i][0].routing_from_workspace(T, ws)
        distinct.append(int(torch.unique(ids).numel()))
    torch.cuda.synchronize()
    for i in range(warmup):
        step(i)
    ms, enq, wall = time_steps(step, steps, hold_s=0.002 + steps * 1e-4)
    spread = step_spread(step, steps, hold_s=0.002 + steps * 1e-4)
    log(f"[bench] {name} M={T}: {ms * 1e3:.2f} us/step (enqueue {enq * 1e3:.1f} ms, wall {wall * 1e3:.1f} ms); "
        f"per step min {spread['min']:.2f} median {spread['median']:.2f} max {spread['max']:.2f} us")
    kt = kernel_times([it[0] for it in insts], step, min(steps, 4 * NROT), hold_s=0.01)
    log(f"[bench] {name} M={T} kernels (us): " + ", ".join(f"{k}={v * 1e3:.2f}" for k, v in kt.items()))
    fc1_b, fc2_b = expert_bytes(spec)
    D = float(np.mean([distinct[i % NROT] for i in range(steps)]))
    H, I, E, k = spec.hidden, spec.inter, spec.num_experts, spec.top_k
    R = T * k
    fc1_bytes = D * fc1_b + T * H * 2 + T * E * 2 + R * I * 4
    layer_bytes = D * (fc1_b + fc2_b) + T * H * 2 * 2 + T * E * 2
    if list(kt) == ["decode_fused"]:
        # one launch computes the whole layer, so a step is exactly one launch of
        # it: its duration is the per-step time of the timed region (the stage
        # hook's events would add the dispatch latency before the launch), and
        # its algorithmic bytes are the layer's (active experts, x, logits, out)
        dom = "decode_fused"
        dom_bytes = layer_bytes
        t_dom = ms * 1e-3
        kt = {"decode_fused": ms}
    else:
        dom = "decode_fc1_swiglu"
        dom_bytes = fc1_bytes
        t_dom = kt[dom] * 1e-3
    return {
        "T": T, "ms_per_step": ms, "tokens_per_s": T / (ms * 1e-3),
        "distinct_experts": D,
        "layer_GBs": layer_bytes / (ms * 1e-3) / 1e9,
        "layer_frac_hbm": layer_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "kernels_us": {kk: v * 1e3 for kk, v in kt.items()},
        "step_us": spread,
        "dominant": {"kernel": dom, "bytes": dom_bytes, "s": t_dom, "GBs": dom_bytes / t_dom / 1e9},
    }


def bench_prefill(steps: int, warmup: int, name: str = "prefill", T: int = 8192):
    spec = qi.QWEN3_INT4 if name == "prefill" else qi.QWEN3_INT3
    log(f"[bench] {name} {T}: building layer")
    wl = qi.make_workload(name, T=T)
    L = make_layer(spec, wl.weights, T)
    x, l = wl.tokens.x.to(DEV), wl.tokens.logits.to(DEV)
    ws = L.workspace(T)
    out = torch.empty((T, spec.hidden), dtype=torch.bfloat16, device=DEV)

    def step(i):
        L.forward(x, l, out=out, workspace=ws)

    for i in range(warmup):
        step(i)
    ids, _ = L.routing_from_workspace(T, ws)
    per_expert = torch.bincount(ids.reshape(-1).long(), minlength=spec.num_experts).float()
    skew = {"max_routes_per_expert": int(per_expert.max().item()),
            "mean_routes_per_active_expert": float(per_expert[per_expert > 0].mean().item()),
            "active_experts": int((per_expert > 0).sum().item())}
    ms, enq, wall = time_steps(step, steps, hold_s=0.005)
    spread = step_spread(step, steps, hold_s=0.005)
    kt = kernel_times([L], step, steps, hold_s=0.005)
    log(f"[bench] {name} {T}: {ms:.3f} ms/step; kernels (us): "
        + ", ".join(f"{k}={v * 1e3:.1f}" for k, v in kt.items()))
    H, I, k = spec.hidden, spec.inter, spec.top_k
    R = T * k
    flops = 2.0 * R * (2 * I * H + H * I)
    fc1_flops = 2.0 * R * 2 * I * H
    t_fc1 = kt["gemm_fc1_swiglu"] * 1e-3
    return {
        "T": T, "ms_per_step": ms, "tokens_per_s": T / (ms * 1e-3),
        "layer_TFLOPs": flops / (ms * 1e-3) / 1e12,
        "layer_frac_mfma": flops / (ms * 1e-3) / 1e12 / F16_PEAK_TFLOPS,
        "kernels_us": {kk: v * 1e3 for kk, v in kt.items()},
        "step_us": spread, "load_skew": skew,
        "fc1": {"flops": fc1_flops, "s": t_fc1, "TFLOPs": fc1_flops / t_fc1 / 1e12},
    }


def bench_small(T: int, steps: int, warmup: int):
    """Batches between decode and prefill (the small-batch path): one layer
    call on T tokens, rotating NROT / 4 seeded instances so the MALL holds
    none of the active experts' weights. Roofline: the active experts'
    weight bytes (each streamed once per call) over the call's time."""
    spec = qi.QWEN3_INT4
    n = NROT // 4
    log(f"[bench] small batch T={T}: building {n} layer instances")
    insts = [device_instance(spec, T, 7000 + T + i, T) for i in range(n)]
    ws = insts[0][0].workspace(T)
    out = torch.empty((T, spec.hidden), dtype=torch.bfloat16, device=DEV)

    def step(i):
        L, x, l = insts[i % n]
        L.forward(x, l, out=out, workspace=ws)

    distinct = []
    for i in range(n):
        step(i)
        ids, _ = insts[i][0].routing_from_workspace(T, ws)
        distinct.append(int(torch.unique(ids).numel()))
    for i in range(warmup):
        step(i)
    ms, enq, wall = time_steps(step, steps, hold_s=0.002 + steps * 2e-4)
    spread = step_spread(step, steps, hold_s=0.002 + steps * 2e-4)
    kt = kernel_times([it[0] for it in insts], step, min(steps, 4 * n), hold_s=0.01)
    fc1_b, fc2_b = expert_bytes(spec)
    D = float(np.mean([distinct[i % n] for i in range(steps)]))
    H, E = spec.hidden, spec.num_experts
    layer_bytes = D * (fc1_b + fc2_b) + T * H * 2 * 2 + T * E * 2
    log(f"[bench] small batch T={T}: {ms * 1e3:.1f} us/step, {D:.1f} experts, kernels (us): "
        + ", ".join(f"{k}={v * 1e3:.1f}" for k, v in kt.items()))
    for L, _, _ in insts:
        L.close()
    return {"T": T, "ms_per_step": ms, "tokens_per_s": T / (ms * 1e-3), "distinct_experts": D,
            "layer_frac_hbm": layer_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "kernels_us": {kk: v * 1e3 for kk, v in kt.items()}, "step_us": spread}


def bench_stack(T: int, steps: int, warmup: int):
    """One pass over the 48 independent INT2 layers (Qwen3-30B-A3B shape,
    Zipf(1.1) routing drawn per layer), layers back to back on one stream.
    T=1 decodes one token per layer; T=32768 is the packed prefill."""
    spec = qi.QWEN3_INT2
    nl = 48
    log(f"[bench] stack T={T}: building {nl} layers")
    layers = [device_instance(spec, T, 5 + l, T, zipf_s=1.1) for l in range(nl)]
    ws = layers[0][0].workspace(T)
    out = torch.empty((T, spec.hidden), dtype=torch.bfloat16, device=DEV)

    def step(i):
        for L, x, lg in layers:
            L.forward(x, lg, out=out, workspace=ws)

    distinct = []
    if T == 1:
        for L, x, lg in layers:
            L.forward(x, lg, out=out, workspace=ws)
            ids, _ = L.routing_from_workspace(T, ws)
            distinct.append(int(torch.unique(ids).numel()))
    torch.cuda.synchronize()
    for i in range(warmup):
        step(i)
    ms, enq, wall = time_steps(step, steps, hold_s=0.002 + steps * nl * (2e-5 if T == 1 else 1e-4))
    log(f"[bench] stack T={T}: {ms:.3f} ms/pass of {nl} layers")
    H, I, k = spec.hidden, spec.inter, spec.top_k
    res = {"T": T, "layers": nl, "ms_per_pass": ms, "tokens_per_s": T / (ms * 1e-3),
           "layer_us": ms * 1e3 / nl}
    if T == 1:
        fc1_b, fc2_b = expert_bytes(spec)
        nbytes = sum(distinct) * (fc1_b + fc2_b) + nl * (H * 2 * 2 + spec.num_experts * 2)
        res["bytes_per_pass"] = nbytes
        res["frac_hbm"] = nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS
    else:
        flops = nl * 2.0 * T * k * (2 * I * H + H * I)
        res["flops_per_pass"] = flops
        res["frac_mfma"] = flops / (ms * 1e-3) / 1e12 / F16_PEAK_TFLOPS
    for L, _, _ in layers:
        L.close()
    del layers, ws
    torch.cuda.empty_cache()
    return res


def cpu_model() -> str:
    """The host CPU's model name, as /proc/cpuinfo and lscpu give it."""
    names = []
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    names.append(line.split(":", 1)[1].strip())
                    break
    except OSError:
        pass
    try:
        import subprocess
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith(("Model name", "Vendor ID", "Socket(s)", "Core(s) per socket")):
                names.append(" ".join(line.split()))
    except Exception:
        pass
    return "; ".join(names) if names else "unknown"


def cpu_baseline(n_tokens: int):
    """The oracle, as it stands, on bounded samples of each workload: all
    host cores (the reported value is the decode workload's), and one thread
    on a smaller sample. The 48 layers of the stack are independent and of
    one shape, so one layer's sampled per-token cost stands for each."""
    import oracle
    threads = oracle.default_threads()

    def timed(name, T, nthreads, **kw):
        wl = qi.make_workload(name, T=T, **kw)
        layer = oracle.Layer.from_spec(wl.spec)
        t0 = time.perf_counter()
        oracle.forward(layer, wl.tokens.x, wl.tokens.logits, wl.weights, nthreads=nthreads)
        return time.perf_counter() - t0

    dt = timed("decode", n_tokens, threads)
    n1 = max(1, n_tokens // 8)
    dt1 = timed("decode", n1, 1)
    others = {}
    for label, name, T in (("prefill_8k_sample", "prefill", 128), ("int3_sample", "int3", 64),
                           ("stack_layer_sample", "stack", 256)):
        d = timed(name, T, threads)
        others[label] = {"value": T / d, "unit": "tokens/s per layer", "tokens": T, "wall_s": d}
    log(f"[bench] cpu baseline: {threads} threads {n_tokens / dt:.1f} tokens/s, "
        f"1 thread {n1 / dt1:.2f} tokens/s; " + ", ".join(f"{k} {v['value']:.1f}" for k, v in others.items()))
    return {"value": n_tokens / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{n_tokens} tokens of the decode workload (Qwen3-30B-A3B-shaped INT4 bs32 "
                      f"layer, uniform routing), {dt:.1f} s wall on {threads} threads",
            "single_thread": {"value": n1 / dt1, "unit": "tokens/s", "sample": f"{n1} tokens"},
            "other_workloads": {
                **others,
                "note": "prefill: the first 128 tokens of the 8192-token Zipf workload; int3: 64 tokens "
                        "of the INT3 bs64 layer; stack: 256 tokens of layer 0 of the 48-layer INT2 "
                        "stack (every layer has this shape and cost; a pass costs 48 times a layer)"},
            "cpu_model": cpu_model()}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--prefill-steps", type=int, default=20)
    ap.add_argument("--no-extra", action="store_true", help="skip the M=1 and 8K prefill entries")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=96)
    ap.add_argument("--only", choices=["decode4", "decode1", "prefill", "int3_decode4",
                                       "int3_prefill", "stack_decode1", "stack_prefill",
                                       "small32", "small64"],
                    default=None,
                    help="run one workload alone (profiling aid); prints its results")
    ap.add_argument("--source-digest", action="store_true",
                    help="print the digest of the fused decode sources and exit")
    args = ap.parse_args()
    if args.source_digest:
        print(kernel_source_digest())
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the layer is measured on one GPU's share)", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    q.lib()   # fail loudly if the HIP library is missing

    if args.only:
        if args.only == "prefill":
            res = bench_prefill(args.steps, args.warmup)
        elif args.only == "int3_prefill":
            res = bench_prefill(args.steps, args.warmup, "int3", 2048)
        elif args.only == "int3_decode4":
            res = bench_decode(4, args.steps, args.warmup, "int3")
        elif args.only.startswith("small"):
            res = bench_small(int(args.only[5:]), args.steps, args.warmup)
        elif args.only.startswith("stack"):
            res = bench_stack(1 if args.only == "stack_decode1" else 32768, args.steps, args.warmup)
        else:
            res = bench_decode(4 if args.only == "decode4" else 1, args.steps, args.warmup)
        print(json.dumps({"only": args.only, **res}), flush=True)
        return

    main_res = bench_decode(4, args.steps, args.warmup)
    extra = []
    if not args.no_extra:
        m1 = bench_decode(1, args.steps, args.warmup)
        pf = bench_prefill(args.prefill_steps, 3)
        i3d = bench_decode(4, args.steps, args.warmup, "int3")
        i3p = bench_prefill(args.prefill_steps, 3, "int3", 2048)
        sd = bench_stack(1, 20, 3)
        sp = bench_stack(32768, 3, 1)
        smalls = [bench_small(T, args.steps // 2, args.warmup) for T in (32, 64)]
        extra = [
            {"workload": "decode M=1", "tokens_per_s": m1["tokens_per_s"],
             "ms_per_step": m1["ms_per_step"], "layer_frac_hbm": m1["layer_frac_hbm"],
             "distinct_experts": m1["distinct_experts"], "kernels_us": m1["kernels_us"],
             "step_us": m1["step_us"],
             "roofline": {"bound": "hbm", "kernel": m1["dominant"]["kernel"],
                          "achieved": m1["dominant"]["GBs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": m1["dominant"]["GBs"] / HBM_PEAK_GBS,
                          "traffic": measured_traffic("decode1")}},
            {"workload": "prefill 8192 tokens (16 packed sequences, Zipf-skewed routing)",
             "tokens_per_s": pf["tokens_per_s"], "ms_per_step": pf["ms_per_step"],
             "layer_frac_mfma": pf["layer_frac_mfma"], "kernels_us": pf["kernels_us"],
             "step_us": pf["step_us"], "load_skew": pf["load_skew"],
             "roofline": {"bound": "mfma", "kernel": "gemm_fc1_swiglu",
                          "achieved": pf["fc1"]["TFLOPs"], "peak": F16_PEAK_TFLOPS,
                          "unit": "TFLOP/s", "frac": pf["fc1"]["TFLOPs"] / F16_PEAK_TFLOPS,
                          "traffic": measured_traffic("prefill", "fc1_hbm_bytes_per_launch")}},
            {"workload": "INT3 bs64 layer decode M=4 (uniform routing)",
             "tokens_per_s": i3d["tokens_per_s"], "ms_per_step": i3d["ms_per_step"],
             "layer_frac_hbm": i3d["layer_frac_hbm"], "distinct_experts": i3d["distinct_experts"],
             "kernels_us": i3d["kernels_us"],
             "roofline": {"bound": "hbm", "kernel": i3d["dominant"]["kernel"],
                          "achieved": i3d["dominant"]["GBs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": i3d["dominant"]["GBs"] / HBM_PEAK_GBS,
                          "traffic": measured_traffic("int3_decode4")}},
            {"workload": "INT3 bs64 layer prefill 2048 tokens (8 packed sequences)",
             "tokens_per_s": i3p["tokens_per_s"], "ms_per_step": i3p["ms_per_step"],
             "layer_frac_mfma": i3p["layer_frac_mfma"], "kernels_us": i3p["kernels_us"],
             "step_us": i3p["step_us"], "load_skew": i3p["load_skew"],
             "roofline": {"bound": "mfma", "kernel": "gemm_fc1_swiglu",
                          "achieved": i3p["fc1"]["TFLOPs"], "peak": F16_PEAK_TFLOPS,
                          "unit": "TFLOP/s", "frac": i3p["fc1"]["TFLOPs"] / F16_PEAK_TFLOPS}},
            {"workload": "48-layer INT2 bs32 stack, M=1 decode pass (Zipf routing per layer)",
             "tokens_per_s": sd["tokens_per_s"], "ms_per_pass": sd["ms_per_pass"],
             "layer_us": sd["layer_us"], "bytes_per_pass": sd["bytes_per_pass"],
             "frac_hbm": sd["frac_hbm"],
             "traffic_per_layer": measured_traffic("stack_decode1")},
            {"workload": "48-layer INT2 bs32 stack, 32768-token packed prefill pass",
             "tokens_per_s": sp["tokens_per_s"], "ms_per_pass": sp["ms_per_pass"],
             "layer_us": sp["layer_us"], "flops_per_pass": sp["flops_per_pass"],
             "frac_mfma": sp["frac_mfma"]},
        ] + [
            {"workload": f"small batch {r['T']} tokens (uniform routing, small-batch path)",
             "tokens_per_s": r["tokens_per_s"], "ms_per_step": r["ms_per_step"],
             "distinct_experts": r["distinct_experts"], "layer_frac_hbm": r["layer_frac_hbm"],
             "kernels_us": r["kernels_us"], "step_us": r["step_us"],
             "fc1_traffic": measured_traffic("small32", "fc1_hbm_bytes_per_launch")
             if r["T"] == 32 else None}
            for r in smalls
        ]
    cpu = None if args.no_cpu_baseline else cpu_baseline(args.cpu_tokens)

    dom = main_res["dominant"]
    line = {
        "metric": METRIC,
        "value": main_res["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "Qwen3-30B-A3B-shaped QMoE layer decode, M=4 tokens per step "
                               "(INT4 bs32, H=2048, I=768, E=128, top-8, bf16 in/out)",
                   "tokens_per_step": 4, "layer_instances_rotated": NROT,
                   "distinct_experts_per_step": main_res["distinct_experts"],
                   "layer_frac_hbm": main_res["layer_frac_hbm"],
                   "kernels_us": main_res["kernels_us"], "step_us": main_res["step_us"]},
        "roofline": {"bound": "hbm", "kernel": dom["kernel"], "achieved": dom["GBs"],
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": dom["GBs"] / HBM_PEAK_GBS,
                     "bytes_per_launch": dom["bytes"],
                     "traffic": measured_traffic("decode4") if dom["kernel"] == "decode_fused" else None},
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
