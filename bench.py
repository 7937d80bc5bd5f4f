#!/usr/bin/env python3
"""Benchmark of the MoE FFN hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-extra]

One step is one pass of the whole sub-block over one batch of synthetic
input: RMSNorm -> router -> permutation -> grouped gate/up GEMM -> grouped
down GEMM -> combine, on the prefill workload (8192 tokens, d 4096, expert
intermediate 2048, 32 of 256 experts local, Zipf-skewed router bias, bf16).
Inputs and weights are resident in HBM before the timed region. W untimed
warm-up steps, then exactly K steps between two device synchronisations;
HIP events on the launch stream bracket every stage of every timed step.
The warm-up default is long enough for the clock to settle after the idle
time of input generation: the first few tens of steps after it run slower.
The same step is then also timed as a HIP graph (the forward captured once
and replayed, W + K replays), each replay checked to reproduce the eager
output bit for bit (`graph_ms_per_step`).

Prints ONE JSON line: tokens/s of the whole step, the roofline of the
dominant kernel (the grouped gate/up GEMM, against the bf16 MFMA peak), the
per-stage times and roofline fractions, extra measurements (decode-shaped
fp8 MoE, the dense TP shard, the router-only workload) and the fp64 CPU
oracle timed on this host (same workload) as a baseline.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE FFN tokens/s per layer on 1 GPU; grouped-GEMM % MFMA peak; decode % HBM BW"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0       # MI355X dense fp8 MFMA
PREFILL = "moe_prefill_8192tok_32exp_bf16"
DECODE = "moe_decode_64tok_256exp_fp8"
PREFILL_FP8 = "moe_prefill_8192tok_32exp_fp8act"
PREFILL_FP8W = "moe_prefill_8192tok_32exp_fp8w"
DECODE_MASKED = "moe_decode_64tok_256exp_fp8_masked"
DENSE = "norm_tp_shard_bf16_4096"
ROUTER = "router_4096tok_E256"


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the decode (contiguous and masked) / fp8-activation prefill / "
                         "dense-shard / router-only "
                         "measurements")
    ap.add_argument("--only", choices=["prefill", "decode", "dense", "router", "prefill_fp8",
                                       "decode_masked", "prefill_fp8w"],
                    default=None,
                    help="run one workload only (for profiling); prints its stage times")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="with --only: first copy a 1 GiB device buffer 3 times (a kernel of "
                         "known traffic to scale HBM byte counters against)")
    ap.add_argument("--no-graph", action="store_true",
                    help="with --only: skip the HIP-graph replays, so that a kernel trace "
                         "averages the eagerly launched steps the line reports")
    return ap.parse_args()


# ----------------------------------------------------------------- work model


def moe_work(T, d, f, E, k, S, active, ec, welt, act_fp8=False):
    """Algorithmic bytes / flops per stage of one MoE FFN step (each tensor once).

    With fp8 activations the RMSNorm pass also writes V's fp8 codes and group
    scales (d + d/32 bytes per token), the gate/up stage reads the fp8 rows,
    and the down stage quantises the live rows of H and reads them as fp8."""
    sc = 0 if welt == 2 else 4 * (f // 128) * (d // 128)  # fp8 scales per matrix
    if act_fp8:
        w = moe_work(T, d, f, E, k, S, active, ec, welt)
        w["rmsnorm"]["bytes"] += T * d + T * d // 32
        w["grouped_gate_up"]["bytes"] = (active * (2 * f * d + 2 * sc) + S * d + S * d // 32
                                         + S * f * 2 + S * 4)
        w["grouped_down"]["bytes"] = (active * (d * f + sc) + S * f * 2 + S * f + S * f // 32
                                      + S * f + S * f // 32 + S * d * 2)
        return w
    return {
        "rmsnorm": dict(bytes=2 * T * d * 2 + d * 2),
        "moe_route": dict(bytes=T * d * 2 + E * d * 2 + E * 4 + T * k * 8, flops=2 * T * d * E),
        # indices only: the rows V[src_token] are gathered by the gate/up GEMM's A load
        "moe_permute": dict(bytes=T * k * 8 + S * 4 + (ec + 1) * 8),
        "grouped_gate_up": dict(bytes=active * (2 * f * d * welt + 2 * sc) + S * d * 2 + S * f * 2
                                + S * 4,
                                flops=4 * S * d * f),
        "grouped_down": dict(bytes=active * (d * f * welt + sc) + S * f * 2 + S * d * 2,
                             flops=2 * S * f * d),
        "moe_combine": dict(bytes=S * d * 2 + T * k * 8 + T * d * 2),
    }


def measured_traffic(kernel: str, profile: str):
    """HBM bytes per launch of `kernel` (FETCH_SIZE + WRITE_SIZE, calibrated) as
    recorded in profiles/<profile>, or None when the kernel's source has changed
    since the counters were taken (the record carries the source's sha256)."""
    import hashlib
    import re
    path = os.path.join(ROOT, "profiles", profile)
    if not os.path.exists(path):
        return None
    pat = re.compile(r"bench-traffic: kernel=(\S+) source=(\S+) sha256=([0-9a-f]+) bytes_per_launch=(\d+)")
    for line in open(path, encoding="utf-8"):
        m = pat.search(line)
        if m and m.group(1) == kernel:
            src = os.path.join(ROOT, m.group(2))
            if not os.path.exists(src):
                return None
            with open(src, "rb") as f:
                if hashlib.sha256(f.read()).hexdigest() != m.group(3):
                    return None
            return int(m.group(4))
    return None


def stage_report(work, us, mfma_peak=PEAK_BF16_TFLOPS):
    out = {}
    for name, w in work.items():
        t = us[name] * 1e-6
        r = dict(us=round(us[name], 2))
        if "bytes" in w:
            gbs = w["bytes"] / t / 1e9
            r.update(gb_s=round(gbs, 1), hbm_frac=round(gbs / PEAK_HBM_GBS, 4))
        if "flops" in w:
            tf = w["flops"] / t / 1e12
            r.update(tflop_s=round(tf, 1), mfma_frac=round(tf / mfma_peak, 4))
        out[name] = r
    return out


# ------------------------------------------------------------------- runners


def summary(vals):
    """mean, median and min of per-rep times (µs)."""
    import statistics
    vals = list(vals)
    return dict(mean=sum(vals) / len(vals), median=statistics.median(vals), min=min(vals))


def warm_clock(seconds=0.25):
    """Keep the GPU under full MFMA load for `seconds` (untimed), so that a
    measurement after seconds of idle input building starts at the loaded
    clock. After 3 s idle the first 20 prefill steps measured 807 µs against
    740 µs once the clock had ramped."""
    import ctypes
    import torch
    from gated_mlp_transformer_amd import _lib
    lib = _lib.load()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    out = torch.empty(cus * 256, dtype=torch.float32, device="cuda")
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            if lib.mf_probe_mfma_bf16(cus, 2000, ctypes.c_void_p(out.data_ptr()), s) != 0:
                raise RuntimeError("bench: probe launch failed")
        torch.cuda.synchronize()


def process_warmup(iters=60):
    """Untimed, once per process before the first timed workload: small
    instances of every pipeline the bench times (1024-token prefill layers
    with 4 local experts in bf16, fp8-activation and fp8-weight form, 64-token
    decode layers with 16 local experts in both layouts, a 512-token dense
    shard and the fp32 dense shard), `iters` forwards each, through the same
    kernels. The first layer a process runs was otherwise slow for tens of
    steps whatever the clock: 1658, 822, 771, 760 µs per step over its first
    four 5-step windows against ≈ 755 µs after, while a fresh full-size layer
    built after this warm-up started at 762 µs. Each timed workload still
    gets exactly W warm-up steps of its own. Returns a description."""
    import torch
    import gated_mlp_transformer_amd as g
    import synth
    from synth.workloads import make_dense, shard_weights
    W = synth.WORKLOADS
    small = [dict(W[PREFILL], T=1024, e_count=4), dict(W[PREFILL_FP8], T=1024, e_count=4),
             dict(W[PREFILL_FP8W], T=1024, e_count=4), dict(W[DECODE], e_count=16),
             dict(W[DECODE_MASKED], e_count=16)]
    for spec in small:
        for norm in ((True, False) if spec is small[0] else (True,)):
            layer, inp = build_layer(spec, "cuda", seed=7, norm=norm)
            for _ in range(iters):
                layer(inp["x"])
            torch.cuda.synchronize()
            del layer, inp
    D = make_dense(512, 4096, 2048, dtype=torch.bfloat16, norm=True, device="cuda", seed=7)
    packed = [g.pack_weights(D[k]) for k in ("w_gate", "w_up", "w_down")]
    v = torch.empty_like(D["x"])
    for _ in range(iters):
        g.rmsnorm(D["x"], D["gamma"], 1e-5, out=v)
        g.tp_shard_mlp(v, *packed)
    spec32 = W["dense_f32_16x64_f256_p4"]
    D32 = make_dense(spec32["T"], spec32["d"], spec32["f"], dtype=torch.float32, device="cuda")
    sh = shard_weights(D32["w_gate"], D32["w_up"], D32["w_down"], spec32["p"], 0)
    for _ in range(iters):
        g.tp_shard_mlp(D32["x"], *sh)
    torch.cuda.synchronize()
    del D, packed, v, D32, sh
    torch.cuda.empty_cache()
    return (f"untimed, before the first timed workload: {iters} forwards each of small "
            "instances of every timed pipeline (1024-token prefill layers with 4 local experts "
            "in bf16 with and without RMSNorm, fp8-activation and fp8-weight form; 64-token "
            "decode layers with 16 local experts, contiguous and masked; a 512-token dense "
            "shard; the fp32 dense shard), through the same kernels")


def time_layer(layer, x, steps, warmup):
    """Warm up, then time exactly `steps` forwards back to back between two
    events. The per-stage breakdown comes from a second pass of `steps`
    forwards with an event between stages: recorded inside the timed pass,
    those events added ≈ 20 µs per prefill step (751-755 vs 730-738 µs).
    Returns (ms per step over the bracketed region, per-stage lists of µs per
    step from the second pass, wall seconds of the timed pass)."""
    import torch
    stream = torch.cuda.current_stream()
    warm_clock()
    for _ in range(warmup):
        layer(x)
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for _ in range(steps):
        layer(x)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = t_start.elapsed_time(t_end) / steps
    marks = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(steps)]
    for i in range(steps):
        layer(x, marks=marks[i])
    torch.cuda.synchronize()
    us = {name: [1e3 * m[s].elapsed_time(m[s + 1]) for m in marks]
          for s, name in enumerate(layer.STAGES)}
    us["step"] = [1e3 * m[0].elapsed_time(m[6]) for m in marks]
    return ms, us, wall


def time_layer_flushed(layer, x, reps, scratch):
    """`reps` forwards, each preceded by an untimed write of `scratch` (larger
    than the 256 MB last-level cache, so no operand stays cached from the
    previous rep). Returns per-stage lists of µs per rep."""
    import torch
    stream = torch.cuda.current_stream()
    marks = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(reps)]
    for i in range(reps):
        scratch.fill_(i & 0x7F)
        layer(x, marks=marks[i])
    torch.cuda.synchronize()
    us = {name: [1e3 * m[s].elapsed_time(m[s + 1]) for m in marks]
          for s, name in enumerate(layer.STAGES)}
    us["step"] = [1e3 * m[0].elapsed_time(m[6]) for m in marks]
    return us


def time_layer_graph(layer, x, steps, warmup):
    """The same step as a HIP graph: one forward captured (no marks), replayed
    `warmup` times untimed, then exactly `steps` replays timed. The replays must
    reproduce the eager forward bit for bit (checked before and after timing)."""
    import torch
    ref = layer(x).clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer(x)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out = layer(x)
    torch.cuda.synchronize()
    for _ in range(max(1, warmup)):
        graph.replay()
    torch.cuda.synchronize()
    if not torch.equal(out, ref):
        raise RuntimeError("bench: graph replay differs from the eager forward")
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for _ in range(steps):
        graph.replay()
    t_end.record()
    torch.cuda.synchronize()
    if not torch.equal(out, ref):
        raise RuntimeError("bench: graph replay differs from the eager forward")
    ms = t_start.elapsed_time(t_end) / steps
    del graph
    return ms


def build_layer(spec, device, seed=0, norm=True):
    import gated_mlp_transformer_amd as g
    from synth.workloads import make_moe
    inp = make_moe(spec["T"], spec["d"], spec["f"], spec["E"], spec["e_begin"], spec["e_count"],
                   wdtype=spec["wdtype"], zipf=spec["zipf"], seed=seed, device=device)
    layer = g.MoEFFNLayer(T=spec["T"], d=spec["d"], f=spec["f"], w_r=inp["w_r"],
                          bias=inp["bias"], gamma=inp["gamma"] if norm else None,
                          w_gate=inp["w_gate"], w_up=inp["w_up"], w_down=inp["w_down"],
                          e_begin=spec["e_begin"], s_gate=inp.get("s_gate"),
                          s_up=inp.get("s_up"), s_down=inp.get("s_down"),
                          act_fp8=spec.get("act_fp8", False),
                          layout=spec.get("layout", "contiguous"))
    return layer, inp


def run_moe(name, steps, warmup, scratch=None, norm=True, graph=True):
    import synth
    spec = synth.WORKLOADS[name]
    log(f"[bench] {name}{'' if norm else ' (no rmsnorm)'}: building inputs")
    layer, inp = build_layer(spec, "cuda", norm=norm)
    ms, us, wall = time_layer(layer, inp["x"], steps, warmup)
    flushed = time_layer_flushed(layer, inp["x"], steps, scratch) if scratch is not None else None
    ms_graph = time_layer_graph(layer, inp["x"], steps, warmup) if graph else None
    S = int(layer.counts.sum().item())  # both layouts (offsets are unused when masked)
    active = int((layer.counts > 0).sum().item())
    counts = layer.counts.cpu()
    welt = 2 if spec["wdtype"] == "bf16" else 1
    work = moe_work(spec["T"], spec["d"], spec["f"], spec["E"], 8, S, active, spec["e_count"],
                    welt, act_fp8=spec.get("act_fp8", False))
    if not norm:
        work["rmsnorm"] = {}
    log(f"[bench] {name}: {ms * 1e3:.1f} us/step"
        + (f", {ms_graph * 1e3:.1f} us as a graph" if graph else "")
        + f", S={S}, active experts {active}")
    info = dict(slots=S, active_experts=active,
                count_min=int(counts.min()), count_max=int(counts.max()),
                count_mean=round(float(counts.float().mean()), 1))
    return dict(spec=spec, layer=layer, inp=inp, ms=ms, ms_graph=ms_graph, us=us, wall=wall,
                flushed=flushed, work=work, info=info)


def run_dense(steps, warmup, scratch=None):
    """RMSNorm + one bf16 TP shard of the gated MLP (4096 x 4096, f_s 2048)."""
    import torch
    import gated_mlp_transformer_amd as g
    import synth
    from synth.workloads import make_dense
    spec = synth.WORKLOADS[DENSE]
    T, d, f = spec["T"], spec["d"], spec["f"]
    D = make_dense(T, d, f, dtype=torch.bfloat16, norm=True, device="cuda")
    packed = [g.pack_weights(D[k]) for k in ("w_gate", "w_up", "w_down")]
    v = torch.empty_like(D["x"])
    h = torch.empty((T, f), dtype=torch.bfloat16, device="cuda")
    part = torch.empty((T, d), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        g.rmsnorm(D["x"], D["gamma"], 1e-5, out=v)
        if ev:
            ev[1].record(stream)
        g.tp_shard_mlp(v, *packed, h_work=h, partial=part)
        if ev:
            ev[2].record(stream)

    def timed(flush):
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
        for i in range(steps):
            if flush:
                scratch.fill_(i & 0x7F)
            step(evs[i])
        torch.cuda.synchronize()
        return ([1e3 * e[0].elapsed_time(e[1]) for e in evs],
                [1e3 * e[1].elapsed_time(e[2]) for e in evs])

    warm_clock()
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    norm_us, shard_us = timed(False)
    fl = timed(True) if scratch is not None else None
    flops = 6 * T * d * f
    norm_bytes = 4 * T * d + 2 * d
    shard_bytes = 2 * T * d + 3 * 2 * d * f + 2 * 2 * T * f + 4 * T * d
    return dict(workload=DENSE, norm_us=norm_us, shard_us=shard_us, flushed=fl,
                work={"rmsnorm": dict(bytes=norm_bytes),
                      "tp_shard_mlp": dict(bytes=shard_bytes, flops=flops)})


def run_dense_f32(steps, warmup):
    """The fp32 dense workload: X 16x64, four TP shards of f = 256 (f_s = 64)
    and the sum of their partials: the latency of the whole sharded MLP."""
    import torch
    import gated_mlp_transformer_amd as g
    import synth
    from synth.workloads import make_dense, shard_weights
    spec = synth.WORKLOADS["dense_f32_16x64_f256_p4"]
    T, d, f, p = spec["T"], spec["d"], spec["f"], spec["p"]
    D = make_dense(T, d, f, dtype=torch.float32, device="cuda")
    shards = [shard_weights(D["w_gate"], D["w_up"], D["w_down"], p, i) for i in range(p)]
    hs = [torch.empty((T, f // p), dtype=torch.float32, device="cuda") for _ in range(p)]
    parts = [torch.empty((T, d), dtype=torch.float32, device="cuda") for _ in range(p)]
    out = torch.empty((T, d), dtype=torch.float32, device="cuda")

    def step():
        for i in range(p):
            g.tp_shard_mlp(D["x"], *shards[i], h_work=hs[i], partial=parts[i])
        torch.sum(torch.stack(parts), dim=0, out=out)

    warm_clock()
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for i in range(steps):
        evs[i][0].record()
        step()
        evs[i][1].record()
    torch.cuda.synchronize()
    us = [1e3 * a.elapsed_time(b) for a, b in evs]
    st = summary(us)
    return dict(workload="dense_f32_16x64_f256_p4", shards=p,
                us_median=round(st["median"], 2), us_min=round(st["min"], 2),
                what="4 tp_shard_mlp calls (fp32) + the sum of their partials")


def run_router(steps, warmup, scratch=None):
    """Router + index-only permutation over all 256 experts, 4096 tokens."""
    import torch
    import gated_mlp_transformer_amd as g
    import synth
    from synth.workloads import make_router
    spec = synth.WORKLOADS[ROUTER]
    T, d, E = spec["T"], spec["d"], spec["E"]
    r = make_router(T, d, E, device="cuda")
    w_r = g.pack_weights(r["w_r"])
    idx = torch.empty((T, 8), dtype=torch.int32, device="cuda")
    w = torch.empty((T, 8), dtype=torch.float32, device="cuda")
    ws = torch.empty(g.moe_permute_workspace_size(T, 8, E), dtype=torch.uint8, device="cuda")
    rws = torch.empty(max(1, g.moe_route_workspace_size(T, d, E)), dtype=torch.uint8,
                      device="cuda")
    bufs = dict(counts=torch.empty(E, dtype=torch.int32, device="cuda"),
                offsets=torch.empty(E + 1, dtype=torch.int32, device="cuda"),
                src_token=torch.empty(T * 8, dtype=torch.int32, device="cuda"),
                inv_pos=torch.empty((T, 8), dtype=torch.int32, device="cuda"))
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        g.moe_route(r["x"], w_r, r["bias"], 8, idx, w, rws)
        if ev:
            ev[1].record(stream)
        g.moe_permute(idx, 0, E, None, workspace=ws, **bufs)
        if ev:
            ev[2].record(stream)

    def timed(flush):
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
        for i in range(steps):
            if flush:
                scratch.fill_(i & 0x7F)
            step(evs[i])
        torch.cuda.synchronize()
        return ([1e3 * e[0].elapsed_time(e[1]) for e in evs],
                [1e3 * e[1].elapsed_time(e[2]) for e in evs])

    warm_clock()
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    route_us, perm_us = timed(False)
    fl = timed(True) if scratch is not None else None
    rbytes = T * d * 2 + E * d * 2 + E * 4 + T * 8 * 8
    return dict(workload=ROUTER, route_us=route_us, perm_us=perm_us, flushed=fl,
                work={"moe_route": dict(bytes=rbytes, flops=2 * T * d * E),
                      "moe_permute": dict(bytes=T * 8 * 4 + T * 8 * 8 + (E + 1) * 8)})


def measure_attainable(reps=10):
    """What this GPU sustains, measured here with the library's probes: bf16
    MFMA FLOP/s with no memory traffic, and HBM read bandwidth over a 4 GiB
    buffer. Each is the best of `reps` timed launches after warm-up."""
    import ctypes
    import torch
    from gated_mlp_transformer_amd import _lib
    lib = _lib.load()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    out = torch.empty(cus * 8 * 256, dtype=torch.float32, device="cuda")
    iters = 4000
    flops = cus * 4 * iters * 16 * 32768

    def best(launch, work):
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
        for _ in range(3):
            if launch() != 0:
                raise RuntimeError("bench: probe launch failed")
        for i in range(reps):
            ev[i][0].record()
            launch()
            ev[i][1].record()
        torch.cuda.synchronize()
        return max(work / (a.elapsed_time(b) * 1e-3) for a, b in ev)

    def mfma():
        return lib.mf_probe_mfma_bf16(cus, iters, ctypes.c_void_p(out.data_ptr()), s)

    mfma_tf = best(mfma, flops) / 1e12
    buf = torch.empty(4 << 30, dtype=torch.uint8, device="cuda")
    buf.fill_(1)

    def read(wgs):
        return lambda: lib.mf_probe_hbm_read(ctypes.c_void_p(buf.data_ptr()), buf.numel(), wgs,
                                             ctypes.c_void_p(out.data_ptr()), s)

    hbm = max(best(read(cus * m), buf.numel()) for m in (1, 2, 4)) / 1e9
    half = buf.numel() // 2

    def copy(wgs):
        return lambda: lib.mf_probe_hbm_copy(ctypes.c_void_p(buf.data_ptr()),
                                             ctypes.c_void_p(buf.data_ptr() + half), half, wgs, s)

    hbm_rw = max(best(copy(cus * m), 2 * half) for m in (2, 4, 8)) / 1e9
    del buf
    torch.cuda.empty_cache()
    return dict(mfma_bf16_tflop_s=round(mfma_tf, 1), hbm_gb_s=round(hbm, 1),
                hbm_rw_gb_s=round(hbm_rw, 1), cus=cus,
                source="mf_probe_mfma_bf16 (back-to-back 32x32x16 bf16 MFMA, 4 waves per CU), "
                       "mf_probe_hbm_read (16-byte loads over 4 GiB, 1/2/4 workgroups per CU) "
                       "and mf_probe_hbm_copy (2 GiB read + 2 GiB written, 2/4/8 workgroups "
                       f"per CU), best of {reps} launches each")


# stages whose traffic is about as much written as read: their attainable
# bandwidth is the copy probe's, not the read probe's
RW_STAGES = ("rmsnorm", "moe_combine")


def full_report(work, us, flushed=None, mfma_peak=PEAK_BF16_TFLOPS, attain=None,
                mfma_attain_key="mfma_bf16_tflop_s"):
    """Per stage: mean / median / min µs of the back-to-back steps (the mean is
    what `us` of stage_report states), the median and min of the flushed reps,
    and the spec-peak and attainable-peak fractions of the median (against the
    copy probe for the read + write stages, the read probe otherwise)."""
    out = {}
    for name, w in work.items():
        if name not in us:
            continue
        st = summary(us[name])
        r = dict(us=round(st["mean"], 2), us_median=round(st["median"], 2),
                 us_min=round(st["min"], 2))
        t = st["median"] * 1e-6
        if w.get("bytes"):
            gbs = w["bytes"] / t / 1e9
            r.update(gb_s=round(gbs, 1), hbm_frac=round(gbs / PEAK_HBM_GBS, 4))
            if attain:
                key = "hbm_rw_gb_s" if name in RW_STAGES and "hbm_rw_gb_s" in attain else "hbm_gb_s"
                r["hbm_frac_attainable"] = round(gbs / attain[key], 4)
        if w.get("flops"):
            tf = w["flops"] / t / 1e12
            r.update(tflop_s=round(tf, 1), mfma_frac=round(tf / mfma_peak, 4))
            if attain and mfma_attain_key in attain:
                r["mfma_frac_attainable"] = round(tf / attain[mfma_attain_key], 4)
        if flushed is not None and name in flushed:
            fs = summary(flushed[name])
            r.update(flushed_us_median=round(fs["median"], 2), flushed_us_min=round(fs["min"], 2))
        out[name] = r
    return out


# ---------------------------------------------------------------- CPU oracle


def host_cores():
    """Cores this process may run on, the machine's count and the BLAS pool."""
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()
                    if i.get("user_api") == "blas"] or [0])
    except Exception:  # threadpoolctl missing
        blas = None
    return dict(cores=cores, cpu_count=os.cpu_count(), blas_threads=blas)


def _bits(t):
    import numpy as np
    import torch
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def cpu_baseline(res):
    """The fp64 oracle on the same prefill step, on this host's cores (the
    headline baseline): whole steps, repeated until about 10 s have elapsed."""
    import numpy as np
    import oracle
    spec, inp = res["spec"], res["inp"]
    hc = host_cores()
    host = {k: _bits(inp[k]) for k in ("x", "gamma", "w_r", "w_gate", "w_up", "w_down")}
    bias = inp["bias"].cpu().numpy().astype(np.float64)
    T = spec["T"]
    log(f"[bench] cpu oracle: {PREFILL}, {hc}")
    dec = oracle.bf16_bits_to_f64
    weights = lambda e: (dec(host["w_gate"][e]).T, dec(host["w_up"][e]).T,  # noqa: E731
                         dec(host["w_down"][e]).T)
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.moe_ffn(dec(host["x"]), dec(host["gamma"]), dec(host["w_r"]), bias, weights,
                       spec["e_begin"], spec["e_count"])
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= 10.0 or reps >= 50:
            break
    return dict(value=round(reps * T / dt, 1), unit="tokens/s", cores=hc["cores"],
                cpu_count=hc["cpu_count"], blas_threads=hc["blas_threads"],
                kind="oracle", seconds=round(dt, 2), steps=reps,
                sample=f"{reps} full {PREFILL} steps ({T} tokens each), fp64 numpy, incl. bf16 "
                       f"decoding of inputs and all 32 local experts' weights")


def cpu_baselines_other(dec_res=None):
    """The oracle on the other workloads, same host, same run: 3 reps of the
    dense fp32, dense bf16 and router workloads; one rep of the whole decode
    workload, streaming each routed expert's dequantisation."""
    import numpy as np
    import torch
    import oracle
    import synth
    from synth.workloads import make_dense, make_router
    out = {}

    def timed(fn, reps):
        ts = []
        for _ in range(reps):
            t0 = time.perf_counter()
            fn()
            ts.append(time.perf_counter() - t0)
        return min(ts), sum(ts) / len(ts)

    dec = oracle.bf16_bits_to_f64
    # dense fp32, 16 x 64, four shards and their sum
    D = make_dense(16, 64, 256, dtype=torch.float32)
    x, wg, wu, wd = (D[k].double().numpy() for k in ("x", "w_gate", "w_up", "w_down"))
    best, mean = timed(lambda: sum(oracle.tp_shard_mlp(x, wg.T, wu.T, wd.T, 4, i)
                                   for i in range(4)), 3)
    out["dense_f32_16x64_f256_p4"] = dict(us_per_rep=round(mean * 1e6, 1), reps=3,
                                          sample="the whole workload: 4 shards + sum")
    # dense bf16, 4096 x 4096, RMSNorm + one shard
    s = synth.WORKLOADS[DENSE]
    D = make_dense(s["T"], s["d"], s["f"], dtype=torch.bfloat16, norm=True)
    x, g_, wg, wu, wd = (dec(_bits(D[k])) for k in ("x", "gamma", "w_gate", "w_up", "w_down"))
    best, mean = timed(lambda: oracle.tp_shard_mlp(oracle.rmsnorm(x, g_), wg.T, wu.T, wd.T, 1, 0),
                       3)
    out[DENSE] = dict(value=round(s["T"] / mean, 1), unit="tokens/s", seconds_per_rep=round(mean, 3),
                      reps=3, sample="the whole workload (4096 tokens): RMSNorm + one shard, fp64")
    # router, 4096 tokens x 256 experts, route + permutation
    s = synth.WORKLOADS[ROUTER]
    r = make_router(s["T"], s["d"], s["E"])
    x, w_r = dec(_bits(r["x"])), dec(_bits(r["w_r"]))
    b = r["bias"].double().numpy()

    def route_perm():
        idx = oracle.route(x, w_r, b)[0]
        oracle.permute(idx, 0, s["E"])

    best, mean = timed(route_perm, 3)
    out[ROUTER] = dict(value=round(s["T"] / mean, 1), unit="tokens/s",
                       seconds_per_rep=round(mean, 3), reps=3,
                       sample="the whole workload (4096 tokens): route + index permutation, fp64")
    # decode: all 64 tokens, each routed expert's weights dequantised when used
    if dec_res is not None:
        spec, inp = dec_res["spec"], dec_res["inp"]
        n = spec["T"]
        host = {k: inp[k][:n].cpu() for k in ("x",)}
        xs = dec(_bits(host["x"]))
        gam = dec(_bits(inp["gamma"]))
        w_r = dec(_bits(inp["w_r"]))
        b = inp["bias"].cpu().double().numpy()

        def weights(e):
            def dq(key):
                q = inp[key][e].cpu().contiguous().view(torch.uint8).numpy()
                sc = inp["s_" + key[2:]][e].cpu().double().numpy()
                return oracle.dequant_block_fp8(q.T, sc.T)
            return dq("w_gate"), dq("w_up"), dq("w_down")

        t0 = time.perf_counter()
        res = oracle.moe_ffn(xs, gam, w_r, b, weights, spec["e_begin"], spec["e_count"])
        dt = time.perf_counter() - t0
        out[DECODE] = dict(value=round(n / dt, 2), unit="tokens/s", seconds=round(dt, 2), reps=1,
                           active_experts=int((res["counts"] > 0).sum()),
                           sample=f"the whole workload ({n} tokens), fp64, incl. the block-fp8 "
                                  "dequantisation of every routed expert's weights")
    return out


# ---------------------------------------------------------------------- main


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported: this build runs on one GPU only "
              "(no collectives, no sharding across GPUs); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible; the HIP path has no CPU fallback", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    import gated_mlp_transformer_amd as g
    log(f"[bench] {g.version()} on {torch.cuda.get_device_name(0)}")

    if args.only:
        if args.copy_calibration:
            src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
            dst = torch.empty_like(src)
            for _ in range(3):
                dst.copy_(src)
            torch.cuda.synchronize()
            del src, dst
            log("[bench] copy calibration: 3 x 1 GiB device-to-device copies done")
        if args.only in ("prefill", "decode", "prefill_fp8", "decode_masked", "prefill_fp8w"):
            name = {"prefill": PREFILL, "decode": DECODE, "prefill_fp8": PREFILL_FP8,
                    "decode_masked": DECODE_MASKED, "prefill_fp8w": PREFILL_FP8W}[args.only]
            res = run_moe(name, args.steps, args.warmup, graph=not args.no_graph)
            peak = PEAK_FP8_TFLOPS if res["spec"].get("act_fp8") else PEAK_BF16_TFLOPS
            print(json.dumps(dict(workload=res["spec"], ms_per_step=res["ms"],
                                  graph_ms_per_step=res["ms_graph"],
                                  stages=full_report(res["work"], res["us"], mfma_peak=peak),
                                  **res["info"]), default=str), flush=True)
        elif args.only == "dense":
            r = run_dense(args.steps, args.warmup)
            print(json.dumps(full_report(r["work"], {"rmsnorm": r["norm_us"],
                                                     "tp_shard_mlp": r["shard_us"]})), flush=True)
        else:
            r = run_router(args.steps, args.warmup)
            print(json.dumps(full_report(r["work"], {"moe_route": r["route_us"],
                                                     "moe_permute": r["perm_us"]})), flush=True)
        return

    # What this GPU sustains, measured first (it also brings the clock up
    # from idle before the timed steps).
    attain = measure_attainable()
    log(f"[bench] attainable: {attain['mfma_bf16_tflop_s']} TFLOP/s bf16 MFMA, "
        f"{attain['hbm_gb_s']} GB/s HBM read, {attain['hbm_rw_gb_s']} GB/s read + write")
    warm_desc = process_warmup()
    log("[bench] process warm-up done")
    # written before every flushed rep: larger than the 256 MB last-level cache
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")

    res = run_moe(PREFILL, args.steps, args.warmup, scratch)
    spec = res["spec"]
    T = spec["T"]
    stages = full_report(res["work"], res["us"], res["flushed"], attain=attain)
    dom = "grouped_gate_up"
    w_dom = res["work"][dom]
    t_dom = summary(res["us"][dom])["mean"] * 1e-6
    achieved = w_dom["flops"] / t_dom / 1e12
    gemm_us = [a + b for a, b in zip(res["us"][dom], res["us"]["grouped_down"])]
    gemm_flops = w_dom["flops"] + res["work"]["grouped_down"]["flops"]
    step = summary(res["us"]["step"])
    fstep = summary(res["flushed"]["step"])
    line = {
        "metric": METRIC,
        "value": round(T / (res["ms"] * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["ms"], 4),
        # before the first workload's own W warm-up steps (untimed)
        "process_warmup": warm_desc,
        # per-step times of K more steps with an event between stages (first
        # stage mark to last)
        "step_us_median": round(step["median"], 2),
        "step_us_min": round(step["min"], 2),
        # K further steps, each after an untimed 512 MB scratch write
        "flushed_step_us_median": round(fstep["median"], 2),
        "flushed_step_us_min": round(fstep["min"], 2),
        # the same step captured once as a HIP graph and replayed (checked bit for
        # bit against the eager step)
        "graph_ms_per_step": round(res["ms_graph"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": PREFILL, "tokens": T, "d": spec["d"], "f": spec["f"],
                   "experts": spec["E"], "local_experts": spec["e_count"], "top_k": 8,
                   "rmsnorm": True, "zipf_amplitude": spec["zipf"], **res["info"]},
        "roofline": {"kernel": "grouped_gate_up (bf16 MFMA grouped GEMM + SiLU*up epilogue)",
                     "bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "frac_attainable": round(achieved / attain["mfma_bf16_tflop_s"], 4),
                     # HBM bytes per launch from the committed rocprofv3 counters
                     # (null once the kernel source differs from the profiled one)
                     "traffic": measured_traffic("grouped_gate_up",
                                                 "moe_prefill_8192tok_hbm_counters.md"),
                     "traffic_unit": "bytes per launch",
                     "algorithmic_bytes": int(w_dom["bytes"]),
                     "hbm_gb_s": round(w_dom["bytes"] / t_dom / 1e9, 1)},
        "attainable": attain,
        "stages": stages,
        "grouped_gemm_mfma_frac": round(
            gemm_flops / (summary(gemm_us)["mean"] * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 4),
    }
    dec = None
    if not args.no_extra:
        ksub = max(10, args.steps // 2)
        nn = run_moe(PREFILL, ksub, args.warmup, scratch, norm=False, graph=False)
        line["prefill_no_rmsnorm"] = {
            "workload": PREFILL + " without rmsnorm (router and experts on x)",
            "tokens_per_s": round(T / (nn["ms"] * 1e-3), 1), "ms_per_step": round(nn["ms"], 4),
            "stages": full_report(nn["work"], nn["us"], nn["flushed"], attain=attain)}
        del nn
        torch.cuda.empty_cache()
        dec = run_moe(DECODE, ksub, args.warmup, scratch)
        gemm_bytes = dec["work"]["grouped_gate_up"]["bytes"] + dec["work"]["grouped_down"]["bytes"]
        dg_us = summary([a + b for a, b in zip(dec["us"]["grouped_gate_up"],
                                                dec["us"]["grouped_down"])])["mean"]
        line["decode"] = {"workload": DECODE, "tokens_per_s": round(64 / (dec["ms"] * 1e-3), 1),
                          "ms_per_step": round(dec["ms"], 4),
                          "graph_ms_per_step": round(dec["ms_graph"], 4), **dec["info"],
                          "grouped_gemm_hbm_frac": round(
                              gemm_bytes / (dg_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                          "grouped_gemm_hbm_frac_attainable": round(
                              gemm_bytes / (dg_us * 1e-6) / 1e9 / attain["hbm_gb_s"], 4),
                          "stages": full_report(dec["work"], dec["us"], dec["flushed"],
                                                attain=attain)}
        dec["layer"] = None  # the packed weights; the inputs stay for the oracle baseline
        torch.cuda.empty_cache()
        dm = run_moe(DECODE_MASKED, ksub, args.warmup, scratch)
        line["decode_masked"] = {
            "workload": DECODE_MASKED, "tokens_per_s": round(64 / (dm["ms"] * 1e-3), 1),
            "ms_per_step": round(dm["ms"], 4), "graph_ms_per_step": round(dm["ms_graph"], 4),
            "vs_contiguous_step": round(line["decode"]["ms_per_step"] / dm["ms"], 4),
            "stages": full_report(dm["work"], dm["us"], dm["flushed"], attain=attain)}
        del dm
        torch.cuda.empty_cache()
        p8 = run_moe(PREFILL_FP8, ksub, args.warmup, scratch)
        gw = p8["work"]["grouped_gate_up"]["flops"] + p8["work"]["grouped_down"]["flops"]
        gus = summary([a + b for a, b in zip(p8["us"]["grouped_gate_up"],
                                             p8["us"]["grouped_down"])])["mean"]
        line["prefill_fp8_activations"] = {
            "workload": PREFILL_FP8, "tokens_per_s": round(T / (p8["ms"] * 1e-3), 1),
            "ms_per_step": round(p8["ms"], 4), "graph_ms_per_step": round(p8["ms_graph"], 4),
            "vs_bf16_step": round(res["ms"] / p8["ms"], 4),
            **p8["info"],
            # the GEMM stages include the activation quantisation that feeds them
            "grouped_gemm_fp8_mfma_frac": round(gw / (gus * 1e-6) / 1e12 / PEAK_FP8_TFLOPS, 4),
            "stages": full_report(p8["work"], p8["us"], p8["flushed"], PEAK_FP8_TFLOPS,
                                  attain=attain)}
        del p8
        torch.cuda.empty_cache()
        pw = run_moe(PREFILL_FP8W, ksub, args.warmup, scratch)
        line["prefill_fp8_weights"] = {
            "workload": PREFILL_FP8W + " (block-fp8 weights, bf16 activations)",
            "tokens_per_s": round(T / (pw["ms"] * 1e-3), 1), "ms_per_step": round(pw["ms"], 4),
            "graph_ms_per_step": round(pw["ms_graph"], 4), **pw["info"],
            "stages": full_report(pw["work"], pw["us"], pw["flushed"], attain=attain)}
        del pw
        torch.cuda.empty_cache()
        dn = run_dense(ksub, args.warmup, scratch)
        line["dense_shard"] = {
            "workload": DENSE,
            "stages": full_report(dn["work"], {"rmsnorm": dn["norm_us"],
                                               "tp_shard_mlp": dn["shard_us"]},
                                  {"rmsnorm": dn["flushed"][0], "tp_shard_mlp": dn["flushed"][1]},
                                  attain=attain)}
        rt = run_router(ksub, args.warmup, scratch)
        line["router_only"] = {
            "workload": ROUTER,
            "stages": full_report(rt["work"], {"moe_route": rt["route_us"],
                                               "moe_permute": rt["perm_us"]},
                                  {"moe_route": rt["flushed"][0], "moe_permute": rt["flushed"][1]},
                                  attain=attain)}
        line["dense_f32"] = run_dense_f32(ksub, args.warmup)
    del scratch
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(res)
        line["cpu_baselines"] = cpu_baselines_other(dec)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
