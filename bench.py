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
                                       "decode_masked"],
                    default=None,
                    help="run one workload only (for profiling); prints its stage times")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="with --only: first copy a 1 GiB device buffer 3 times (a kernel of "
                         "known traffic to scale HBM byte counters against)")
    return ap.parse_args()


# ----------------------------------------------------------------- work model


def moe_work(T, d, f, E, k, S, active, ec, welt, act_fp8=False):
    """Algorithmic bytes / flops per stage of one MoE FFN step (each tensor once).

    With fp8 activations the gate/up stage also quantises V (read 2d, write
    d + d/32 bytes per token) and reads the fp8 rows, and the down stage
    quantises the live rows of H and reads them as fp8."""
    sc = 0 if welt == 2 else 4 * (f // 128) * (d // 128)  # fp8 scales per matrix
    if act_fp8:
        w = moe_work(T, d, f, E, k, S, active, ec, welt)
        w["grouped_gate_up"]["bytes"] = (active * (2 * f * d + 2 * sc) + T * d * 2 + T * d
                                         + T * d // 32 + S * d + S * d // 32 + S * f * 2 + S * 4)
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


def time_layer(layer, x, steps, warmup):
    """Warm up, then time exactly `steps` forwards with per-stage events."""
    import torch
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        layer(x)
    torch.cuda.synchronize()
    marks = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for i in range(steps):
        layer(x, marks=marks[i])
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = t_start.elapsed_time(t_end) / steps
    us = {}
    for s, name in enumerate(layer.STAGES):
        us[name] = 1e3 * sum(m[s].elapsed_time(m[s + 1]) for m in marks) / steps
    return ms, us, wall


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


def build_layer(spec, device, seed=0):
    import gated_mlp_transformer_amd as g
    from synth.workloads import make_moe
    inp = make_moe(spec["T"], spec["d"], spec["f"], spec["E"], spec["e_begin"], spec["e_count"],
                   wdtype=spec["wdtype"], zipf=spec["zipf"], seed=seed, device=device)
    layer = g.MoEFFNLayer(T=spec["T"], d=spec["d"], f=spec["f"], w_r=inp["w_r"],
                          bias=inp["bias"], gamma=inp["gamma"], w_gate=inp["w_gate"],
                          w_up=inp["w_up"], w_down=inp["w_down"], e_begin=spec["e_begin"],
                          s_gate=inp.get("s_gate"), s_up=inp.get("s_up"),
                          s_down=inp.get("s_down"), act_fp8=spec.get("act_fp8", False),
                          layout=spec.get("layout", "contiguous"))
    return layer, inp


def run_moe(name, steps, warmup):
    import torch
    import synth
    spec = synth.WORKLOADS[name]
    log(f"[bench] {name}: building inputs")
    layer, inp = build_layer(spec, "cuda")
    ms, us, wall = time_layer(layer, inp["x"], steps, warmup)
    ms_graph = time_layer_graph(layer, inp["x"], steps, warmup)
    S = int(layer.counts.sum().item())  # both layouts (offsets are unused when masked)
    active = int((layer.counts > 0).sum().item())
    counts = layer.counts.cpu()
    welt = 2 if spec["wdtype"] == "bf16" else 1
    work = moe_work(spec["T"], spec["d"], spec["f"], spec["E"], 8, S, active, spec["e_count"],
                    welt, act_fp8=spec.get("act_fp8", False))
    log(f"[bench] {name}: {ms * 1e3:.1f} us/step, {ms_graph * 1e3:.1f} us as a graph, "
        f"S={S}, active experts {active}")
    info = dict(slots=S, active_experts=active,
                count_min=int(counts.min()), count_max=int(counts.max()),
                count_mean=round(float(counts.float().mean()), 1))
    return dict(spec=spec, layer=layer, inp=inp, ms=ms, ms_graph=ms_graph, us=us, wall=wall,
                work=work, info=info)


def run_dense(steps, warmup):
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

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    norm_us = 1e3 * sum(e[0].elapsed_time(e[1]) for e in evs) / steps
    shard_us = 1e3 * sum(e[1].elapsed_time(e[2]) for e in evs) / steps
    flops = 6 * T * d * f
    return dict(workload=DENSE, rmsnorm_us=round(norm_us, 2),
                rmsnorm_hbm_frac=round((4 * T * d + 2 * d) / (norm_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                tp_shard_us=round(shard_us, 2),
                tp_shard_tflop_s=round(flops / (shard_us * 1e-6) / 1e12, 1),
                tp_shard_mfma_frac=round(flops / (shard_us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 4))


def run_router(steps, warmup):
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
    rws = torch.empty(g.moe_route_workspace_size(T, d, E), dtype=torch.uint8, device="cuda")
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

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    route_us = 1e3 * sum(e[0].elapsed_time(e[1]) for e in evs) / steps
    perm_us = 1e3 * sum(e[1].elapsed_time(e[2]) for e in evs) / steps
    rbytes = T * d * 2 + E * d * 2 + E * 4 + T * 8 * 8
    return dict(workload=ROUTER, route_us=round(route_us, 2),
                route_hbm_frac=round(rbytes / (route_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                route_tflop_s=round(2 * T * d * E / (route_us * 1e-6) / 1e12, 1),
                permute_index_us=round(perm_us, 2))


# ---------------------------------------------------------------- CPU oracle


def cpu_baseline(res):
    """The fp64 oracle on the same prefill step, on this host's cores."""
    import numpy as np
    import torch
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"] or [1])
    except Exception:  # threadpoolctl missing: report what the process may use
        threads = len(os.sched_getaffinity(0))
    spec, inp = res["spec"], res["inp"]

    def bits(t):
        return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)

    host = {k: bits(inp[k]) for k in ("x", "gamma", "w_r", "w_gate", "w_up", "w_down")}
    bias = inp["bias"].cpu().numpy().astype(np.float64)
    T = spec["T"]
    log(f"[bench] cpu oracle: {T} tokens on {threads} BLAS threads")
    dec = oracle.bf16_bits_to_f64
    weights = lambda e: (dec(host["w_gate"][e]).T, dec(host["w_up"][e]).T,  # noqa: E731
                         dec(host["w_down"][e]).T)
    # whole steps, repeated until about 10 s of CPU work have been timed
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.moe_ffn(dec(host["x"]), dec(host["gamma"]), dec(host["w_r"]), bias, weights,
                       spec["e_begin"], spec["e_count"])
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= 10.0 or reps >= 50:
            break
    return dict(value=round(reps * T / dt, 1), unit="tokens/s", cores=int(threads),
                kind="oracle", seconds=round(dt, 2), steps=reps,
                sample=f"{reps} full {PREFILL} steps ({T} tokens each), fp64 numpy, incl. bf16 "
                       f"decoding of inputs and all 32 local experts' weights")


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
        if args.only in ("prefill", "decode", "prefill_fp8", "decode_masked"):
            name = {"prefill": PREFILL, "decode": DECODE, "prefill_fp8": PREFILL_FP8,
                    "decode_masked": DECODE_MASKED}[args.only]
            res = run_moe(name, args.steps, args.warmup)
            peak = PEAK_FP8_TFLOPS if res["spec"].get("act_fp8") else PEAK_BF16_TFLOPS
            print(json.dumps(dict(workload=res["spec"], ms_per_step=res["ms"],
                                  graph_ms_per_step=res["ms_graph"],
                                  stages=stage_report(res["work"], res["us"], peak), **res["info"]),
                             default=str), flush=True)
        elif args.only == "dense":
            print(json.dumps(run_dense(args.steps, args.warmup)), flush=True)
        else:
            print(json.dumps(run_router(args.steps, args.warmup)), flush=True)
        return

    res = run_moe(PREFILL, args.steps, args.warmup)
    spec = res["spec"]
    T = spec["T"]
    stages = stage_report(res["work"], res["us"])
    dom = "grouped_gate_up"
    w_dom = res["work"][dom]
    t_dom = res["us"][dom] * 1e-6
    achieved = w_dom["flops"] / t_dom / 1e12
    line = {
        "metric": METRIC,
        "value": round(T / (res["ms"] * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["ms"], 4),
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
                     # HBM bytes per launch from the committed rocprofv3 counters
                     # (null once the kernel source differs from the profiled one)
                     "traffic": measured_traffic("grouped_gate_up",
                                                 "moe_prefill_8192tok_hbm_counters.md"),
                     "traffic_unit": "bytes per launch",
                     "algorithmic_bytes": int(w_dom["bytes"]),
                     "hbm_gb_s": round(w_dom["bytes"] / t_dom / 1e9, 1)},
        "stages": stages,
        "grouped_gemm_mfma_frac": round(
            (w_dom["flops"] + res["work"]["grouped_down"]["flops"])
            / ((res["us"][dom] + res["us"]["grouped_down"]) * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 4),
    }
    if not args.no_extra:
        dec = run_moe(DECODE, max(10, args.steps // 2), args.warmup)
        dstage = stage_report(dec["work"], dec["us"])
        gemm_bytes = dec["work"]["grouped_gate_up"]["bytes"] + dec["work"]["grouped_down"]["bytes"]
        gemm_us = dec["us"]["grouped_gate_up"] + dec["us"]["grouped_down"]
        line["decode"] = {"workload": DECODE, "tokens_per_s": round(64 / (dec["ms"] * 1e-3), 1),
                          "ms_per_step": round(dec["ms"], 4),
                          "graph_ms_per_step": round(dec["ms_graph"], 4), **dec["info"],
                          "grouped_gemm_hbm_frac": round(
                              gemm_bytes / (gemm_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                          "stages": dstage}
        del dec
        torch.cuda.empty_cache()
        dm = run_moe(DECODE_MASKED, max(10, args.steps // 2), args.warmup)
        line["decode_masked"] = {
            "workload": DECODE_MASKED, "tokens_per_s": round(64 / (dm["ms"] * 1e-3), 1),
            "ms_per_step": round(dm["ms"], 4), "graph_ms_per_step": round(dm["ms_graph"], 4),
            "vs_contiguous_step": round(line["decode"]["ms_per_step"] / dm["ms"], 4),
            "stages": stage_report(dm["work"], dm["us"])}
        del dm
        torch.cuda.empty_cache()
        p8 = run_moe(PREFILL_FP8, max(10, args.steps // 2), args.warmup)
        gw = p8["work"]["grouped_gate_up"]["flops"] + p8["work"]["grouped_down"]["flops"]
        gus = p8["us"]["grouped_gate_up"] + p8["us"]["grouped_down"]
        line["prefill_fp8_activations"] = {
            "workload": PREFILL_FP8, "tokens_per_s": round(T / (p8["ms"] * 1e-3), 1),
            "ms_per_step": round(p8["ms"], 4), "graph_ms_per_step": round(p8["ms_graph"], 4),
            **p8["info"],
            # the GEMM stages include the activation quantisation that feeds them
            "grouped_gemm_fp8_mfma_frac": round(gw / (gus * 1e-6) / 1e12 / PEAK_FP8_TFLOPS, 4),
            "stages": stage_report(p8["work"], p8["us"], PEAK_FP8_TFLOPS)}
        del p8
        torch.cuda.empty_cache()
        line["dense_shard"] = run_dense(max(10, args.steps // 2), args.warmup)
        line["router_only"] = run_router(max(10, args.steps // 2), args.warmup)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(res)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
