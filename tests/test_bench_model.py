"""Host-side arithmetic of bench.py: the algorithmic work model behind every
roofline fraction it prints, and the rule that reports measured HBM traffic
only while the profiled kernel source is unchanged."""

import hashlib
import importlib.util
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_prefill_gate_up_work(bench):
    # 8192 tokens, d 4096, f 2048, 32 of 256 experts local, all active, S = 10417 slots
    T, d, f, E, k, S, active, ec = 8192, 4096, 2048, 256, 8, 10417, 32, 32
    w = bench.moe_work(T, d, f, E, k, S, active, ec, welt=2)
    gu = w["grouped_gate_up"]
    weights = active * 2 * (f * d) * 2          # W_gate and W_up of every active expert, bf16
    rows_in = S * d * 2                          # the gathered rows of V
    rows_out = S * f * 2                         # H
    index = S * 4                                # one int32 row index per slot
    assert gu["bytes"] == weights + rows_in + rows_out + index == 1201787588
    assert gu["flops"] == 2 * S * d * (2 * f)
    dn = w["grouped_down"]
    assert dn["bytes"] == active * d * f * 2 + S * f * 2 + S * d * 2
    assert dn["flops"] == 2 * S * f * d
    assert w["rmsnorm"]["bytes"] == 2 * T * d * 2 + d * 2
    assert w["moe_route"]["flops"] == 2 * T * d * E


def test_fp8_weight_work_counts_scales(bench):
    T, d, f, E, k, S, active, ec = 64, 4096, 2048, 256, 8, 512, 215, 256
    w = bench.moe_work(T, d, f, E, k, S, active, ec, welt=1)
    scales = 4 * (f // 128) * (d // 128)        # one fp32 per 128 x 128 block per matrix
    assert w["grouped_gate_up"]["bytes"] == (active * (2 * f * d + 2 * scales) + S * d * 2
                                             + S * f * 2 + S * 4)
    assert w["grouped_down"]["bytes"] == active * (d * f + scales) + S * f * 2 + S * d * 2


def test_stage_report_fractions(bench):
    # 4 TB and 1.25 PFLOP in one second: half of the 8 TB/s and of the 2.5 PFLOP/s bf16 peaks
    work = {"a": dict(bytes=4_000_000_000_000, flops=1_250_000_000_000_000), "b": dict(bytes=8_000_000)}
    r = bench.stage_report(work, {"a": 1e6, "b": 1.0})
    assert r["a"]["gb_s"] == 4000.0 and r["a"]["hbm_frac"] == 0.5
    assert r["a"]["tflop_s"] == 1250.0 and r["a"]["mfma_frac"] == 0.5
    assert r["b"]["gb_s"] == 8000.0 and r["b"]["hbm_frac"] == 1.0 and "mfma_frac" not in r["b"]


def test_measured_traffic_follows_the_source_hash(bench, tmp_path, monkeypatch):
    src = tmp_path / "kern.hip"
    src.write_bytes(b"kernel source v1\n")
    digest = hashlib.sha256(src.read_bytes()).hexdigest()
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "p.md").write_text(
        "header\n"
        f"bench-traffic: kernel=other source=kern.hip sha256={digest} bytes_per_launch=7\n"
        f"bench-traffic: kernel=k source=kern.hip sha256={digest} bytes_per_launch=12345\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("k", "p.md") == 12345
    assert bench.measured_traffic("missing", "p.md") is None
    assert bench.measured_traffic("k", "absent.md") is None
    src.write_bytes(b"kernel source v2\n")       # the kernel changed since the counters
    assert bench.measured_traffic("k", "p.md") is None
    src.unlink()
    assert bench.measured_traffic("k", "p.md") is None


def _run_bench(*args, env_extra=None):
    import subprocess
    import sys
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, timeout=300, env=env)


def test_bench_refuses_several_gpus():
    r = _run_bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_bench_has_no_cpu_fallback():
    # with no GPU visible the benchmark stops instead of timing anything on the host
    r = _run_bench("--steps", "1", "--warmup", "0", env_extra={"HIP_VISIBLE_DEVICES": "-1",
                                                               "CUDA_VISIBLE_DEVICES": "-1"})
    assert r.returncode == 1
    assert "no GPU visible" in r.stderr and r.stdout == ""
