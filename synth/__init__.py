"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only DRAWS inputs. It holds none of the FFN's arithmetic: it
produces activations, norm gains, router weights and biases, and expert weights
(bf16, or fp8 E4M3FN with per-128x128-block float32 scales) with the shapes and
distributions of the workloads, and nothing else. Both sides of a parity check
receive the very same tensors from here; neither the oracle nor the GPU library
imports this module.

Every tensor is drawn from its own torch generator, seeded from
``(seed, tensor name, sub-stream)``, so a tensor does not depend on which
other tensors were drawn before it and large expert sets can be drawn one
expert at a time. Values are drawn as float32 standard normals, scaled and
shifted, then rounded to nearest-even into the storage dtype by torch's cast.
Drawing on ``cuda`` and on ``cpu`` gives different (equally distributed)
streams; a parity check always hands the oracle a host copy of the exact
tensor the GPU received.

Storage layout (row-major, contiguous):
  x         [T, d]            activations
  gamma     [d]               RMSNorm gain
  w_r       [E, d]            router weight (z = x w_r^T)
  bias      [E]  float32      router bias
  w_gate    [E_loc, f, d]     gate projection, stored [out, in]
  w_up      [E_loc, f, d]     up projection,   stored [out, in]
  w_down    [E_loc, d, f]     down projection, stored [out, in]
  s_gate/s_up [E_loc, f/128, d/128], s_down [E_loc, d/128, f/128]  fp8 scales
"""

from __future__ import annotations

import zlib

import torch

FP8_MAX = 448.0  # largest finite E4M3FN value
FP8_BLOCK = 128


def _stream_seed(seed: int, name: str, sub: int) -> int:
    h = zlib.crc32(f"{name}#{sub}".encode())
    return (seed * 0x9E3779B97F4A7C15 + h * 0xBF58476D1CE4E5B9 + sub) % (2**63 - 1)


def normal(shape, *, name: str, seed: int = 0, sub: int = 0, std: float = 1.0,
           mean: float = 0.0, dtype=torch.bfloat16, device="cpu") -> torch.Tensor:
    """N(mean, std^2) draws of ``shape`` from the stream (seed, name, sub)."""
    g = torch.Generator(device=device)
    g.manual_seed(_stream_seed(seed, name, sub))
    t = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    if mean != 0.0:
        t.add_(mean)
    return t.to(dtype)


def integers(shape, low: int, high: int, *, name: str, seed: int = 0, sub: int = 0,
             device="cpu") -> torch.Tensor:
    """Uniform integers in [low, high) (int64) from the stream (seed, name, sub)."""
    g = torch.Generator(device=device)
    g.manual_seed(_stream_seed(seed, name, sub))
    return torch.randint(low, high, tuple(shape), generator=g, device=device)


def quantize_block_fp8(w: torch.Tensor, block: int = FP8_BLOCK):
    """Quantise a float weight [..., N, K] to E4M3FN with one scale per block.

    One float32 scale per ``block x block`` tile of the last two dims:
    ``scale = amax / 448`` (1 where the tile is all zero), ``q = RNE(w / scale)``
    clamped to +-448. Returns ``(q float8_e4m3fn, scale float32 [..., N/b, K/b])``.
    This is input preparation (weights are quantised once, offline); both the
    GPU library and the oracle receive the same (q, scale).
    """
    *lead, N, K = w.shape
    assert N % block == 0 and K % block == 0, (N, K)
    wf = w.float().reshape(*lead, N // block, block, K // block, block)
    amax = wf.abs().amax(dim=(-3, -1))
    scale = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax))
    q = (wf / scale.unsqueeze(-1).unsqueeze(-3)).clamp_(-FP8_MAX, FP8_MAX)
    q = q.reshape(*lead, N, K).to(torch.float8_e4m3fn)
    return q, scale.to(torch.float32).contiguous()


def zipf_bias_skew(E: int, amplitude: float, exponent: float = 1.1,
                   device="cpu") -> torch.Tensor:
    """Additive router-bias skew ``A * (e + 1)^-exponent`` for expert e.

    Expert rank is the expert id, so low ids (the local range [0, 32) of the
    skewed prefill workload) receive uneven, larger token counts.
    """
    e = torch.arange(E, device=device, dtype=torch.float64)
    return (amplitude * (e + 1.0) ** (-exponent)).to(torch.float32)


from .workloads import (  # noqa: E402,F401
    WORKLOADS,
    make_dense,
    make_router,
    make_moe,
)
