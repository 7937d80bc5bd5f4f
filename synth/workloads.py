"""The synthetic workloads: shapes, distributions and seeds.

Five named workloads mirror the configurations the hot path is measured on;
the builder functions also take smaller shapes for parity cases.

  dense_f32_16x64_f256_p4          X 16x64 ~N(0,1) f32; W_gate, W_up 64x256 and
                                   W_down 256x64 ~N(0,0.02) f32; 4 TP shards
  norm_tp_shard_bf16_4096          RMSNorm (gamma ~1+N(0,0.1)) + one TP shard,
                                   X 4096x4096 ~N(0,1) bf16; W_gate, W_up
                                   4096x2048, W_down 2048x4096 ~N(0,0.02) bf16
  router_4096tok_E256              X 4096x4096 ~N(0,1) bf16, W_r 256x4096
                                   ~N(0,0.02) bf16, b ~N(0,0.01) f32
  moe_prefill_8192tok_32exp_bf16   8192 tokens, d 4096, f 2048, E 256 with the
                                   32 local experts [0,32), bias skewed by
                                   A*(e+1)^-1.1, bf16 experts ~N(0,0.02)
  moe_prefill_8192tok_32exp_fp8act the prefill shape and routing with the experts
                                   drawn ~N(0,0.02) f32 then block-fp8 quantised,
                                   run with fp8 activations (per-token 1x128)
  moe_decode_64tok_256exp_fp8_masked  the decode workload in the masked layout
                                   (fixed blocks of 64 rows per expert)
  moe_decode_64tok_256exp_fp8      64 tokens, all 256 experts local, experts
                                   drawn ~N(0,0.02) f32 then block-fp8 quantised
"""

from __future__ import annotations

import torch

from . import normal, quantize_block_fp8, zipf_bias_skew

# Amplitude of the Zipf(1.1) bias skew of the prefill workload, chosen so the
# 32 local experts' token counts span roughly 0.5x to 3x their mean.
ZIPF_AMPLITUDE = 0.09

WORKLOADS = {
    "dense_f32_16x64_f256_p4": dict(kind="dense", T=16, d=64, f=256, p=4,
                                    dtype=torch.float32, norm=False),
    "norm_tp_shard_bf16_4096": dict(kind="dense", T=4096, d=4096, f=2048, p=1,
                                    dtype=torch.bfloat16, norm=True),
    "router_4096tok_E256": dict(kind="router", T=4096, d=4096, E=256),
    "moe_prefill_8192tok_32exp_bf16": dict(kind="moe", T=8192, d=4096, f=2048,
                                           E=256, e_begin=0, e_count=32,
                                           wdtype="bf16", zipf=ZIPF_AMPLITUDE),
    "moe_prefill_8192tok_32exp_fp8act": dict(kind="moe", T=8192, d=4096, f=2048,
                                             E=256, e_begin=0, e_count=32, wdtype="fp8",
                                             act_fp8=True, zipf=ZIPF_AMPLITUDE),
    "moe_prefill_8192tok_32exp_fp8w": dict(kind="moe", T=8192, d=4096, f=2048,
                                           E=256, e_begin=0, e_count=32, wdtype="fp8",
                                           zipf=ZIPF_AMPLITUDE),
    "moe_decode_64tok_256exp_fp8": dict(kind="moe", T=64, d=4096, f=2048, E=256,
                                        e_begin=0, e_count=256, wdtype="fp8",
                                        zipf=0.0),
    "moe_decode_64tok_256exp_fp8_masked": dict(kind="moe", T=64, d=4096, f=2048, E=256,
                                               e_begin=0, e_count=256, wdtype="fp8",
                                               zipf=0.0, layout="masked"),
}


def make_dense(T: int, d: int, f: int, *, dtype=torch.bfloat16, norm: bool = False,
               seed: int = 0, device="cpu", w_std: float = 0.02) -> dict:
    """Dense gated-MLP inputs: x [T,d], gamma [d] (if norm), weights [out,in]."""
    out = dict(
        x=normal((T, d), name="dense.x", seed=seed, dtype=dtype, device=device),
        w_gate=normal((f, d), name="dense.w_gate", seed=seed, std=w_std, dtype=dtype, device=device),
        w_up=normal((f, d), name="dense.w_up", seed=seed, std=w_std, dtype=dtype, device=device),
        w_down=normal((d, f), name="dense.w_down", seed=seed, std=w_std, dtype=dtype, device=device),
    )
    if norm:
        out["gamma"] = normal((d,), name="gamma", seed=seed, std=0.1, mean=1.0,
                              dtype=dtype, device=device)
    return out


def shard_weights(w_gate: torch.Tensor, w_up: torch.Tensor, w_down: torch.Tensor,
                  p: int, i: int):
    """Rank i's contiguous copies of its TP shard ([out,in] storage).

    W_gate and W_up are split by output feature (rows of the [f, d] storage),
    W_down by input feature (columns of the [d, f] storage). This is weight
    placement done once per rank, not part of the timed path.
    """
    f = w_gate.shape[0]
    assert f % p == 0
    fs = f // p
    sl = slice(i * fs, (i + 1) * fs)
    return (w_gate[sl].contiguous(), w_up[sl].contiguous(), w_down[:, sl].contiguous())


def make_router(T: int, d: int, E: int, *, seed: int = 0, device="cpu",
                zipf: float = 0.0) -> dict:
    """Router inputs: x [T,d] bf16 ~N(0,1), w_r [E,d] bf16 ~N(0,0.02), bias [E] f32."""
    bias = normal((E,), name="router.bias", seed=seed, std=0.01, dtype=torch.float32,
                  device=device)
    if zipf:
        bias = bias + zipf_bias_skew(E, zipf, device=device)
    return dict(
        x=normal((T, d), name="router.x", seed=seed, dtype=torch.bfloat16, device=device),
        w_r=normal((E, d), name="router.w_r", seed=seed, std=0.02, dtype=torch.bfloat16,
                   device=device),
        bias=bias.contiguous(),
    )


def make_expert(e: int, d: int, f: int, *, wdtype: str = "bf16", seed: int = 0,
                device="cpu", w_std: float = 0.02) -> dict:
    """Expert e's weights in [out,in] storage (bf16, or fp8 q + block scales)."""
    if wdtype == "bf16":
        return dict(
            w_gate=normal((f, d), name="expert.w_gate", sub=e, seed=seed, std=w_std, device=device),
            w_up=normal((f, d), name="expert.w_up", sub=e, seed=seed, std=w_std, device=device),
            w_down=normal((d, f), name="expert.w_down", sub=e, seed=seed, std=w_std, device=device),
        )
    assert wdtype == "fp8"
    out = {}
    for key, shape in (("w_gate", (f, d)), ("w_up", (f, d)), ("w_down", (d, f))):
        w = normal(shape, name="expert." + key, sub=e, seed=seed, std=w_std,
                   dtype=torch.float32, device=device)
        q, s = quantize_block_fp8(w)
        out[key] = q
        out["s_" + key[2:]] = s
    return out


def make_moe(T: int, d: int, f: int, E: int, e_begin: int, e_count: int, *,
             wdtype: str = "bf16", zipf: float = 0.0, seed: int = 0, device="cpu",
             norm: bool = True) -> dict:
    """Full MoE-FFN inputs for one rank holding experts [e_begin, e_begin+e_count)."""
    r = make_router(T, d, E, seed=seed, device=device, zipf=zipf)
    out = dict(x=normal((T, d), name="moe.x", seed=seed, device=device),
               w_r=r["w_r"], bias=r["bias"])
    if norm:
        out["gamma"] = normal((d,), name="gamma", seed=seed, std=0.1, mean=1.0,
                              device=device)
    experts = [make_expert(e_begin + e, d, f, wdtype=wdtype, seed=seed, device=device)
               for e in range(e_count)]
    for key in experts[0]:
        out[key] = torch.stack([ex[key] for ex in experts]).contiguous()
    return out
