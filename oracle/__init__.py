"""CPU oracle for the MoE / SwiGLU FFN hot path (fp64 numpy).

This package is TEST INFRASTRUCTURE. Only the test suite, the smoke check and
the benchmark's CPU-baseline leg may import it. The GPU library never imports
it, links it or falls back to it, and the oracle imports nothing from the GPU
package: the two share no code.

Every function is a plain definition written out from the pages it cites, in
float64, on inputs converted exactly from their stored bit patterns (bf16 by a
bit shift, fp8 E4M3FN by the oracle's own 256-entry decode table). Nothing is
blocked, fused or reordered beyond what the definition states.

Pages cited (by title, section and equation):
  [P1] "推理计算流梳理" (huanyp.cn): Norm&Residual (Pre-Norm block equations and
       the RMSNorm equation), 张量并行和通信 (列并行 / 行并行 equations),
       实际 MLP 计算策略 (gated MLP equation), 专家并行 / MoE Router 过程 (router
       equation), EP 路径.
  [P2] "LLM推理并行优化的必备知识" (jia.baoyu2023.top): §1.1 场景一 (column split),
       §1.3 场景三, §1.4 场景四 (B column split + C row split).
  [P3] "tensor_parallelism" (zdszero.github.io): Gemm, Outer Dim and Inner Dim
       equations.
  [P4] "Megatron张量并行：MLP和Attention怎么切" (aiqz.cc): column/row-parallel
       MLP simulations.
  [P5] "「赤兔」Chitu 框架深度解读（七）：混合专家模型 (MoE) 的高效处理": token
       dispatchers, expert computation (tokens laid out contiguously by expert
       id; FP8 GEMMs for prefill), quantisation support (block fp8).

``quant`` holds the fp8-activation side of the block-fp8 prefill variant
(per-token 1x128 activation groups, READINGS R32 and R33).

Parity status: every function here is pinned by the CPU tests in
``tests/test_oracle_*.py`` (library cross-checks, closed forms, brute force,
the pages' worked example and invariants). No function is "parity unpinned".
"""

from .ffn import (  # noqa: F401
    bf16_bits_to_f64,
    e4m3fn_decode_table,
    fp8_bits_to_f64,
    dequant_block_fp8,
    rmsnorm,
    sigmoid,
    silu,
    swiglu,
    column_parallel,
    row_parallel_partial,
    tp_shard_mlp,
    route,
    route_weights,
    permute,
    dispatch_masked,
    experts,
    combine,
    moe_ffn,
)
from .quant import (  # noqa: F401
    e4m3fn_encode,
    bf16_round,
    quantize_rows,
    dequant_rows,
    swiglu_a8,
    experts_a8,
)
