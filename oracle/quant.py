"""fp8 activations for the block-fp8 prefill variant, as plain definitions.

TEST INFRASTRUCTURE ONLY (see the package docstring): imported by the tests,
the smoke check and the benchmark's CPU-baseline leg, never by the GPU path.

[P5] ("「赤兔」Chitu 框架深度解读（七）", 专家计算实现): for prefill the experts run as
FP8 GEMMs (DeepGEMM ``fp8_gemm_nt``) on tokens laid out contiguously by expert,
and quantised experts follow the block-fp8 scheme (量化支持, blockfp8). The pages
name the scheme but do not spell out the activation side; the readings used
here (also listed in the design document):

READING R32: a linear layer with block-fp8 weights quantises its bf16 input
  per token and per group of 128 consecutive input channels: the group scale
  is ``s = max(amax, 1e-4) / 448`` and the code is the E4M3FN value nearest to
  ``x / s`` (ties to even, saturating at 448). Scale and quotient are computed
  in float32 (the precision both sides take the code decision in).
READING R33: between the two linear layers of an expert the intermediate
  ``H = SiLU(X W_gate) * (X W_up)`` is held in bf16 (as in the bf16 path) and
  is quantised by R32 as the down projection's input.

Weights keep their own 128x128 block scales (READING R21, ``dequant_block_fp8``).
Every product of dequantised values below is exact float64 arithmetic.
"""

from __future__ import annotations

import numpy as np

from .ffn import e4m3fn_decode_table, silu

_TABLE = e4m3fn_decode_table()
# the 127 finite non-negative codes 0x00 .. 0x7E, in increasing value
_POS_CODES = np.arange(0x7F, dtype=np.int64)
_POS_VALS = _TABLE[:0x7F]
AMAX_FLOOR = np.float32(1e-4)
E4M3_MAX = np.float32(448.0)


def e4m3fn_encode(v) -> np.ndarray:
    """Nearest E4M3FN code of each value (ties to the even code, i.e. an even
    last mantissa bit), saturating to +-448; the sign is kept, so a negative
    value that rounds to zero gives the code 0x80.
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.minimum(np.abs(v), 448.0)
    hi = np.clip(np.searchsorted(_POS_VALS, a, side="left"), 0, 0x7E)
    lo = np.clip(hi - 1, 0, 0x7E)
    d_hi = np.abs(_POS_VALS[hi] - a)
    d_lo = np.abs(a - _POS_VALS[lo])
    take_lo = (d_lo < d_hi) | ((d_lo == d_hi) & (_POS_CODES[lo] % 2 == 0))
    mag = np.where(take_lo, _POS_CODES[lo], _POS_CODES[hi])
    sign = np.signbit(v)
    return (mag | np.where(sign, 0x80, 0)).astype(np.uint8)


def bf16_round(x) -> np.ndarray:
    """Round each value to the nearest bf16 value (8 significant bits, ties to
    even). Finite inputs well inside the bf16 range."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)  # x = m * 2^e, 0.5 <= |m| < 1
    return np.ldexp(np.rint(m * 256.0), e - 8)


def quantize_rows(x, group: int = 128):
    """READING R32 on the rows of ``x`` ([rows, K], values exact in float32):
    returns ``(codes uint8 [rows, K], scales float64 [rows, K/group])``.

    Per group: ``amax`` (exact), ``s = fl32(max(amax, 1e-4) / 448)``, then the
    code of ``fl32(x / s)``.
    """
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    rows, K = x32.shape
    assert K % group == 0
    g = x32.reshape(rows, K // group, group)
    amax = np.max(np.abs(g), axis=2)
    s = (np.maximum(amax, AMAX_FLOOR) / E4M3_MAX).astype(np.float32)
    v = (g / s[:, :, None]).astype(np.float32)
    codes = e4m3fn_encode(v.astype(np.float64)).reshape(rows, K)
    return codes, s.astype(np.float64)


def dequant_rows(codes, scales, group: int = 128) -> np.ndarray:
    """``x[r, k] = value(codes[r, k]) * scales[r, k // group]``, exact."""
    q = _TABLE[np.asarray(codes, dtype=np.uint8)]
    s = np.asarray(scales, dtype=np.float64)
    return q * np.repeat(s, group, axis=1)


def swiglu_a8(x, w_gate, w_up, w_down):
    """One expert's gated MLP with fp8 activations (READINGS R32, R33).

    ``x`` [m, d] (bf16 values); weights dequantised float64 in the pages'
    orientation (``[d, f]``, ``[d, f]``, ``[f, d]``). Returns ``(y, h)`` with
    ``h`` the bf16-held intermediate.
    """
    xq, xs = quantize_rows(x)
    xd = dequant_rows(xq, xs)
    h = bf16_round(silu(xd @ np.asarray(w_gate)) * (xd @ np.asarray(w_up)))
    hq, hs = quantize_rows(h)
    return dequant_rows(hq, hs) @ np.asarray(w_down), h


def experts_a8(x_perm, offsets, weights):
    """``experts`` ([P1] EP 路径, grouped) with every expert run by ``swiglu_a8``.

    Returns ``(y_perm, h)``; ``weights`` is a sequence of dequantised (Wg, Wu,
    Wd) float64 triples or a callable ``e -> triple``.
    """
    x_perm = np.asarray(x_perm, dtype=np.float64)
    offsets = np.asarray(offsets)
    get = weights if callable(weights) else (lambda e: weights[e])
    y = np.zeros_like(x_perm)
    h = None
    for e in range(len(offsets) - 1):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b > a:
            wg, wu, wd = get(e)
            ye, he = swiglu_a8(x_perm[a:b], wg, wu, wd)
            if h is None:
                h = np.zeros((x_perm.shape[0], he.shape[1]))
            y[a:b] = ye
            h[a:b] = he
    return y, h
