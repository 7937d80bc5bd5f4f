"""Parity checking between the HIP path and the fp64 oracle.

Conversions hand the oracle the exact values the GPU received (bf16 and fp8
bit patterns decoded by the oracle's own decoders). Tolerances:

  * integers (expert ids, counts, offsets, permutation, inverse positions):
    bit-exact, except that a token whose 8th/9th biased-score gap (fp64) is
    below TIE may carry any expert set that is a valid top-8 within TIE
    (members all have key >= key_(8) - TIE and every expert with
    key > key_(9) + TIE is a member); the oracle then continues with the
    GPU's set for that token.
  * floating point with bf16 data: relative Frobenius error <= 5e-3 and max
    abs error <= 2e-2 on final outputs; relative Frobenius <= 5e-3 on the bf16
    intermediates H and Y_perm (max abs reported).
  * fp8 (block-scaled E4M3FN) weights: relative Frobenius <= 3e-2.
"""

from __future__ import annotations

import numpy as np
import torch

import oracle

TIE = 1e-6
REL_BF16, ABS_BF16 = 5e-3, 2e-2
REL_FP8 = 3e-2


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 values of a tensor (bf16 / f32 / fp8 via the oracle's decoders)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return oracle.bf16_bits_to_f64(t.view(torch.int16).numpy().view(np.uint16))
    if t.dtype == torch.float8_e4m3fn:
        return oracle.fp8_bits_to_f64(t.view(torch.uint8).numpy())
    return t.numpy().astype(np.float64)


def fp8_weight_f64(q: torch.Tensor, s: torch.Tensor) -> np.ndarray:
    """[N, K] E4M3FN codes + [N/128, K/128] scales -> the pages' [K, N] float64 weight."""
    qb = q.detach().cpu().contiguous().view(torch.uint8).numpy()
    return oracle.dequant_block_fp8(qb.T, s.detach().cpu().numpy().T)


def to_i64(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy().astype(np.int64)


def errors(got, ref) -> dict:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    diff = got - ref
    nref = np.linalg.norm(ref)
    return dict(rel=float(np.linalg.norm(diff) / nref) if nref > 0 else float(np.linalg.norm(diff)),
                max_abs=float(np.max(np.abs(diff))) if diff.size else 0.0)


def assert_fp(name, got, ref, rel=REL_BF16, max_abs=ABS_BF16) -> dict:
    e = errors(got, ref)
    assert np.all(np.isfinite(np.asarray(got, dtype=np.float64))), f"{name}: non-finite output"
    assert e["rel"] <= rel, f"{name}: rel Frobenius {e['rel']:.3e} > {rel:.1e} (max abs {e['max_abs']:.3e})"
    if max_abs is not None:
        assert e["max_abs"] <= max_abs, f"{name}: max abs {e['max_abs']:.3e} > {max_abs:.1e} (rel {e['rel']:.3e})"
    return e


def check_route(gpu_idx: np.ndarray, key: np.ndarray, gap: np.ndarray, ref_idx: np.ndarray,
                k: int = 8, tie: float = TIE) -> int:
    """Router ids: bit-exact where the oracle's 8th/9th gap >= tie, valid top-k otherwise.

    Returns the number of near-tie tokens whose GPU set differs from the oracle's.
    """
    gpu_idx = np.asarray(gpu_idx, dtype=np.int64)
    T, E = key.shape
    assert gpu_idx.shape == ref_idx.shape == (T, k)
    assert np.all(np.diff(gpu_idx, axis=1) > 0), "ids must be distinct and ascending"
    assert np.all((gpu_idx >= 0) & (gpu_idx < E))
    reconciled = 0
    for t in np.nonzero(np.any(gpu_idx != ref_idx, axis=1))[0]:
        assert gap[t] < tie, f"token {t}: expert set differs with 8th/9th gap {gap[t]:.3e} >= {tie}"
        kt = key[t]
        order = np.lexsort((np.arange(E), -kt))
        k8, k9 = kt[order[k - 1]], kt[order[k]]
        members = set(gpu_idx[t].tolist())
        assert all(kt[e] >= k8 - tie for e in members), f"token {t}: member below the tie band"
        must = {e for e in range(E) if kt[e] > k9 + tie}
        assert must <= members, f"token {t}: misses an expert clearly above the 9th key"
        reconciled += 1
    return reconciled
