"""GPU parity of the block-fp8 prefill variant: per-token 1x128 activation
quantisation and the fp8-activation grouped GEMMs, against the fp64 oracle.

The quantiser's codes and scales are compared bit for bit (both sides take the
code decision in float32 with IEEE division and round to nearest even). Each
GEMM is compared with the oracle evaluated on the GPU's own codes (bf16
output tolerance), and the whole expert MLP with the oracle from the raw bf16
rows (the fp8 tolerance).
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.parity import REL_BF16, REL_FP8, assert_fp, fp8_weight_f64, to_f64
from tests.test_gpu_stages import DEV, _expert_weights, _offsets

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def g():
    import gated_mlp_transformer_amd as g_
    assert torch.cuda.is_available()
    return g_


def _codes(q):
    return q.cpu().numpy().astype(np.uint8)


def _rows_with_structure(rows, K, seed):
    """bf16 rows whose 128-groups span magnitudes 1e-3 .. 30, one all-zero
    group and tiny negatives (which quantise to the negative zero code)."""
    x = synth.normal((rows, K), name="t.q8.x", sub=seed, device=DEV).float()
    mag = synth.normal((rows, K // 128), name="t.q8.mag", sub=seed, std=1.0, mean=-0.75,
                       dtype=torch.float32, device=DEV).clamp(-3.0, 1.5)
    x = x * torch.pow(10.0, mag).repeat_interleave(128, dim=1)
    if rows > 2 and K >= 256:
        x[1, 128:256] = 0.0
        x[2, :8] = -1e-9
        x[2, 8] = 1.0
    return x.to(torch.bfloat16)


@pytest.mark.parametrize("rows,K", [(1, 128), (3, 256), (37, 384), (300, 4096), (5, 8192)])
def test_quantize_fp8_rows_bit_exact(g, rows, K):
    x = _rows_with_structure(rows, K, seed=rows * 7 + K)
    q, s = g.quantize_fp8_rows(x)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quantize_rows(to_f64(x))
    assert np.array_equal(s.double().cpu().numpy(), s_ref)
    got = _codes(q)
    bad = np.argwhere(got != q_ref)
    assert bad.size == 0, f"{len(bad)} codes differ, first {bad[:3].tolist()}: " \
                          f"{got[tuple(bad[0])]:#x} vs {q_ref[tuple(bad[0])]:#x}"


@pytest.mark.parametrize("live", [0, 1, 57, 300, 500])
def test_quantize_fp8_rows_device_row_count(g, live):
    # only rows < min(*row_count, rows) are written; the rest keep their contents
    rows, K = 300, 512
    x = _rows_with_structure(rows, K, seed=live + 11)
    q = torch.full((rows, K), 0xA5, dtype=torch.uint8, device=DEV)
    s = torch.full((rows, K // 128), -1.0, dtype=torch.float32, device=DEV)
    cnt = torch.tensor([live], dtype=torch.int32, device=DEV)
    g.quantize_fp8_rows(x, row_count=cnt, q=q, scales=s)
    torch.cuda.synchronize()
    n = min(live, rows)
    q_ref, s_ref = oracle.quantize_rows(to_f64(x[:n])) if n else (np.zeros((0, K)), np.zeros((0, 4)))
    assert np.array_equal(_codes(q[:n]), q_ref) and np.array_equal(s[:n].double().cpu().numpy(), s_ref)
    assert (q[n:] == 0xA5).all() and (s[n:] == -1.0).all()


def test_quantize_fp8_rows_zero_rows(g):
    x = torch.zeros((0, 256), dtype=torch.bfloat16, device=DEV)
    q, s = g.quantize_fp8_rows(x)
    assert q.shape == (0, 256) and s.shape == (0, 2)


def _oracle_w(W, e):
    return (fp8_weight_f64(W["w_gate"][e], W["s_gate"][e]),
            fp8_weight_f64(W["w_up"][e], W["s_up"][e]),
            fp8_weight_f64(W["w_down"][e], W["s_down"][e]))


@pytest.mark.parametrize("counts,d,f", [
    ([1, 3, 0, 17, 2, 16], 256, 512),
    ([40], 512, 256),
    ([0, 0, 0], 256, 256),
    ([1, 33, 65, 97, 128, 129, 31, 32], 256, 256),     # every tail sub-tile count
    ([300] * 3 + [0, 77, 513] + [300] * 4, 1024, 512),  # several tiles and rounds
    ([5, 40, 0, 33], 768, 256),   # gate/up: six stages (a four-stage body and a tail)
    ([7, 64], 256, 768),          # down: six stages
    # odd slab counts (d, f multiples of 128 only) and a down n-tile of 128 rows
    ([5, 40, 0, 33], 384, 128),   # three and one stages
    ([7, 64, 200], 640, 640),     # five stages: a four-stage body and one
    ([3, 300], 896, 1152),        # seven and nine stages
])
@pytest.mark.parametrize("gather", [False, True])
def test_grouped_a8(g, counts, d, f, gather):
    ec = len(counts)
    S = int(sum(counts))
    max_rows = S + 5
    W = _expert_weights(ec, d, f, "fp8", seed=S + d + 1)
    offsets = _offsets(counts)
    pw = [g.pack_weights(W[k_]) for k_ in ("w_gate", "w_up", "w_down")]
    h = torch.full((max_rows, f), float("nan"), dtype=torch.bfloat16, device=DEV)
    y = torch.full((max_rows, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    if gather:
        src_rows = max(1, S // 3 + 7)
        x_src = synth.normal((src_rows, d), name="t.a8.xsrc", sub=S, device=DEV)
        ri = synth.integers((max_rows,), 0, src_rows, name="t.a8.ri", sub=S).to(torch.int32)
        if S >= 2:
            ri[0], ri[S - 1] = -5, src_rows + 11
        ri = ri.to(DEV)
        xq, xs = g.quantize_fp8_rows(x_src)
        g.grouped_gate_up_a8(xq, xs, offsets, pw[0], pw[1], W["s_gate"], W["s_up"],
                             row_index=ri, h_out=h)
        idx = ri.long().clamp(0, src_rows - 1)
        x_perm = x_src[idx].contiguous()
        xq_rows, xs_rows = xq[idx], xs[idx]
    else:
        x_perm = synth.normal((max_rows, d), name="t.a8.x", sub=S, device=DEV)
        xq, xs = g.quantize_fp8_rows(x_perm)
        g.grouped_gate_up_a8(xq, xs, offsets, pw[0], pw[1], W["s_gate"], W["s_up"], h_out=h)
        xq_rows, xs_rows = xq, xs
    hq, hs = g.quantize_fp8_rows(h[:S].contiguous() if S else h[:0])
    hq_full = torch.zeros((max_rows, f), dtype=torch.uint8, device=DEV)
    hs_full = torch.ones((max_rows, f // 128), dtype=torch.float32, device=DEV)
    hq_full[:S], hs_full[:S] = hq, hs
    g.grouped_down_a8(hq_full, hs_full, offsets, pw[2], W["s_down"], y_perm=y)
    torch.cuda.synchronize()
    # rows past the last expert are never written
    assert torch.isnan(h[S:].float()).all() and torch.isnan(y[S:].float()).all()
    if S == 0:
        return
    off = offsets.cpu().numpy()
    xd = oracle.dequant_rows(_codes(xq_rows[:S]), xs_rows[:S].double().cpu().numpy())
    hd = oracle.dequant_rows(_codes(hq), hs.double().cpu().numpy())
    h_ref = np.zeros((S, f))
    y_ref = np.zeros((S, d))
    for e in range(ec):
        a, b = off[e], off[e + 1]
        if b > a:
            wg, wu, wd = _oracle_w(W, e)
            h_ref[a:b] = oracle.silu(xd[a:b] @ wg) * (xd[a:b] @ wu)
            y_ref[a:b] = hd[a:b] @ wd
    # each GEMM on the GPU's own fp8 operands: bf16 output rounding only
    assert_fp("H (gate/up on the GPU's codes)", to_f64(h[:S]), h_ref, rel=REL_BF16, max_abs=None)
    assert_fp("Y (down on the GPU's codes)", to_f64(y[:S]), y_ref, rel=REL_BF16, max_abs=None)
    # the H quantisation on the GPU's H is bit-exact
    hq_ref, hs_ref = oracle.quantize_rows(to_f64(h[:S]))
    assert np.array_equal(_codes(hq), hq_ref) and np.array_equal(hs.double().cpu().numpy(), hs_ref)
    # the whole expert MLP from the raw bf16 rows
    y_e2e, _ = oracle.experts_a8(to_f64(x_perm[:S]), off, lambda e: _oracle_w(W, e))
    assert_fp("Y_perm (fp8 path end to end)", to_f64(y[:S]), y_e2e, rel=REL_FP8, max_abs=None)
