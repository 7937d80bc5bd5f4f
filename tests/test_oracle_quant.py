"""Pins of the fp8-activation oracle (``oracle.quant``).

Each test checks the oracle against something other than itself: torch's
float8_e4m3fn and bfloat16 casts (library routines with their own rounding
code), closed forms of the quantiser (group maximum -> 448, power-of-two scale
invariance, the all-zero group), the e4m3 half-ulp error bound, brute force
over explicit block indices on a tiny product, and the lossless case where
the fp8 path reduces to the bf16 expert oracle.
"""

import numpy as np
import torch

import oracle


def rng(seed=0):
    return np.random.default_rng(seed)


def test_e4m3_encode_roundtrips_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = oracle.fp8_bits_to_f64(codes)
    assert np.array_equal(oracle.e4m3fn_encode(vals), codes)


def test_e4m3_encode_matches_torch_cast_in_range():
    r = rng(3)
    v = np.concatenate([r.uniform(-448, 448, 20000), r.normal(0, 0.01, 20000),
                        r.normal(0, 2.0 ** -8, 5000)]).astype(np.float32)
    ours = oracle.e4m3fn_encode(v.astype(np.float64))
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_encode_ties_go_to_even_code_and_saturate():
    t = oracle.e4m3fn_decode_table()
    # midpoint between 1.0 (0x38) and 1.125 (0x39) -> 0x38 (even); between
    # 1.125 and 1.25 (0x3A) -> 0x3A
    assert oracle.e4m3fn_encode([1.0625])[0] == 0x38
    assert oracle.e4m3fn_encode([1.1875])[0] == 0x3A
    assert oracle.e4m3fn_encode([-1.1875])[0] == 0xBA
    assert oracle.e4m3fn_encode([1000.0, -1000.0]).tolist() == [0x7E, 0xFE]
    assert t[0x7E] == 448.0
    # smallest subnormal 2^-9: half of it ties to zero (even), just above rounds up
    assert oracle.e4m3fn_encode([2.0 ** -10, 2.0 ** -10 * 1.01]).tolist() == [0x00, 0x01]


def test_bf16_round_matches_torch_cast_of_float32():
    r = rng(4)
    v = np.concatenate([r.normal(0, 1, 20000), r.normal(0, 1e-3, 5000)]).astype(np.float32)
    ours = oracle.bf16_round(v.astype(np.float64))
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(ours, ref)


def bf16_values(shape, seed, scale=1.0):
    v = rng(seed).normal(0, scale, shape).astype(np.float32)
    return torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()


def test_quantize_rows_group_max_maps_to_448_and_error_bound():
    x = bf16_values((16, 512), 5)
    q, s = oracle.quantize_rows(x)
    assert q.shape == x.shape and s.shape == (16, 4)
    vals = oracle.fp8_bits_to_f64(q)
    for r_ in range(16):
        for g in range(4):
            blk = x[r_, 128 * g:128 * (g + 1)]
            j = int(np.argmax(np.abs(blk)))
            assert abs(vals[r_, 128 * g + j]) == 448.0
            assert np.sign(vals[r_, 128 * g + j]) == np.sign(blk[j])
    # |x - q s| <= half an e4m3 ulp at |x/s| (3 mantissa bits), times s, plus
    # the two float32 roundings of s and x/s
    xd = oracle.dequant_rows(q, s)
    ratio = np.abs(x) / np.repeat(s, 128, axis=1)
    ulp = np.where(ratio >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(ratio, 2.0 ** -6))) - 3),
                   2.0 ** -9)
    bound = (0.5 * ulp + ratio * 2.0 ** -23) * np.repeat(s, 128, axis=1)
    assert np.all(np.abs(x - xd) <= bound * (1 + 1e-12))


def test_quantize_rows_matches_torch_division_and_cast():
    x = bf16_values((8, 384), 6)
    q, s = oracle.quantize_rows(x)
    xt = torch.from_numpy(x.astype(np.float32)).view(8, 3, 128)
    amax = xt.abs().amax(dim=2).clamp_min(torch.tensor(1e-4, dtype=torch.float32))
    st = amax / torch.tensor(448.0, dtype=torch.float32)
    qt = (xt / st[:, :, None]).to(torch.float8_e4m3fn).view(torch.uint8).reshape(8, 384)
    assert np.array_equal(q, qt.numpy())
    assert np.array_equal(s, st.double().numpy())


def test_quantize_rows_power_of_two_invariance_and_zero_group():
    x = bf16_values((4, 256), 7)
    q1, s1 = oracle.quantize_rows(x)
    q2, s2 = oracle.quantize_rows(x * 2.0 ** 5)
    assert np.array_equal(q1, q2) and np.array_equal(s2, s1 * 2.0 ** 5)
    z = np.zeros((2, 128))
    qz, sz = oracle.quantize_rows(z)
    assert not qz.any() and np.all(sz == np.float64(np.float32(np.float32(1e-4) / np.float32(448))))


def test_fp8_product_brute_force_block_indices():
    # two 128-channel groups, two 128-column weight blocks: a slip in the scale
    # indexing (row/column of the weight scale, group of the activation scale)
    # changes the result
    r = rng(8)
    x = bf16_values((3, 256), 9)
    xq, xs = oracle.quantize_rows(x)
    wq = r.integers(0, 0x7E, size=(256, 256)).astype(np.uint8) | (r.integers(0, 2, (256, 256)) << 7).astype(np.uint8)
    ws = r.uniform(0.5, 2.0, size=(2, 2))
    fast = oracle.dequant_rows(xq, xs) @ oracle.dequant_block_fp8(wq, ws)
    xv, wv = oracle.fp8_bits_to_f64(xq), oracle.fp8_bits_to_f64(wq)
    for t in range(3):
        for n in (0, 1, 127, 128, 200, 255):
            acc = 0.0
            for k in range(256):
                acc += xv[t, k] * xs[t, k // 128] * wv[k, n] * ws[k // 128, n // 128]
            assert abs(fast[t, n] - acc) <= 1e-9 * (1 + abs(acc))


def test_swiglu_a8_lossless_inputs_reduce_to_bf16_oracle():
    # rows whose groups are exactly code x 2^-4 with a 448 entry quantise
    # losslessly, so the gate/up half equals the plain oracle (rounded to bf16)
    r = rng(10)
    codes = r.integers(0, 0x7E, size=(5, 256)).astype(np.uint8)
    codes[:, 0] = 0x7E
    codes[:, 128] = 0xFE
    x = oracle.fp8_bits_to_f64(codes) * 2.0 ** -4
    wg = r.normal(0, 0.02, (256, 128))
    wu = r.normal(0, 0.02, (256, 128))
    wd = r.normal(0, 0.02, (128, 256))
    xq, xs = oracle.quantize_rows(x)
    assert np.array_equal(oracle.dequant_rows(xq, xs), x)
    y, h = oracle.swiglu_a8(x, wg, wu, wd)
    assert np.array_equal(h, oracle.bf16_round(oracle.silu(x @ wg) * (x @ wu)))
    # and the down half is the plain product of the requantised intermediate
    hq, hs = oracle.quantize_rows(h)
    assert np.allclose(y, oracle.dequant_rows(hq, hs) @ wd, rtol=0, atol=1e-12)
    # which is within the fp8 tolerance of the unquantised MLP
    ref = oracle.swiglu(x, wg, wu, wd)
    assert np.linalg.norm(y - ref) / np.linalg.norm(ref) < 3e-2


def test_experts_a8_runs_each_expert_on_its_rows():
    x = bf16_values((10, 128), 11)
    offsets = np.array([0, 4, 4, 10])
    r = rng(12)
    W = [(r.normal(0, 0.05, (128, 128)), r.normal(0, 0.05, (128, 128)), r.normal(0, 0.05, (128, 128)))
         for _ in range(3)]
    y, h = oracle.experts_a8(x, offsets, W)
    for e, (a, b) in enumerate([(0, 4), (4, 4), (4, 10)]):
        if b > a:
            ye, he = oracle.swiglu_a8(x[a:b], *W[e])
            assert np.array_equal(y[a:b], ye) and np.array_equal(h[a:b], he)


def _torch_quantize_rows(x64: np.ndarray) -> np.ndarray:
    """Per-token 1x128 fp8 activations written with torch's own float32
    arithmetic and float8_e4m3fn cast (not the oracle's encoder): returns the
    dequantised values code * scale."""
    x = torch.from_numpy(x64).float()
    rows, K = x.shape
    g = x.reshape(rows, K // 128, 128)
    s = torch.clamp(g.abs().amax(dim=2), min=1e-4) / 448.0
    q = (g / s[:, :, None]).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
    return (q.double() * s.double()[:, :, None]).reshape(rows, K).numpy()


def _bf16(x64: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.asarray(x64)).float().bfloat16().double().numpy()


def test_moe_ffn_fp8_activations_matches_per_token_definition():
    # The block-fp8 prefill sub-block, token by token from its definition:
    # v = bf16(RMSNorm(x)); routed set and weights from v; for each local
    # expert e in the set: h = bf16(SiLU(Q(v) Wg_e) * (Q(v) Wu_e)) and
    # y = Q(h) Wd_e with Q the per-token 1x128 fp8 quantise-dequantise;
    # out = sum over local e of w_e * y_e. Torch ops throughout (rms_norm,
    # float32 division, the float8_e4m3fn and bfloat16 casts), so a wiring slip
    # in the oracle's permute -> experts_a8 -> combine path (a dropped bf16
    # rounding of V, the unquantised V in one product, a wrong expert's
    # weights, a mis-scaled combine) shows up here.
    import torch.nn.functional as F
    r = rng(46)
    T, d, f, E, eb, ec = 19, 256, 128, 12, 2, 7
    x = r.standard_normal((T, d))
    gam = 1 + 0.1 * r.standard_normal(d)
    w_r, b = r.standard_normal((E, d)) * 0.05, r.standard_normal(E) * 0.05
    ws = [tuple(r.normal(0, 0.05, s) for s in ((d, f), (d, f), (f, d))) for _ in range(ec)]
    res = oracle.moe_ffn(x, gam, w_r, b, ws, eb, ec, act_fp8=True)
    v = F.rms_norm(torch.from_numpy(x), (d,), weight=torch.from_numpy(gam), eps=1e-5).numpy()
    vb = _bf16(v)
    for t in range(T):
        # routing is the same as the bf16 path's (on v, not on its bf16 copy)
        z = v[t] @ w_r.T
        s = 1 / (1 + np.exp(-z))
        top = np.sort(np.lexsort((np.arange(E), -(s + b)))[:8])
        assert np.array_equal(res["idx"][t], top)
        acc = np.zeros(d)
        xq = _torch_quantize_rows(vb[t:t + 1])
        for e in top:
            if eb <= e < eb + ec:
                wg, wu, wd = ws[e - eb]
                h = _bf16(F.silu(torch.from_numpy(xq @ wg)).numpy() * (xq @ wu))
                acc += s[e] / s[top].sum() * (_torch_quantize_rows(h) @ wd)[0]
        assert np.allclose(res["out"][t], acc, rtol=1e-10, atol=1e-12), t
    # some tokens have no local expert (exact zeros), most have several
    n_local = np.isin(res["idx"], np.arange(eb, eb + ec)).sum(1)
    assert np.all(res["out"][n_local == 0] == 0)
    assert n_local.max() >= 3
