"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: a library
routine (torch float64 ops, numpy's stable argsort, torch.topk, torch's fp8 and
bf16 casts), a closed form, brute force on tiny inputs, the pages' worked
example (tests/golden), or an invariant the pages state. Each is chosen so that
a plausible slip in the oracle (a dropped term, a wrong sign or index, a
transposed operand, the bias in the wrong place, SiLU on the wrong branch)
fails at least one of them.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rng(seed=0):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- decoding --

def test_bf16_decode_matches_torch_cast():
    bits = rng(1).integers(0, 2**16, size=20000, dtype=np.uint16)
    bits[:4] = [0x0000, 0x8000, 0x3F80, 0xC2F7]  # +0, -0, 1.0, -123.5
    ours = oracle.bf16_bits_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(ours, ref, equal_nan=True)
    assert ours[2] == 1.0 and ours[3] == -123.5


def test_e4m3fn_table_matches_torch_for_all_codes():
    table = oracle.e4m3fn_decode_table()
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(table, ref, equal_nan=True)
    assert table[0x7E] == 448.0 and table[0x01] == 2.0 ** -9 and np.isnan(table[0x7F])


def test_block_fp8_dequant_scales_each_block_in_place():
    # Distinct power-of-two scale per block: a transposed or shifted scale
    # array, or a scale applied per row instead of per block, changes values.
    K, N = 256, 384
    q = rng(2).integers(0, 256, size=(K, N)).astype(np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x38  # no NaN codes
    s = np.array([[2.0 ** (i + 3 * j) for j in range(N // 128)] for i in range(K // 128)],
                 dtype=np.float32)
    w = oracle.dequant_block_fp8(q, s)
    codes = torch.from_numpy(q).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for bi in range(K // 128):
        for bj in range(N // 128):
            blk = (slice(bi * 128, (bi + 1) * 128), slice(bj * 128, (bj + 1) * 128))
            assert np.array_equal(w[blk], codes[blk] * 2.0 ** (bi + 3 * bj))


def test_block_fp8_roundtrip_error_bound():
    # Quantising with torch's RNE cast, the oracle's dequantisation is within
    # half an E4M3 ulp (relative 2^-4) of every value in the normal range.
    w = rng(3).standard_normal((256, 256)) * 0.02
    blocks = w.reshape(2, 128, 2, 128)
    amax = np.abs(blocks).max(axis=(1, 3))
    scale = (amax / 448.0).astype(np.float32)
    qf = torch.from_numpy(blocks / scale[:, None, :, None].astype(np.float64)).clamp(-448, 448)
    q = qf.to(torch.float8_e4m3fn).view(torch.uint8).numpy().reshape(256, 256)
    deq = oracle.dequant_block_fp8(q, scale)
    srep = np.repeat(np.repeat(scale.astype(np.float64), 128, 0), 128, 1)
    normal = np.abs(w) >= srep * 2.0 ** -6
    rel = np.abs(deq - w)[normal] / np.abs(w)[normal]
    assert rel.max() <= 2.0 ** -4 + 1e-12


# ---------------------------------------------------------------- RMSNorm --

def test_rmsnorm_matches_torch_rms_norm():
    x = rng(4).standard_normal((37, 96)) * 3.0
    g = 1.0 + 0.1 * rng(5).standard_normal(96)
    ours = oracle.rmsnorm(x, g, 1e-5)
    ref = F.rms_norm(torch.from_numpy(x), (96,), weight=torch.from_numpy(g), eps=1e-5).numpy()
    assert np.allclose(ours, ref, rtol=1e-14, atol=1e-14)


def test_rmsnorm_closed_forms():
    d = 4096
    g = np.linspace(0.5, 1.5, d)
    c = 0.003  # small enough that eps matters: checks eps sits inside the sqrt
    y = oracle.rmsnorm(np.full((1, d), c), g, 1e-5)
    assert np.allclose(y[0], g * c / math.sqrt(c * c + 1e-5), rtol=1e-15)
    assert np.array_equal(oracle.rmsnorm(np.zeros((2, d)), g, 1e-5), np.zeros((2, d)))
    # the mean runs over the hidden dim: one nonzero entry a gives a/sqrt(a^2/d+eps)
    x = np.zeros((1, d))
    x[0, 7] = 2.0
    y = oracle.rmsnorm(x, np.ones(d), 1e-5)
    assert math.isclose(y[0, 7], 2.0 / math.sqrt(4.0 / d + 1e-5), rel_tol=1e-15)
    # scale invariance once |x| >> sqrt(eps): eps's share shrinks as 1/alpha^2
    xr = rng(6).standard_normal((3, 64))
    assert np.allclose(oracle.rmsnorm(1e4 * xr, 1.0), oracle.rmsnorm(xr, 1.0, eps=0.0), rtol=1e-9)
    assert not np.allclose(oracle.rmsnorm(xr, 1.0), oracle.rmsnorm(xr, 1.0, eps=0.0), rtol=1e-7)


# ------------------------------------------------------------ gated MLP --

def test_sigmoid_silu_closed_forms():
    assert oracle.sigmoid(0.0) == 0.5
    assert math.isclose(float(oracle.sigmoid(math.log(3.0))), 0.75, rel_tol=1e-15)
    a = np.linspace(-20, 20, 101)
    assert np.allclose(oracle.silu(a), F.silu(torch.from_numpy(a)).numpy(), rtol=1e-14, atol=1e-300)


def test_swiglu_one_by_one_closed_form_catches_branch_swap():
    # d = f = 1: Y = SiLU(x g) (x u) d with SiLU(ln 3) = 0.75 ln 3.
    y = oracle.swiglu([[1.0]], [[math.log(3.0)]], [[2.0]], [[5.0]])
    assert math.isclose(y[0, 0], 0.75 * math.log(3.0) * 2.0 * 5.0, rel_tol=1e-14)
    # SiLU on the up branch instead would give SiLU(2) ln3 * 5
    assert not math.isclose(y[0, 0], 2.0 / (1 + math.exp(-2.0)) * math.log(3.0) * 5.0, rel_tol=1e-3)


def test_swiglu_matches_torch_float64():
    r = rng(7)
    x, wg, wu, wd = (r.standard_normal(s) for s in ((9, 32), (32, 48), (32, 48), (48, 32)))
    ours = oracle.swiglu(x, wg, wu, wd)
    tx, tg, tu, td = (torch.from_numpy(a) for a in (x, wg, wu, wd))
    ref = ((F.silu(tx @ tg) * (tx @ tu)) @ td).numpy()
    assert np.allclose(ours, ref, rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------- TP shards --

def test_tp_linear_worked_example():
    ex = json.load(open(os.path.join(GOLDEN, "tp_linear_worked_example.json")))
    W, X, p = np.array(ex["W"], float), np.array(ex["X"], float), ex["p"]
    for i in range(p):
        assert np.array_equal(oracle.column_parallel(X, W, p, i), np.array(ex["column_shards"][i]))
        assert np.array_equal(oracle.row_parallel_partial(X, W, p, i), np.array(ex["row_partials"][i]))
    cat = np.concatenate([oracle.column_parallel(X, W, p, i) for i in range(p)], axis=1)
    tot = sum(oracle.row_parallel_partial(X, W, p, i) for i in range(p))
    assert np.array_equal(cat, np.array(ex["Y_full"])) and np.array_equal(tot, np.array(ex["Y_full"]))


def test_column_split_exact_on_integer_matrices():
    # "LLM推理并行优化的必备知识" §1.1: integer matrices, column split, concat == A@B exactly.
    r = rng(8)
    A = r.integers(0, 10, size=(3, 4)).astype(float)
    B = r.integers(0, 10, size=(4, 6)).astype(float)
    full = (A.astype(np.int64) @ B.astype(np.int64)).astype(float)
    cat = np.concatenate([oracle.column_parallel(A, B, 3, i) for i in range(3)], axis=1)
    assert np.array_equal(cat, full)
    tot = sum(oracle.row_parallel_partial(A, B, 2, i) for i in range(2))
    assert np.array_equal(tot, full)


def test_tp_shard_partials_sum_to_full_mlp():
    r = rng(9)
    x = r.standard_normal((16, 64))
    wg, wu = r.standard_normal((64, 256)) * 0.02, r.standard_normal((64, 256)) * 0.02
    wd = r.standard_normal((256, 64)) * 0.02
    full = oracle.swiglu(x, wg, wu, wd)
    parts = [oracle.tp_shard_mlp(x, wg, wu, wd, 4, i) for i in range(4)]
    assert np.allclose(sum(parts), full, rtol=1e-12, atol=1e-15)
    # each part differs from the full result (it really is only part of the sum)
    assert all(not np.allclose(pt, full) for pt in parts)
    # the gate projection's column shards concatenate to the full projection
    cat = np.concatenate([oracle.column_parallel(x, wg, 4, i) for i in range(4)], axis=1)
    assert np.array_equal(cat, x @ wg)


# ------------------------------------------------------------- router --

def _brute_force_topk(key, k):
    """The unique k-subset every member of which beats every non-member
    under (key descending, id ascending), found by enumerating all subsets."""
    E = len(key)

    def beats(a, b):
        return key[a] > key[b] or (key[a] == key[b] and a < b)

    found = []
    for sub in itertools.combinations(range(E), k):
        rest = [e for e in range(E) if e not in sub]
        if all(beats(a, b) for a in sub for b in rest):
            found.append(sub)
    assert len(found) == 1
    return np.array(found[0])


@pytest.mark.parametrize("E", [8, 9, 12])
def test_route_brute_force_small(E):
    r = rng(10 + E)
    x = r.standard_normal((25, 16))
    w_r = r.standard_normal((E, 16)) * 0.3
    b = r.standard_normal(E) * 0.05
    idx, w, s, key, gap = oracle.route(x, w_r, b, 8)
    for t in range(25):
        assert np.array_equal(idx[t], _brute_force_topk(key[t], 8))
        assert np.all(np.diff(idx[t]) > 0)
    assert np.all(w > 0) and np.allclose(w.sum(1), 1.0, atol=1e-12)
    # s really is the sigmoid of x W_r^T (router input contracted with W_r's rows)
    z = torch.from_numpy(x) @ torch.from_numpy(w_r).T
    assert np.allclose(s, torch.sigmoid(z).numpy(), rtol=1e-14)


def test_route_exact_ties_pick_lower_index():
    r = rng(20)
    d, E = 16, 12
    w_r = r.standard_normal((E, d)) * 0.3
    w_r[5] = w_r[2]   # experts 2 and 5 score identically
    w_r[9] = w_r[2]   # and 9
    b = np.zeros(E)
    x = r.standard_normal((200, d))
    idx, *_ , key, gap = oracle.route(x, w_r, b, 8)
    for t in range(200):
        sel = set(idx[t].tolist())
        # whenever only some of the tied trio make it, the lower ids win
        trio = [2, 5, 9]
        inside = [e for e in trio if e in sel]
        assert inside == trio[:len(inside)]
        assert np.array_equal(idx[t], _brute_force_topk(key[t], 8))


def test_route_without_bias_equals_topk_of_logits():
    r = rng(21)
    x = r.standard_normal((64, 32))
    w_r = r.standard_normal((40, 32)) * 0.2
    idx, *_ = oracle.route(x, w_r, np.zeros(40), 8)
    z = torch.from_numpy(x) @ torch.from_numpy(w_r).T
    ref = torch.topk(z, 8, dim=1).indices.sort(dim=1).values.numpy()
    assert np.array_equal(idx, ref)


def test_route_bias_added_after_sigmoid_and_not_in_weights():
    # "推理计算流梳理", MoE Router 过程: I = Top8(s + b) with s = sigmoid(z), and
    # the bias takes no part in the weights. Experts 0..6 are certain picks;
    # expert 7 (z = 5, b = 0) and expert 8 (z = 0, b = 0.6) compete for the
    # 8th place: with the bias after the sigmoid 0.5 + 0.6 > sigmoid(5), so
    # expert 8 wins; with the bias added to z, expert 7 would win.
    E, d = 10, 10
    w_r = np.eye(E, d)
    b = np.array([1.0] * 7 + [0.0, 0.6, -1.0])
    x = np.array([[10.0] * 7 + [5.0, 0.0, 0.0]])
    idx, w, s, key, gap = oracle.route(x, w_r, b, 8)
    assert idx[0].tolist() == [0, 1, 2, 3, 4, 5, 6, 8]
    sz = 1 / (1 + np.exp(-x[0]))
    assert np.allclose(w[0], sz[idx[0]] / sz[idx[0]].sum(), rtol=1e-15)
    # weights are independent of the bias once the set is fixed
    idx2, w2, *_ = oracle.route(x, w_r, b + np.array([0.1] * 7 + [0.0, 0.1, 0.0]), 8)
    assert np.array_equal(idx2, idx) and np.array_equal(w2, w)
    assert math.isclose(gap[0], key[0, 8] - key[0, 7])


# ------------------------------------------------------------ permute --

def _routing(T, E, k, seed):
    r = rng(seed)
    return np.sort(np.array([r.choice(E, size=k, replace=False) for _ in range(T)]), axis=1)


@pytest.mark.parametrize("e_begin,e_count", [(0, 32), (8, 9), (0, 1), (31, 1)])
def test_permute_matches_stable_argsort(e_begin, e_count):
    T, E, k = 301, 32, 8
    idx = _routing(T, E, k, 30)
    x = rng(31).standard_normal((T, 5))
    counts, offsets, src, inv, xp = oracle.permute(idx, e_begin, e_count, x)
    flat_e = idx.reshape(-1)
    flat_t = np.repeat(np.arange(T), k)
    local = (flat_e >= e_begin) & (flat_e < e_begin + e_count)
    order = np.argsort(flat_e[local], kind="stable")
    assert np.array_equal(src, flat_t[local][order])
    assert np.array_equal(counts, np.bincount(flat_e[local] - e_begin, minlength=e_count))
    assert offsets[0] == 0 and offsets[-1] == counts.sum() == local.sum()
    for e in range(e_count):
        seg = src[offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(seg) > 0)
    for t in range(T):
        for j in range(k):
            if e_begin <= idx[t, j] < e_begin + e_count:
                r_ = inv[t, j]
                assert src[r_] == t and offsets[idx[t, j] - e_begin] <= r_ < offsets[idx[t, j] - e_begin + 1]
                assert np.array_equal(xp[r_], x[t])
            else:
                assert inv[t, j] == -1


def test_permute_all_local_counts_sum_to_tokens_times_k():
    idx = _routing(100, 16, 8, 32)
    counts, offsets, src, inv, _ = oracle.permute(idx, 0, 16)
    assert counts.sum() == 100 * 8 and np.all(inv >= 0)
    assert sorted(inv.reshape(-1).tolist()) == list(range(800))


# ------------------------------------------------- experts and combine --

def test_moe_with_shared_expert_weights_equals_dense_mlp():
    # All experts share one weight set and all are local: since the router
    # weights sum to 1, the MoE output equals the dense gated MLP of V.
    r = rng(40)
    T, d, f, E = 40, 32, 48, 12
    x = r.standard_normal((T, d))
    wg, wu, wd = r.standard_normal((d, f)) * 0.2, r.standard_normal((d, f)) * 0.2, r.standard_normal((f, d)) * 0.2
    res = oracle.moe_ffn(x, np.ones(d), r.standard_normal((E, d)) * 0.3, r.standard_normal(E) * 0.01,
                         [(wg, wu, wd)] * E, 0, E)
    dense = oracle.swiglu(oracle.rmsnorm(x, np.ones(d)), wg, wu, wd)
    assert np.allclose(res["out"], dense, rtol=1e-12, atol=1e-14)


def test_combine_identity_expert_returns_input():
    T, E, k, d = 50, 16, 8, 7
    idx = _routing(T, E, k, 41)
    x = rng(42).standard_normal((T, d))
    w = rng(43).random((T, k)) + 0.1
    w /= w.sum(1, keepdims=True)
    counts, offsets, src, inv, xp = oracle.permute(idx, 0, E, x)
    out = oracle.combine(xp, inv, w)  # identity experts: y_perm = x_perm
    assert np.allclose(out, x, rtol=1e-14, atol=1e-14)


def test_combine_residual_passes_through_without_local_experts():
    # [P1] Norm&Residual: block output = R + FFN(V). A token none of whose
    # experts is local has FFN part 0 on this rank, so its output is exactly R;
    # elsewhere the residual is the difference between the two combines.
    T, E, k, d = 40, 16, 8, 5
    idx = _routing(T, E, k, 45)
    r = rng(46)
    x, R = r.standard_normal((T, d)), r.standard_normal((T, d))
    w = r.random((T, k)) + 0.1
    w /= w.sum(1, keepdims=True)
    _, _, _, inv, xp = oracle.permute(idx, 0, 2, x)
    none = np.all(inv < 0, axis=1)
    assert none.any() and (~none).any()
    with_r = oracle.combine(xp, inv, w, residual=R)
    assert np.array_equal(with_r[none], R[none])
    assert np.allclose(with_r - oracle.combine(xp, inv, w), R, rtol=0, atol=1e-12)


def test_expert_parallel_partials_sum_to_all_local_output():
    # Disjoint expert ranges (8 ranks of 2 experts) give partial outputs that
    # add up to the all-local output: the combine keeps the global weights.
    r = rng(44)
    T, d, f, E = 30, 16, 24, 16
    x = r.standard_normal((T, d))
    w_r, b = r.standard_normal((E, d)) * 0.3, r.standard_normal(E) * 0.01
    ws = [tuple(r.standard_normal(s) * 0.2 for s in ((d, f), (d, f), (f, d))) for _ in range(E)]
    full = oracle.moe_ffn(x, np.ones(d), w_r, b, ws, 0, E)["out"]
    parts = [oracle.moe_ffn(x, np.ones(d), w_r, b, ws[2 * q:2 * q + 2], 2 * q, 2)["out"] for q in range(8)]
    assert np.allclose(sum(parts), full, rtol=1e-12, atol=1e-14)
    # a token whose 8 experts are all outside a range gets exactly zero there
    res = oracle.moe_ffn(x, np.ones(d), w_r, b, ws[:1], 0, 1)
    none = np.all(res["inv_pos"] < 0, axis=1)
    assert np.all(res["out"][none] == 0)


def test_moe_ffn_matches_per_token_definition():
    # The permute/experts/combine route must equal the per-token definition
    # out[t] = sum over local e in I_t of w_te * SwiGLU_e(v_t).
    r = rng(45)
    T, d, f, E, eb, ec = 23, 16, 32, 12, 3, 6
    x = r.standard_normal((T, d))
    g = 1 + 0.1 * r.standard_normal(d)
    w_r, b = r.standard_normal((E, d)) * 0.3, r.standard_normal(E) * 0.05
    ws = [tuple(r.standard_normal(s) * 0.2 for s in ((d, f), (d, f), (f, d))) for _ in range(ec)]
    res = oracle.moe_ffn(x, g, w_r, b, ws, eb, ec)
    v = F.rms_norm(torch.from_numpy(x), (d,), weight=torch.from_numpy(g), eps=1e-5).numpy()
    for t in range(T):
        acc = np.zeros(d)
        z = v[t] @ w_r.T
        s = 1 / (1 + np.exp(-z))
        top = _brute_force_topk(s + b, 8)
        for e in top:
            if eb <= e < eb + ec:
                wg, wu, wd = ws[e - eb]
                h = F.silu(torch.from_numpy(v[t] @ wg)).numpy() * (v[t] @ wu)
                acc += s[e] / s[top].sum() * (h @ wd)
        assert np.allclose(res["out"][t], acc, rtol=1e-11, atol=1e-13)


# ---------------------------------------------------------- masked dispatch --

def test_dispatch_masked_blocks_are_the_contiguous_buckets():
    r = rng(21)
    T, E, k, eb, ec = 50, 24, 8, 4, 12
    idx = np.sort(np.stack([r.choice(E, k, replace=False) for _ in range(T)]), axis=1)
    counts, offsets, src, inv, _ = oracle.permute(idx, eb, ec)
    cap = T  # a token picks an expert at most once: nothing is dropped
    mc, rows, pos = oracle.dispatch_masked(idx, eb, ec, cap)
    assert np.array_equal(mc, counts)
    for e in range(ec):
        blk = rows[e * cap:(e + 1) * cap]
        assert np.array_equal(blk[:counts[e]], src[offsets[e]:offsets[e + 1]])
        assert (blk[counts[e]:] == -1).all()
    local = inv >= 0
    e_of = idx - eb
    assert np.array_equal(pos >= 0, local)
    assert np.array_equal(pos[local] - e_of[local] * cap,
                          inv[local] - offsets[e_of[local]])


def test_dispatch_masked_capacity_keeps_the_first_tokens():
    r = rng(22)
    T, E, k, cap = 40, 10, 4, 3
    idx = np.sort(np.stack([r.choice(E, k, replace=False) for _ in range(T)]), axis=1)
    mc, rows, pos = oracle.dispatch_masked(idx, 0, E, cap)
    for e in range(E):
        toks = np.nonzero((idx == e).any(axis=1))[0]      # ascending token ids routed to e
        keep = toks[:cap]
        assert mc[e] == len(keep)
        assert np.array_equal(rows[e * cap:e * cap + len(keep)], keep)
        for t in toks[cap:]:                               # dropped slots
            assert pos[t][idx[t] == e][0] == -1


def test_combine_is_layout_independent():
    r = rng(23)
    T, E, k, d = 30, 16, 8, 5
    idx = np.sort(np.stack([r.choice(E, k, replace=False) for _ in range(T)]), axis=1)
    w = r.uniform(0, 1, (T, k))
    val = r.normal(0, 1, (T, k, d))                       # the expert output of each slot
    counts, offsets, src, inv, _ = oracle.permute(idx, 0, E)
    y_c = np.zeros((T * k, d))
    mc, rows, pos = oracle.dispatch_masked(idx, 0, E, T)
    y_m = np.zeros((E * T, d))
    for t in range(T):
        for j in range(k):
            y_c[inv[t, j]] = val[t, j]
            y_m[pos[t, j]] = val[t, j]
    assert np.allclose(oracle.combine(y_c, inv, w), oracle.combine(y_m, pos, w), rtol=0, atol=0)
