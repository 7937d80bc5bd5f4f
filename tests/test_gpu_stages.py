"""GPU parity of every C-ABI call against the fp64 oracle, stage by stage.

Each call is fed seeded synthetic inputs (or the GPU's own upstream outputs),
and the oracle runs the same stage on exactly the same input values. Shapes
span several tiles with ragged tails, empty experts, single-row experts,
experts that span several 128-row tiles, and the degenerate sizes.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from synth.workloads import make_dense, make_expert, make_router, shard_weights
from tests.parity import (REL_FP8, assert_fp, check_route, errors, fp8_weight_f64, to_f64,
                          to_i64)

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def g():
    import gated_mlp_transformer_amd as mod
    return mod


def routing_ids(T, E, k, seed):
    r = np.random.default_rng(seed)
    ids = np.sort(np.stack([r.choice(E, size=k, replace=False) for _ in range(T)]), axis=1) \
        if T else np.zeros((0, k), dtype=np.int64)
    return torch.from_numpy(ids.astype(np.int32)).to(DEV)


# ------------------------------------------------------------------ rmsnorm --

@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("T,d", [(1, 64), (37, 256), (300, 4096), (5, 8192), (9, 6208),
                                 (64, 4096), (200, 2048), (257, 1024)])
def test_rmsnorm(g, dtype, T, d):
    x = synth.normal((T, d), name="t.rms.x", sub=d, dtype=dtype, device=DEV)
    if T > 2:
        x[0] = 0
        x[1] = 0.75
    gamma = synth.normal((d,), name="t.rms.g", std=0.1, mean=1.0, dtype=dtype, device=DEV)
    y = g.rmsnorm(x, gamma, 1e-5)
    torch.cuda.synchronize()
    ref = oracle.rmsnorm(to_f64(x), to_f64(gamma), 1e-5)
    tol = dict(rel=5e-3, max_abs=2e-2) if dtype == torch.bfloat16 else dict(rel=1e-6, max_abs=1e-5)
    assert_fp("rmsnorm", to_f64(y), ref, **tol)


@pytest.mark.parametrize("T,d", [(1, 128), (37, 384), (300, 4096), (5, 8192), (64, 1152),
                                 (64, 4096), (3, 512)])
def test_rmsnorm_quantize_fp8(g, T, d):
    """The fused pass writes rmsnorm's output bit for bit and, from it, the
    codes and scales of quantize_fp8_rows and of the oracle's quantiser."""
    x = synth.normal((T, d), name="t.rmsq.x", sub=d, device=DEV)
    if T > 2:
        x[0] = 0
        x[1, :128] = 0
    gamma = synth.normal((d,), name="t.rmsq.g", std=0.1, mean=1.0, device=DEV)
    y, q, sc = g.rmsnorm_quantize_fp8(x, gamma, 1e-5)
    y_ref = g.rmsnorm(x, gamma, 1e-5)
    q_ref, sc_ref = g.quantize_fp8_rows(y_ref)
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref)
    assert torch.equal(q, q_ref) and torch.equal(sc, sc_ref)
    oq, osc = oracle.quantize_rows(to_f64(y))
    assert np.array_equal(q.cpu().numpy(), oq)
    assert np.array_equal(sc.double().cpu().numpy(), osc)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_rmsnorm_rows_beyond_8192_are_unsupported(g, dtype):
    x = torch.zeros((2, 8256), dtype=dtype, device=DEV)
    gamma = torch.ones(8256, dtype=dtype, device=DEV)
    with pytest.raises(g.MoEFFNError) as e:
        g.rmsnorm(x, gamma, 1e-5)
    assert e.value.status == -2  # MF_EUNSUPPORTED, nothing enqueued


def test_rmsnorm_in_place(g):
    x = synth.normal((40, 512), name="t.rms.inplace", device=DEV)
    gamma = synth.normal((512,), name="t.rms.g2", std=0.1, mean=1.0, device=DEV)
    ref = oracle.rmsnorm(to_f64(x), to_f64(gamma), 1e-5)
    g.rmsnorm(x, gamma, 1e-5, out=x)
    torch.cuda.synchronize()
    assert_fp("rmsnorm in place", to_f64(x), ref)


# -------------------------------------------------------------------- route --

@pytest.mark.parametrize("T,d,E", [(1, 256, 8), (37, 256, 12), (300, 256, 64), (257, 512, 256),
                                   (64, 4096, 256), (1000, 1024, 200), (4096, 768, 9),
                                   (129, 2048, 100), (5000, 1024, 256), (2000, 2048, 160),
                                   (600, 768, 256), (256, 4096, 256), (200, 768, 9),
                                   (33, 1024, 162), (96, 8192, 31),
                                   # hidden sizes that are multiples of 64 only: the
                                   # few-token kernel, the split-K product with a
                                   # two-stage K tail, split and unsplit
                                   (64, 320, 256), (300, 320, 64), (4096, 4224, 256),
                                   (1000, 4160, 96),
                                   # many-token selection at prefill sizes (two
                                   # or four splits, a ragged last workgroup),
                                   # and a large T with E not a multiple of 4
                                   (8200, 1024, 256), (8192, 2048, 64), (9000, 512, 9)])
def test_route(g, T, d, E):
    r = make_router(T, d, E, seed=T + d + E, device=DEV)
    idx, w = g.moe_route(r["x"], g.pack_weights(r["w_r"]), r["bias"])
    torch.cuda.synchronize()
    ref_idx, ref_w, s, key, gap = oracle.route(to_f64(r["x"]), to_f64(r["w_r"]), to_f64(r["bias"]))
    n = check_route(to_i64(idx), key, gap, ref_idx)
    assert n <= max(2, T // 500)
    w_ref = oracle.route_weights(s, to_i64(idx))
    assert_fp("router weights", to_f64(w), w_ref, rel=1e-5, max_abs=1e-5)
    assert np.allclose(to_f64(w).sum(1), 1.0, atol=1e-5)


@pytest.mark.parametrize("T,E", [(200, 64), (600, 64), (1000, 256), (8200, 256)])
def test_route_exact_ties_pick_lower_index(g, T, E):
    # Only E/16 distinct router rows, each repeated 16 times, and a zero bias:
    # every token has exact ties inside its winning group, and the 8 lowest
    # ids of the group with the highest score must be chosen. T = 200 takes
    # the few-token kernels, the larger T the many-token selection.
    d = 256
    base = synth.normal((E // 16, d), name="t.tie.w", std=0.05, device=DEV)
    w_r = base.repeat_interleave(16, dim=0).contiguous()
    x = synth.normal((T, d), name="t.tie.x", device=DEV)
    bias = torch.zeros(E, dtype=torch.float32, device=DEV)
    idx, w = g.moe_route(x, g.pack_weights(w_r), bias)
    torch.cuda.synchronize()
    ref_idx, *_ = oracle.route(to_f64(x), to_f64(w_r), np.zeros(E))
    got = to_i64(idx)
    assert np.array_equal(got, ref_idx)
    assert np.allclose(to_f64(w), 1.0 / 8, atol=1e-7)


# ------------------------------------------------------------------ permute --

@pytest.mark.parametrize("T", [1, 255, 256, 257, 1000])
@pytest.mark.parametrize("eb,ec", [(0, 64), (16, 16), (63, 1), (3, 40)])
def test_permute(g, T, eb, ec):
    E, k, d = 64, 8, 128
    idx = routing_ids(T, E, k, seed=T * 7 + ec)
    x = synth.normal((T, d), name="t.perm.x", sub=T, device=DEV)
    res = g.moe_permute(idx, eb, ec, x)
    torch.cuda.synchronize()
    counts, offsets, src, inv, _ = oracle.permute(to_i64(idx), eb, ec)
    S = int(offsets[-1])
    assert np.array_equal(to_i64(res.counts), counts)
    assert np.array_equal(to_i64(res.offsets), offsets)
    assert np.array_equal(to_i64(res.src_token)[:S], src)
    assert np.array_equal(to_i64(res.inv_pos), inv)
    xp = res.x_perm[:S].cpu()
    assert torch.equal(xp, x.cpu()[torch.from_numpy(src)])


@pytest.mark.parametrize("T,E,k,eb,ec", [
    (20000, 256, 8, 0, 256),   # 79 blocks x 256 experts: count table scanned in its own pass
    (16384, 256, 8, 0, 256),   # 64 x 256: the largest table each block scans itself
    (700, 48, 6, 5, 30),       # k below 8
])
def test_permute_block_prefix_paths(g, T, E, k, eb, ec):
    idx = routing_ids(T, E, k, seed=T + k)
    res = g.moe_permute(idx, eb, ec, None)
    torch.cuda.synchronize()
    counts, offsets, src, inv, _ = oracle.permute(to_i64(idx), eb, ec)
    S = int(offsets[-1])
    assert np.array_equal(to_i64(res.counts), counts)
    assert np.array_equal(to_i64(res.offsets), offsets)
    assert np.array_equal(to_i64(res.src_token)[:S], src)
    assert np.array_equal(to_i64(res.inv_pos), inv)


def test_permute_f32_rows_and_index_only(g):
    T, E, k, d = 300, 32, 8, 20  # 80-byte f32 rows
    idx = routing_ids(T, E, k, seed=5)
    x = synth.normal((T, d), name="t.perm.f32", dtype=torch.float32, device=DEV)
    res = g.moe_permute(idx, 4, 20, x)
    res2 = g.moe_permute(idx, 4, 20, None)
    torch.cuda.synchronize()
    counts, offsets, src, inv, _ = oracle.permute(to_i64(idx), 4, 20)
    S = int(offsets[-1])
    assert torch.equal(res.x_perm[:S].cpu(), x.cpu()[torch.from_numpy(src)])
    for r in (res, res2):
        assert np.array_equal(to_i64(r.offsets), offsets)
        assert np.array_equal(to_i64(r.inv_pos), inv)


def test_permute_zero_tokens_writes_zero_counts(g):
    idx = torch.zeros((0, 8), dtype=torch.int32, device=DEV)
    counts = torch.full((16,), 7, dtype=torch.int32, device=DEV)
    offsets = torch.full((17,), 7, dtype=torch.int32, device=DEV)
    res = g.moe_permute(idx, 0, 16, None, counts=counts, offsets=offsets)
    torch.cuda.synchronize()
    assert res.counts.cpu().tolist() == [0] * 16
    assert res.offsets.cpu().tolist() == [0] * 17


@pytest.mark.parametrize("T,E,k,eb,ec,cap", [
    (64, 256, 8, 0, 256, 64),     # decode shape, one block, nothing dropped
    (0, 32, 8, 0, 16, 4),         # no tokens: zero counts
    (255, 64, 8, 3, 40, 255),
    (1000, 64, 8, 0, 64, 1000),   # several blocks
    (1000, 64, 6, 5, 30, 40),     # capacity drops, k below 8
    (300, 16, 8, 0, 16, 7),
])
def test_dispatch_masked(g, T, E, k, eb, ec, cap):
    idx = routing_ids(T, E, k, seed=T * 3 + cap) if T else torch.zeros((0, k), dtype=torch.int32, device=DEV)
    row_index = torch.full((ec * cap,), -7, dtype=torch.int32, device=DEV)
    res = g.moe_dispatch_masked(idx, eb, ec, cap, row_index=row_index)
    torch.cuda.synchronize()
    counts, rows, pos = oracle.dispatch_masked(to_i64(idx) if T else np.zeros((0, k)), eb, ec, cap)
    assert np.array_equal(to_i64(res.counts), counts)
    got_rows = to_i64(res.row_index)
    used = rows >= 0
    assert np.array_equal(got_rows[used], rows[used])
    assert (got_rows[~used] == -7).all()          # unused rows are not written
    if T:
        assert np.array_equal(to_i64(res.pos), pos)


@pytest.mark.parametrize("wdtype,counts,cap,d,f", [
    ("bf16", [0, 1, 130, 257, 3], 300, 256, 768),
    ("bf16", [1, 33, 65, 97], 128, 256, 256),
    ("fp8", [1, 3, 0, 17, 2, 16], 20, 256, 512),
    ("fp8", [16] * 6, 16, 512, 256),
])
def test_grouped_masked_matches_contiguous(g, wdtype, counts, cap, d, f):
    """The masked GEMMs over blocks of cap rows give, row for row, the
    contiguous GEMMs' results (same per-row arithmetic) and match the oracle.
    (fp8 weights: both layouts at decode-like row counts, where the contiguous
    call also takes the decode kernels; with more rows per expert it takes
    the tiled kernels, whose block sums are ordered differently.)"""
    ec = len(counts)
    S = int(sum(counts))
    W = _expert_weights(ec, d, f, wdtype, seed=S + cap)
    pw = [g.pack_weights(W[k_]) for k_ in ("w_gate", "w_up", "w_down")]
    src_rows = max(1, S // 2 + 5)
    x_src = synth.normal((src_rows, d), name="t.gm.x", sub=S, device=DEV)
    tok = synth.integers((S,), 0, src_rows, name="t.gm.tok", sub=S).to(torch.int32).to(DEV)
    # contiguous: rows grouped by expert; masked: the same rows at e*cap + r
    offsets = _offsets(counts)
    row_index = torch.full((ec * cap,), 0, dtype=torch.int32, device=DEV)
    off = offsets.cpu().numpy()
    for e in range(ec):
        row_index[e * cap:e * cap + counts[e]] = tok[off[e]:off[e + 1]]
    cnt = torch.tensor(counts, dtype=torch.int32, device=DEV)
    h_c = torch.empty((S + 1, f), dtype=torch.bfloat16, device=DEV)
    y_c = torch.empty((S + 1, d), dtype=torch.bfloat16, device=DEV)
    tok_pad = torch.cat([tok, tok[:1]])
    g.grouped_gate_up(x_src, offsets, pw[0], pw[1], W.get("s_gate"), W.get("s_up"),
                      row_index=tok_pad, h_out=h_c)
    g.grouped_down(h_c, offsets, pw[2], W.get("s_down"), y_perm=y_c)
    h_m = torch.full((ec * cap, f), float("nan"), dtype=torch.bfloat16, device=DEV)
    y_m = torch.full((ec * cap, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    g.grouped_gate_up_masked(x_src, row_index, cnt, cap, pw[0], pw[1], W.get("s_gate"),
                             W.get("s_up"), h_out=h_m)
    g.grouped_down_masked(h_m, cnt, cap, pw[2], W.get("s_down"), y_perm=y_m)
    torch.cuda.synchronize()
    xs = to_f64(x_src)
    for e in range(ec):
        a, b = off[e], off[e + 1]
        blk = slice(e * cap, e * cap + counts[e])
        assert torch.equal(h_m[blk], h_c[a:b]) and torch.equal(y_m[blk], y_c[a:b])
        # rows past the count in each block are not written
        assert torch.isnan(h_m[e * cap + counts[e]:(e + 1) * cap].float()).all()
        if b > a:
            wg, wu, wd = _oracle_weights(W, e, wdtype)
            xe = xs[to_i64(tok[a:b])]
            rel = 5e-3 if wdtype == "bf16" else REL_FP8
            assert_fp("H masked", to_f64(h_m[blk]), oracle.silu(xe @ wg) * (xe @ wu), rel=rel,
                      max_abs=None)
            assert_fp("Y masked", to_f64(y_m[blk]), to_f64(h_m[blk]) @ wd, rel=rel, max_abs=None)


# ------------------------------------------------------------------ packing --

def _pack_reference(w: np.ndarray, fp8: bool) -> np.ndarray:
    """The packed byte order, written out with numpy index arithmetic."""
    G, N, K = w.shape
    rb, cb = (16, 128) if fp8 else (32, 16)
    nb = -(-N // rb)
    wp = np.zeros((G, nb * rb, K), dtype=w.dtype)
    wp[:, :N] = w
    l = np.arange(64)
    if fp8:
        h = np.arange(2)
        b = np.arange(16)
        rows = (np.arange(nb)[:, None, None, None, None] * 16 + (l % 16)[None, None, None, :, None])
        cols = (np.arange(K // 128)[None, :, None, None, None] * 128 + 32 * (l // 16)[None, None, None, :, None]
                + 16 * h[None, None, :, None, None] + b[None, None, None, None, :])
        # [G, nb, kb, h, l, b] -> slab-major [kb, G, nb, h, l, b]
        return wp[:, rows, cols].transpose(2, 0, 1, 3, 4, 5)
    v = np.arange(8)
    rows = np.arange(nb)[:, None, None, None] * 32 + (l % 32)[None, None, :, None]
    cols = (np.arange(K // 16)[None, :, None, None] * 16 + 8 * (l // 32)[None, None, :, None]
            + v[None, None, None, :])
    return wp[:, rows, cols]


@pytest.mark.parametrize("fp8,G,N,K", [(False, 3, 96, 64), (False, 1, 12, 256), (False, 2, 300, 48),
                                       (True, 2, 48, 256), (True, 1, 20, 128)])
def test_pack_weights_is_the_documented_permutation(g, fp8, G, N, K):
    dt = torch.float8_e4m3fn if fp8 else torch.bfloat16
    w = synth.normal((G, N, K), name="t.pack", sub=N, dtype=torch.float32, device=DEV).to(dt)
    packed = g.pack_weights(w)
    torch.cuda.synchronize()
    view = np.uint8 if fp8 else np.uint16
    src = w.cpu().view(torch.uint8 if fp8 else torch.int16).numpy().view(view)
    ref = _pack_reference(src, fp8).reshape(-1)
    got = packed.data.cpu().numpy().view(view)
    assert got.shape == ref.shape and np.array_equal(got, ref)


@pytest.mark.parametrize("fp8,G,N,K", [(False, 3, 96, 64), (False, 1, 12, 256), (False, 2, 300, 48),
                                       (True, 2, 48, 256), (True, 1, 20, 128), (True, 3, 200, 384)])
def test_pack_weights_kn_equals_packing_the_transpose(g, fp8, G, N, K):
    # a [groups, K, N] source packs to the bytes of its [groups, N, K] transpose
    dt = torch.float8_e4m3fn if fp8 else torch.bfloat16
    w_kn = synth.normal((G, K, N), name="t.packkn", sub=N, dtype=torch.float32,
                        device=DEV).to(dt)
    w_nk = w_kn.transpose(1, 2).contiguous()
    a = g.pack_weights_kn(w_kn)
    b = g.pack_weights(w_nk)
    torch.cuda.synchronize()
    assert (a.groups, a.N, a.K) == (b.groups, b.N, b.K) == (G, N, K)
    assert torch.equal(a.data, b.data)
    view = np.uint8 if fp8 else np.uint16
    src = w_nk.cpu().view(torch.uint8 if fp8 else torch.int16).numpy().view(view)
    assert np.array_equal(a.data.cpu().numpy().view(view), _pack_reference(src, fp8).reshape(-1))


# ------------------------------------------------------------ grouped GEMM --

def _offsets(counts):
    return torch.tensor(np.concatenate([[0], np.cumsum(counts)]).astype(np.int32), device=DEV)


def _expert_weights(ec, d, f, wdtype, seed):
    ws = [make_expert(e, d, f, wdtype=wdtype, seed=seed, device=DEV, w_std=0.05)
          for e in range(ec)]
    out = {key: torch.stack([w[key] for w in ws]).contiguous() for key in ws[0]}
    return out


def _oracle_weights(W, e, wdtype):
    if wdtype == "bf16":
        return (to_f64(W["w_gate"][e]).T, to_f64(W["w_up"][e]).T, to_f64(W["w_down"][e]).T)
    return (fp8_weight_f64(W["w_gate"][e], W["s_gate"][e]),
            fp8_weight_f64(W["w_up"][e], W["s_up"][e]),
            fp8_weight_f64(W["w_down"][e], W["s_down"][e]))


@pytest.mark.parametrize("wdtype,counts,d,f", [
    ("bf16", [0, 1, 130, 257, 3], 256, 768),
    ("bf16", [200, 0, 0, 7], 512, 256),
    ("bf16", [1000], 256, 256),
    ("bf16", [0, 0, 0], 256, 256),
    ("bf16", [1, 33, 65, 97, 128, 129, 31, 32], 256, 256),   # every tail sub-tile count
    ("bf16", [300] * 5 + [0, 77, 513] + [300] * 8, 1024, 1024),  # > 256 tiles: several rounds
    # a last round at most half full runs its tiles as two row halves (with
    # 256 CUs, gate/up here: 264 tiles = one full round + 8 split; the case
    # above with every tail sub-tile count splits its down GEMM, one-sub-tile
    # chunks included, whose second half is empty)
    ("bf16", [300] * 66, 256, 256),
    ("fp8", [1, 3, 0, 17, 2, 16], 256, 512),
    ("fp8", [40], 512, 256),
    ("bf16", [(7 * e) % 5 for e in range(256)], 256, 256),   # the most groups (256)
    ("bf16", [3, 40], 8192, 256),     # the longest contraction: 256 K stages
    ("fp8", [3, 17, 2], 256, 8448),   # down contraction of 66 slabs: two scale chunks
    ("fp8", [9, 0, 4], 8448, 256),    # gate/up contraction of 66 slabs
    # many rows per expert: the tiled fp8-weight kernels (128-row tiles)
    ("fp8", [300, 0, 513, 1, 77, 256, 129], 512, 768),
    ("fp8", [330] * 4, 1024, 512),
    ("fp8", [200, 45], 8448, 256),    # gate/up contraction of 66 slabs, tiled
    ("fp8", [150], 256, 8448),        # down contraction of 66 slabs, tiled
    # sizes that are multiples of 64 (bf16) or 128 (fp8) only: K tails of two
    # stages (bf16) or an odd slab count (fp8), partial last n-tiles
    ("bf16", [0, 70, 129, 5], 320, 192),
    ("bf16", [33, 300], 448, 704),
    ("bf16", [100, 1], 384, 640),
    ("fp8", [3, 17, 0, 9], 384, 640),        # decode-shaped: 3 and 5 slabs
    ("fp8", [300, 45, 0, 129], 384, 640),    # tiled: 3 and 5 slabs, down n-tile of 128
    ("fp8", [3, 9], 8320, 128),              # 65 slabs: a second scale chunk of one slab
    ("fp8", [200, 45], 8320, 128),           # 65 slabs, tiled
])
@pytest.mark.parametrize("gather", [False, True])
def test_grouped_swiglu(g, wdtype, counts, d, f, gather):
    ec = len(counts)
    S = int(sum(counts))
    max_rows = S + 5
    W = _expert_weights(ec, d, f, wdtype, seed=S + d)
    offsets = _offsets(counts)
    h = torch.full((max_rows, f), float("nan"), dtype=torch.bfloat16, device=DEV)
    y = torch.full((max_rows, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    pw = [g.pack_weights(W[k_]) for k_ in ("w_gate", "w_up", "w_down")]
    if gather:
        # the GEMM gathers row r from x_src[row_index[r]]; out-of-range indices
        # are clamped into the source rows
        src_rows = max(1, S // 3 + 7)
        x_src = synth.normal((src_rows, d), name="t.gs.xsrc", sub=S, device=DEV)
        ri = synth.integers((max_rows,), 0, src_rows, name="t.gs.ri", sub=S).to(torch.int32)
        if S >= 2:
            ri[0], ri[S - 1] = -5, src_rows + 11
        ri = ri.to(DEV)
        x_perm = x_src[ri.long().clamp(0, src_rows - 1)].contiguous()
        g.grouped_swiglu(x_src, offsets, *pw, W.get("s_gate"), W.get("s_up"), W.get("s_down"),
                         row_index=ri, h_work=h, y_perm=y)
    else:
        x_perm = synth.normal((max_rows, d), name="t.gs.x", sub=S, device=DEV)
        g.grouped_swiglu(x_perm, offsets, *pw, W.get("s_gate"),
                         W.get("s_up"), W.get("s_down"), h_work=h, y_perm=y)
    torch.cuda.synchronize()
    # rows past the last expert are never written
    assert torch.isnan(h[S:].float()).all() and torch.isnan(y[S:].float()).all()
    if S == 0:
        return
    xp = to_f64(x_perm)
    off = offsets.cpu().numpy()
    h_ref = np.zeros((S, f))
    h_gpu = to_f64(h[:S])
    y_from_gpu_h = np.zeros((S, d))
    for e in range(ec):
        a, b = off[e], off[e + 1]
        if b > a:
            wg, wu, wd = _oracle_weights(W, e, wdtype)
            h_ref[a:b] = oracle.silu(xp[a:b] @ wg) * (xp[a:b] @ wu)
            y_from_gpu_h[a:b] = h_gpu[a:b] @ wd
    y_ref = oracle.experts(xp[:S], off, lambda e: _oracle_weights(W, e, wdtype))
    rel = 5e-3 if wdtype == "bf16" else REL_FP8
    assert_fp("H", h_gpu, h_ref, rel=rel, max_abs=None)
    # down GEMM alone, on the GPU's own H
    assert_fp("Y from GPU H", to_f64(y[:S]), y_from_gpu_h, rel=rel, max_abs=None)
    assert_fp("Y_perm", to_f64(y[:S]), y_ref, rel=rel, max_abs=None)


# ------------------------------------------------------------------ combine --

@pytest.mark.parametrize("out_dtype,with_residual", [(torch.bfloat16, False),
                                                     (torch.float32, False),
                                                     (torch.bfloat16, True),
                                                     (torch.float32, True)])
# launch shapes: two vectors per thread (<= 1024 tokens; d = 4096 in one pass,
# and 1088 with a ragged second vector), one vector per thread (> 1024 tokens)
@pytest.mark.parametrize("T,d", [(300, 256), (64, 4096), (5, 1088), (1500, 512)])
def test_combine(g, out_dtype, with_residual, T, d):
    E, k = 64, 8
    idx = routing_ids(T, E, k, seed=11 + T)
    res = g.moe_permute(idx, 8, 24, None)
    S_max = T * k
    y_perm = synth.normal((S_max, d), name="t.comb.y", device=DEV)
    w = torch.rand((T, k), generator=torch.Generator(DEV).manual_seed(3), device=DEV) + 0.05
    w = (w / w.sum(1, keepdim=True)).float().contiguous()
    r = synth.normal((T, d), name="t.comb.r", dtype=out_dtype, device=DEV) if with_residual else None
    out = g.moe_combine(y_perm, res.inv_pos, w, out_dtype=out_dtype, residual=r)
    torch.cuda.synchronize()
    ref = oracle.combine(to_f64(y_perm), to_i64(res.inv_pos), to_f64(w),
                         residual=None if r is None else to_f64(r))
    none_local = np.all(to_i64(res.inv_pos) < 0, axis=1)
    if T >= 300:  # enough tokens that both kinds occur
        assert none_local.any() and (~none_local).any()
    got = to_f64(out)
    # no local expert: the output is the residual (or 0) exactly
    assert np.all(got[none_local] == (0 if r is None else to_f64(r)[none_local]))
    tol = dict(rel=5e-3, max_abs=2e-2) if out_dtype == torch.bfloat16 else dict(rel=1e-6, max_abs=1e-5)
    assert_fp("combine", got, ref, **tol)


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("T,d", [(300, 256), (64, 4096)])
def test_combine_out_aliases_residual(g, out_dtype, T, d):
    """out may be the residual buffer itself (the residual stream updated in
    place): the result equals the combine into a separate buffer, bit for bit."""
    E, k = 64, 8
    idx = routing_ids(T, E, k, seed=12)
    res = g.moe_permute(idx, 0, 40, None)
    y_perm = synth.normal((T * k, d), name="t.comb.alias.y", device=DEV)
    w = torch.rand((T, k), generator=torch.Generator(DEV).manual_seed(4), device=DEV) + 0.05
    w = (w / w.sum(1, keepdim=True)).float().contiguous()
    r = synth.normal((T, d), name="t.comb.alias.r", dtype=out_dtype, device=DEV)
    sep = g.moe_combine(y_perm, res.inv_pos, w, out_dtype=out_dtype, residual=r)
    stream_buf = r.clone()
    same = g.moe_combine(y_perm, res.inv_pos, w, out_dtype=out_dtype, residual=stream_buf,
                         out=stream_buf)
    torch.cuda.synchronize()
    assert same.data_ptr() == stream_buf.data_ptr()
    assert torch.equal(sep, stream_buf)
    ref = oracle.combine(to_f64(y_perm), to_i64(res.inv_pos), to_f64(w), residual=to_f64(r))
    tol = dict(rel=5e-3, max_abs=2e-2) if out_dtype == torch.bfloat16 else dict(rel=1e-6, max_abs=1e-5)
    assert_fp("combine in place", to_f64(stream_buf), ref, **tol)


# ------------------------------------------------------------- TP shards --

def test_tp_shard_f32_dense_config(g):
    # X 16x64, W_gate/W_up 64x256, W_down 256x64 (fp32), p = 4 shards.
    D = make_dense(16, 64, 256, dtype=torch.float32, device=DEV)
    x = D["x"]
    wg, wu, wd = (to_f64(D[k_]) for k_ in ("w_gate", "w_up", "w_down"))
    xf = to_f64(x)
    parts, hs = [], []
    for i in range(4):
        sg, su, sd = shard_weights(D["w_gate"], D["w_up"], D["w_down"], 4, i)
        p_, h_ = g.tp_shard_mlp(x, sg, su, sd)
        parts.append(p_)
        hs.append(h_)
    torch.cuda.synchronize()
    for i in range(4):
        ref = oracle.tp_shard_mlp(xf, wg.T, wu.T, wd.T, 4, i)
        assert_fp(f"partial {i}", to_f64(parts[i]), ref, rel=1e-5, max_abs=1e-6)
    full = oracle.swiglu(xf, wg.T, wu.T, wd.T)
    assert_fp("sum of partials", sum(to_f64(p_) for p_ in parts), full, rel=1e-5, max_abs=1e-6)
    h_full = oracle.silu(xf @ wg.T) * (xf @ wu.T)
    assert_fp("concat of H shards", np.concatenate([to_f64(h_) for h_ in hs], axis=1), h_full,
              rel=1e-5, max_abs=1e-6)


@pytest.mark.parametrize("T,d,f,p", [(300, 256, 512, 2), (129, 512, 256, 1), (1, 256, 256, 1),
                                     (300, 320, 640, 2), (77, 192, 320, 1)])
def test_tp_shard_bf16(g, T, d, f, p):
    D = make_dense(T, d, f, dtype=torch.bfloat16, device=DEV, w_std=0.05)
    xf = to_f64(D["x"])
    wg, wu, wd = (to_f64(D[k_]).T for k_ in ("w_gate", "w_up", "w_down"))
    total = 0
    for i in range(p):
        sg, su, sd = shard_weights(D["w_gate"], D["w_up"], D["w_down"], p, i)
        part, h = g.tp_shard_mlp(D["x"], *(g.pack_weights(w_) for w_ in (sg, su, sd)))
        torch.cuda.synchronize()
        ref = oracle.tp_shard_mlp(xf, wg, wu, wd, p, i)
        assert_fp(f"partial {i}", to_f64(part), ref)
        total = total + to_f64(part)
    assert_fp("sum of partials", total, oracle.swiglu(xf, wg, wu, wd))


# ------------------------------------------------------- binding argument checks --

def test_binding_rejects_wrong_buffers(g):
    """Undersized outputs, wrong index dtypes and missing fp8 scales are refused
    before anything is enqueued (the kernels would otherwise run past them)."""
    T, d, f, E = 64, 256, 256, 4
    x = torch.zeros((T, d), dtype=torch.bfloat16, device=DEV)
    w = g.pack_weights(torch.zeros((E, f, d), dtype=torch.bfloat16, device=DEV))
    wd = g.pack_weights(torch.zeros((E, d, f), dtype=torch.bfloat16, device=DEV))
    offsets = torch.tensor([0, 16, 32, 48, 64], dtype=torch.int32, device=DEV)
    with pytest.raises(ValueError, match="h_out"):
        g.grouped_gate_up(x, offsets, w, w, h_out=torch.empty((T - 1, f), dtype=torch.bfloat16,
                                                             device=DEV))
    with pytest.raises(ValueError, match="offsets"):
        g.grouped_gate_up(x, offsets.long(), w, w)
    with pytest.raises(ValueError, match="y_perm"):
        g.grouped_down(torch.zeros((T, f), dtype=torch.bfloat16, device=DEV), offsets, wd,
                       y_perm=torch.empty((T, d - 64), dtype=torch.bfloat16, device=DEV))
    w8 = g.pack_weights(torch.zeros((E, f, d), dtype=torch.float8_e4m3fn, device=DEV))
    with pytest.raises(ValueError, match="need s_gate"):
        g.grouped_gate_up(x, offsets, w8, w8)
    idx = torch.zeros((T, 8), dtype=torch.int32, device=DEV)
    with pytest.raises(ValueError, match="inv_pos"):
        g.moe_permute(idx, 0, E, inv_pos=torch.empty((T, 4), dtype=torch.int32, device=DEV))
    with pytest.raises(ValueError, match="out"):
        g.moe_combine(torch.zeros((T * 8, d), dtype=torch.bfloat16, device=DEV), idx,
                      torch.zeros((T, 8), dtype=torch.float32, device=DEV),
                      out=torch.empty((T // 2, d), dtype=torch.bfloat16, device=DEV))
    torch.cuda.synchronize()


def test_zero_tokens_through_every_call(g):
    """T = 0 is a valid call everywhere: nothing is launched and every output
    is an empty tensor of the right shape (zero-size buffers may be NULL)."""
    d, f, E, ec = 256, 256, 16, 4
    bf = torch.bfloat16
    x = torch.empty((0, d), dtype=bf, device=DEV)
    v = g.rmsnorm(x, torch.ones(d, dtype=bf, device=DEV))
    idx, w = g.moe_route(v, g.pack_weights(torch.zeros((E, d), dtype=bf, device=DEV)),
                         torch.zeros(E, dtype=torch.float32, device=DEV))
    res = g.moe_permute(idx, 0, ec)
    wg, wu = (g.pack_weights(torch.zeros((ec, f, d), dtype=bf, device=DEV)) for _ in range(2))
    wd = g.pack_weights(torch.zeros((ec, d, f), dtype=bf, device=DEV))
    h = g.grouped_gate_up(v, res.offsets, wg, wu, row_index=res.src_token)
    y = g.grouped_down(h, res.offsets, wd)
    out = g.moe_combine(y, res.inv_pos, w)
    q, sc = g.quantize_fp8_rows(x)
    shards = [g.pack_weights(torch.zeros(s, dtype=bf, device=DEV)) for s in ((f, d), (f, d), (d, f))]
    part, hw = g.tp_shard_mlp(x, *shards)
    torch.cuda.synchronize()
    assert v.shape == (0, d) and idx.shape == (0, 8) and w.shape == (0, 8)
    assert torch.equal(res.counts.cpu(), torch.zeros(ec, dtype=torch.int32))
    assert torch.equal(res.offsets.cpu(), torch.zeros(ec + 1, dtype=torch.int32))
    assert h.shape == (0, f) and y.shape == (0, d) and out.shape == (0, d)
    assert q.shape == (0, d) and sc.shape == (0, d // 128)
    assert part.shape == (0, d) and hw.shape == (0, f)
