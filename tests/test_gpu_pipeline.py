"""GPU parity of the whole FFN sub-block, small and at the workloads' full sizes.

Each run goes RMSNorm -> router -> permutation -> grouped gated MLP -> combine
through the C ABI (MoEFFNLayer) and is checked stage by stage against the
fp64 oracle on the very inputs each stage received, then end to end from the
raw inputs:

  * V = RMSNorm(x): floating-point tolerance.
  * routing, on the GPU's V (the router's own input): expert ids bit-exact
    except for tokens whose 8th/9th biased-score gap is below 1e-6 (then any
    valid top-8 within that band is accepted); weights within tolerance.
  * permutation, on the GPU's ids: counts, offsets, src_token, inv_pos
    bit-exact (the layer permutes indices only).
  * expert GEMMs, on the rows V[src_token] that the gate/up GEMM gathers in
    its A load, and on the GPU's H: tolerance on H and Y_perm.
  * combine, on the GPU's Y_perm: tolerance.
  * end to end: the oracle's fp64 sub-block from the raw x with the routed
    sets the GPU chose (accepted above): tolerance on the output.

Every size is checked in full: every token, every row of H and Y_perm and
every column. The oracle's end-to-end pass visits each local expert once, and
the stage references of that expert's rows are computed from the same fp64
weights in that visit.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from synth.workloads import WORKLOADS, make_dense, make_moe
from tests.parity import (REL_FP8, assert_fp, check_route, fp8_weight_f64, to_f64, to_i64)

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def g():
    import gated_mlp_transformer_amd as mod
    return mod


def build_layer(g, inp, T, d, f, e_begin, act_fp8=False):
    return g.MoEFFNLayer(T=T, d=d, f=f, w_r=inp["w_r"], bias=inp["bias"], gamma=inp.get("gamma"),
                         w_gate=inp["w_gate"], w_up=inp["w_up"], w_down=inp["w_down"],
                         e_begin=e_begin, s_gate=inp.get("s_gate"), s_up=inp.get("s_up"),
                         s_down=inp.get("s_down"), act_fp8=act_fp8)


def expert_f64(inp, e, wdtype):
    """Expert e's (W_gate, W_up, W_down) in the pages' orientation, fp64."""
    if wdtype == "bf16":
        return tuple(to_f64(inp[k][e]).T for k in ("w_gate", "w_up", "w_down"))
    return (fp8_weight_f64(inp["w_gate"][e], inp["s_gate"][e]),
            fp8_weight_f64(inp["w_up"][e], inp["s_up"][e]),
            fp8_weight_f64(inp["w_down"][e], inp["s_down"][e]))


def check_layer(g, layer, inp, T, d, f, E, eb, ec, wdtype, *, masked=None):
    """Stage-by-stage and end-to-end parity of one forward pass (see module doc),
    on every token, row and column.

    With the layer's fp8 activations (block-fp8 prefill variant) the GEMMs are
    checked on the GPU's own codes: gate/up on the quantised V rows it
    gathers, down on the quantised H (whose codes are compared bit for bit
    with the oracle's quantiser on the GPU's H); end to end against the
    oracle's fp8-activation sub-block. A layer without gamma runs the router
    on x itself (no RMSNorm), and so does the oracle. ``masked``, a twin layer
    with the masked (fixed-capacity) layout on the same inputs, is checked
    against the same oracle values: its dispatch integers, its H and Y rows at
    the slots' block rows, and its output."""
    a8 = getattr(layer, "act_fp8", False)
    norm = layer.gamma is not None
    rel = 5e-3 if wdtype == "bf16" else REL_FP8
    out = layer(inp["x"])
    out_m = masked(inp["x"]) if masked is not None else None
    torch.cuda.synchronize()
    x = to_f64(inp["x"])
    gamma = to_f64(inp["gamma"]) if norm else None

    # RMSNorm
    if norm:
        v_gpu = to_f64(layer.v)
        assert_fp("V", v_gpu, oracle.rmsnorm(x, gamma, 1e-5))
    else:
        v_gpu = x

    # router on the GPU's V
    w_r, bias = to_f64(inp["w_r"]), to_f64(inp["bias"])
    ref_idx, _, s, key, gap = oracle.route(v_gpu, w_r, bias)
    gpu_idx = to_i64(layer.idx)
    n_near = check_route(gpu_idx, key, gap, ref_idx)
    assert n_near <= max(2, T // 1000)
    assert_fp("router w", to_f64(layer.topk_w), oracle.route_weights(s, gpu_idx), rel=1e-5,
              max_abs=1e-5)

    # permutation on the GPU's ids
    counts, offsets, src, inv, _ = oracle.permute(gpu_idx, eb, ec)
    S = int(offsets[-1])
    assert np.array_equal(to_i64(layer.counts), counts)
    assert np.array_equal(to_i64(layer.offsets), offsets)
    assert np.array_equal(to_i64(layer.src_token)[:S], src)
    assert np.array_equal(to_i64(layer.inv_pos), inv)

    # the GEMMs' own inputs: the rows V[src_token] the gate/up GEMM gathers,
    # and the GPU's H for the down GEMM
    if a8:
        vq = layer.vq.cpu().numpy().astype(np.uint8)
        # V's fp8 codes and scales are the quantiser's on the GPU's bf16 V
        vq_ref, vs_ref = oracle.quantize_rows(v_gpu)
        assert np.array_equal(vq, vq_ref)
        assert np.array_equal(layer.vs.double().cpu().numpy(), vs_ref)
        xp = oracle.dequant_rows(vq[src], layer.vs.double().cpu().numpy()[src])
        hq_ref, hs_ref = oracle.quantize_rows(to_f64(layer.h[:S]))
        assert np.array_equal(layer.hq[:S].cpu().numpy().astype(np.uint8), hq_ref)
        assert np.array_equal(layer.hs[:S].double().cpu().numpy(), hs_ref)
        h_in = oracle.dequant_rows(hq_ref, hs_ref)
        rel_gemm = 5e-3   # each GEMM on its fp8 operands: bf16 output rounding only
    else:
        xp = v_gpu[src]
        h_in = to_f64(layer.h[:S])
        rel_gemm = rel
    h_ref = np.zeros((S, f))
    y_ref = np.zeros((S, d))

    def weights(e):
        # The oracle's end-to-end pass asks for each local expert that holds
        # rows once, in ascending order; the stage references of that expert's
        # rows are computed here from the same fp64 weights.
        wg, wu, wd = expert_f64(inp, e, wdtype)
        a, b = int(offsets[e]), int(offsets[e + 1])
        h_ref[a:b] = oracle.silu(xp[a:b] @ wg) * (xp[a:b] @ wu)
        y_ref[a:b] = h_in[a:b] @ wd
        return wg, wu, wd

    # end to end from the raw inputs, with the GPU's accepted routed sets
    ref = oracle.moe_ffn(x, gamma, w_r, bias, weights, eb, ec, idx=gpu_idx, act_fp8=a8,
                         norm=norm)
    assert np.array_equal(ref["offsets"], offsets)
    h_gpu = to_f64(layer.h[:S])
    y_gpu = to_f64(layer.y_perm[:S])
    assert_fp("H", h_gpu, h_ref, rel=rel_gemm, max_abs=None)
    assert_fp("Y_perm (from GPU H)", y_gpu, y_ref, rel=rel_gemm, max_abs=None)

    # combine on the GPU's Y_perm
    out_gpu = to_f64(out)
    comb = oracle.combine(to_f64(layer.y_perm), inv, to_f64(layer.topk_w))
    assert_fp("combine", out_gpu, comb)

    max_abs = 2e-2 if wdtype == "bf16" else None
    assert_fp("FFN output (end to end)", out_gpu, ref["out"], rel=rel, max_abs=max_abs)

    if masked is not None:
        cap = masked.cap
        m_counts, m_rows, m_pos = oracle.dispatch_masked(to_i64(masked.idx), eb, ec, cap)
        assert np.array_equal(to_i64(masked.idx), gpu_idx)
        assert np.array_equal(to_i64(masked.counts), m_counts)
        assert np.array_equal(to_i64(masked.inv_pos), m_pos)
        used = m_rows >= 0
        assert np.array_equal(to_i64(masked.row_index)[used], m_rows[used])
        local = inv >= 0
        assert np.array_equal(m_pos >= 0, local)  # cap >= T: no slot dropped
        # slot (t, j) lives at contiguous row inv[t, j] and masked row m_pos[t, j]
        hm = to_f64(masked.h)[m_pos[local]]
        ym = to_f64(masked.y_perm)[m_pos[local]]
        assert_fp("masked H", hm, h_ref[inv[local]], rel=rel_gemm, max_abs=None)
        # its H rows are the contiguous layer's (same rows, same kernels), so
        # y_ref (computed from the contiguous H) is its down GEMM's reference
        assert np.array_equal(hm, h_gpu[inv[local]])
        assert_fp("masked Y (from its H)", ym, y_ref[inv[local]], rel=rel_gemm, max_abs=None)
        assert_fp("masked FFN output (end to end)", to_f64(out_m), ref["out"], rel=rel,
                  max_abs=max_abs)
    return dict(S=S, near_ties=n_near)


@pytest.mark.parametrize("wdtype", ["bf16", "fp8"])
@pytest.mark.parametrize("T,eb,ec", [(200, 16, 16), (77, 0, 64), (1, 60, 4)])
def test_moe_ffn_small(g, wdtype, T, eb, ec):
    d, f, E = 256, 256, 64
    inp = make_moe(T, d, f, E, eb, ec, wdtype=wdtype, seed=T + ec, device=DEV)
    layer = build_layer(g, inp, T, d, f, eb)
    check_layer(g, layer, inp, T, d, f, E, eb, ec, wdtype)


@pytest.mark.parametrize("T,eb,ec", [(200, 16, 16), (77, 0, 64), (1, 60, 4)])
def test_moe_ffn_small_fp8_activations(g, T, eb, ec):
    d, f, E = 256, 256, 64
    inp = make_moe(T, d, f, E, eb, ec, wdtype="fp8", seed=T + ec + 3, device=DEV)
    layer = build_layer(g, inp, T, d, f, eb, act_fp8=True)
    check_layer(g, layer, inp, T, d, f, E, eb, ec, "fp8")


@pytest.mark.parametrize("wdtype,d,f,act_fp8", [("bf16", 320, 192, False),
                                                ("fp8", 384, 640, False),
                                                ("fp8", 384, 640, True)])
def test_moe_ffn_sizes_beyond_multiples_of_256(g, wdtype, d, f, act_fp8):
    # d, f multiples of 64 (bf16) or 128 (fp8) only, end to end
    T, E, eb, ec = 150, 64, 8, 16
    inp = make_moe(T, d, f, E, eb, ec, wdtype=wdtype, seed=d + f, device=DEV)
    layer = build_layer(g, inp, T, d, f, eb, act_fp8=act_fp8)
    check_layer(g, layer, inp, T, d, f, E, eb, ec, wdtype)


def test_moe_ffn_forced_empty_and_single_expert(g):
    # A bias of -10 on every local expert but one: the others get no tokens.
    T, d, f, E, eb, ec = 300, 256, 256, 32, 8, 8
    inp = make_moe(T, d, f, E, eb, ec, seed=5, device=DEV)
    inp["bias"][eb:eb + ec] = -10.0
    inp["bias"][eb + 3] = 5.0   # every token picks local expert eb+3
    layer = build_layer(g, inp, T, d, f, eb)
    res = check_layer(g, layer, inp, T, d, f, E, eb, ec, "bf16")
    assert res["S"] == T
    counts = to_i64(layer.counts)
    assert counts[3] == T and counts.sum() == T


def test_workload_router_4096tok(g):
    """Router + index-only permutation, 4096 tokens, E = 256, full parity."""
    spec = WORKLOADS["router_4096tok_E256"]
    from synth.workloads import make_router
    r = make_router(spec["T"], spec["d"], spec["E"], device=DEV)
    idx, w = g.moe_route(r["x"], g.pack_weights(r["w_r"]), r["bias"])
    res = g.moe_permute(idx, 0, spec["E"], None)
    torch.cuda.synchronize()
    ref_idx, _, s, key, gap = oracle.route(to_f64(r["x"]), to_f64(r["w_r"]), to_f64(r["bias"]))
    n = check_route(to_i64(idx), key, gap, ref_idx)
    assert n <= 4
    assert_fp("router w", to_f64(w), oracle.route_weights(s, to_i64(idx)), rel=1e-5, max_abs=1e-5)
    counts, offsets, src, inv, _ = oracle.permute(to_i64(idx), 0, spec["E"])
    assert counts.sum() == spec["T"] * 8
    assert np.array_equal(to_i64(res.offsets), offsets)
    assert np.array_equal(to_i64(res.src_token), src)
    assert np.array_equal(to_i64(res.inv_pos), inv)


def test_workload_dense_shard_4096(g):
    """RMSNorm + one bf16 TP shard (4096 x 4096, f_s 2048): every row and column."""
    spec = WORKLOADS["norm_tp_shard_bf16_4096"]
    T, d, f = spec["T"], spec["d"], spec["f"]
    D = make_dense(T, d, f, dtype=torch.bfloat16, norm=True, device=DEV)
    v = g.rmsnorm(D["x"], D["gamma"], 1e-5)
    part, h = g.tp_shard_mlp(v, *(g.pack_weights(D[k]) for k in ("w_gate", "w_up", "w_down")))
    torch.cuda.synchronize()
    x = to_f64(D["x"])
    assert_fp("V", to_f64(v), oracle.rmsnorm(x, to_f64(D["gamma"]), 1e-5))
    vg = to_f64(v)
    wg, wu, wd = (to_f64(D[k]).T for k in ("w_gate", "w_up", "w_down"))
    assert_fp("H", to_f64(h), oracle.silu(vg @ wg) * (vg @ wu), max_abs=None)
    # the down GEMM on the GPU's H, then the shard end to end from the GPU's V
    assert_fp("partial (from GPU H)", to_f64(part), to_f64(h) @ wd, max_abs=None)
    assert_fp("partial", to_f64(part), oracle.tp_shard_mlp(vg, wg, wu, wd, 1, 0))


@pytest.fixture(scope="module")
def prefill(g):
    spec = WORKLOADS["moe_prefill_8192tok_32exp_bf16"]
    inp = make_moe(spec["T"], spec["d"], spec["f"], spec["E"], spec["e_begin"], spec["e_count"],
                   wdtype="bf16", zipf=spec["zipf"], device=DEV)
    layer = build_layer(g, inp, spec["T"], spec["d"], spec["f"], spec["e_begin"])
    return spec, inp, layer


def test_workload_prefill_8192tok(g, prefill):
    """The prefill workload in full: every token, row and column."""
    spec, inp, layer = prefill
    res = check_layer(g, layer, inp, spec["T"], spec["d"], spec["f"], spec["E"],
                      spec["e_begin"], spec["e_count"], "bf16")
    counts = to_i64(layer.counts)
    # the skewed bias gives the local experts uneven loads (0.5x to 3x the mean)
    assert counts.max() > 2 * counts.mean() and counts.min() > 0
    assert res["S"] == counts.sum()


def test_workload_prefill_8192tok_without_rmsnorm(g, prefill):
    """The same workload with the router and experts fed x directly (no
    RMSNorm stage): the sub-block as the workload list states it."""
    spec, inp, _ = prefill
    no_norm = dict(inp)
    no_norm["gamma"] = None
    layer = build_layer(g, no_norm, spec["T"], spec["d"], spec["f"], spec["e_begin"])
    assert layer.v is None
    res = check_layer(g, layer, no_norm, spec["T"], spec["d"], spec["f"], spec["E"],
                      spec["e_begin"], spec["e_count"], "bf16")
    assert res["S"] == to_i64(layer.counts).sum()


def test_prefill_is_deterministic(g, prefill):
    spec, inp, layer = prefill
    a = layer(inp["x"]).clone()
    b = layer(inp["x"]).clone()
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def _masked_twin(g, inp, T, d, f, eb, cap=None):
    return g.MoEFFNLayer(T=T, d=d, f=f, w_r=inp["w_r"], bias=inp["bias"], gamma=inp.get("gamma"),
                         w_gate=inp["w_gate"], w_up=inp["w_up"], w_down=inp["w_down"],
                         e_begin=eb, s_gate=inp.get("s_gate"), s_up=inp.get("s_up"),
                         s_down=inp.get("s_down"), layout="masked", cap=cap)


def test_workload_decode_64tok_fp8(g):
    """The decode workload in full (all 64 tokens, every row and column), in
    the contiguous layout and in the masked layout, each against the oracle."""
    spec = WORKLOADS["moe_decode_64tok_256exp_fp8"]
    inp = make_moe(spec["T"], spec["d"], spec["f"], spec["E"], spec["e_begin"], spec["e_count"],
                   wdtype="fp8", device=DEV)
    layer = build_layer(g, inp, spec["T"], spec["d"], spec["f"], spec["e_begin"])
    masked = _masked_twin(g, inp, spec["T"], spec["d"], spec["f"], spec["e_begin"])
    res = check_layer(g, layer, inp, spec["T"], spec["d"], spec["f"], spec["E"],
                      spec["e_begin"], spec["e_count"], "fp8", masked=masked)
    assert res["S"] == 64 * 8
    assert int(masked.counts.sum()) == spec["T"] * 8


def test_workload_prefill_8192tok_fp8_activations(g):
    """The block-fp8 prefill variant in full: every token, row and column."""
    spec = WORKLOADS["moe_prefill_8192tok_32exp_fp8act"]
    inp = make_moe(spec["T"], spec["d"], spec["f"], spec["E"], spec["e_begin"], spec["e_count"],
                   wdtype="fp8", zipf=spec["zipf"], device=DEV)
    layer = build_layer(g, inp, spec["T"], spec["d"], spec["f"], spec["e_begin"], act_fp8=True)
    res = check_layer(g, layer, inp, spec["T"], spec["d"], spec["f"], spec["E"],
                      spec["e_begin"], spec["e_count"], "fp8")
    assert res["S"] == to_i64(layer.counts).sum()


def test_workload_prefill_8192tok_fp8_weights(g):
    """The prefill workload with block-fp8 weights and bf16 activations (190
    to 956 rows per expert: the tiled fp8-weight GEMMs), in full."""
    spec = WORKLOADS["moe_prefill_8192tok_32exp_fp8w"]
    inp = make_moe(spec["T"], spec["d"], spec["f"], spec["E"], spec["e_begin"], spec["e_count"],
                   wdtype="fp8", zipf=spec["zipf"], device=DEV)
    layer = build_layer(g, inp, spec["T"], spec["d"], spec["f"], spec["e_begin"])
    res = check_layer(g, layer, inp, spec["T"], spec["d"], spec["f"], spec["E"],
                      spec["e_begin"], spec["e_count"], "fp8")
    counts = to_i64(layer.counts)
    assert counts.min() >= 128 and res["S"] == counts.sum()


@pytest.mark.parametrize("wdtype,T,eb,ec", [("bf16", 200, 16, 16), ("fp8", 64, 0, 64)])
def test_masked_layout_equals_contiguous(g, wdtype, T, eb, ec):
    """The masked (fixed-capacity) layout changes where rows live, not their
    arithmetic: both layers are checked against the oracle, and the masked
    output is bit-identical to the contiguous one."""
    d, f, E = 256, 256, 64
    inp = make_moe(T, d, f, E, eb, ec, wdtype=wdtype, seed=T + ec + 9, device=DEV)
    contig = build_layer(g, inp, T, d, f, eb)
    masked = _masked_twin(g, inp, T, d, f, eb)
    check_layer(g, contig, inp, T, d, f, E, eb, ec, wdtype, masked=masked)
    a = contig(inp["x"]).clone()
    b = masked(inp["x"]).clone()
    torch.cuda.synchronize()
    assert torch.equal(a, b)
