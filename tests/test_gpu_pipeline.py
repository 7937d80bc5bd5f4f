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

At full sizes the floating-point stages are checked on sampled rows or
columns the oracle computes one by one (tokens and columns are independent).
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


def weight_rows_f64(inp, key, e, rows, wdtype):
    """Rows `rows` of expert e's [out, in] weight `key`, fp64 (fp8: dequantised)."""
    if wdtype == "bf16":
        return to_f64(inp[key][e][rows])
    out = []
    for r in rows:  # dequantise the 128-row block holding each row (cached per block)
        b = r // 128
        if not out or out[-1][0] != b:
            q = inp[key][e][b * 128:(b + 1) * 128]
            s = inp["s_" + key[2:]][e][b:b + 1]
            out.append((b, fp8_weight_f64(q, s).T, []))  # block as [128, K]
        out[-1][2].append(out[-1][1][r - b * 128])
    return np.stack([row for _, _, rs in out for row in rs])


def check_layer(g, layer, inp, T, d, f, E, eb, ec, wdtype, *, token_sample=None,
                col_sample=None, e2e_tokens=None):
    """Stage-by-stage and end-to-end parity of one forward pass (see module doc).

    With the layer's fp8 activations (block-fp8 prefill variant) the GEMMs are
    checked on the GPU's own codes: gate/up on the quantised V rows it
    gathers, down on the quantised H (whose codes are compared bit for bit
    with the oracle's quantiser on the GPU's H); end to end against the
    oracle's fp8-activation sub-block."""
    a8 = getattr(layer, "act_fp8", False)
    rel = 5e-3 if wdtype == "bf16" else REL_FP8
    out = layer(inp["x"])
    torch.cuda.synchronize()
    x = to_f64(inp["x"])
    rows = np.arange(T) if token_sample is None else np.asarray(token_sample)

    # RMSNorm
    v_gpu = to_f64(layer.v)
    assert_fp("V", v_gpu[rows], oracle.rmsnorm(x[rows], to_f64(inp["gamma"]), 1e-5))

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

    # expert GEMMs on the gathered rows V[src_token] (H) and the GPU's H
    # (Y_perm): all rows, sampled columns
    if a8:
        vq = layer.vq.cpu().numpy().astype(np.uint8)
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
    h_gpu = to_f64(layer.h[:S])
    y_gpu = to_f64(layer.y_perm[:S])
    hc = np.arange(f) if col_sample is None else np.asarray(col_sample)
    yc = np.arange(d) if col_sample is None else np.asarray(col_sample)
    h_ref = np.zeros((S, len(hc)))
    y_ref = np.zeros((S, len(yc)))
    for e in range(ec):
        a, b = offsets[e], offsets[e + 1]
        if b == a:
            continue
        wg = weight_rows_f64(inp, "w_gate", e, list(hc), wdtype)
        wu = weight_rows_f64(inp, "w_up", e, list(hc), wdtype)
        wd = weight_rows_f64(inp, "w_down", e, list(yc), wdtype)
        h_ref[a:b] = oracle.silu(xp[a:b] @ wg.T) * (xp[a:b] @ wu.T)
        y_ref[a:b] = h_in[a:b] @ wd.T
    assert_fp("H", h_gpu[:, hc], h_ref, rel=rel_gemm, max_abs=None)
    assert_fp("Y_perm (from GPU H)", y_gpu[:, yc], y_ref, rel=rel_gemm, max_abs=None)

    # combine on the GPU's Y_perm
    out_gpu = to_f64(out)
    comb = oracle.combine(to_f64(layer.y_perm), inv[rows], to_f64(layer.topk_w)[rows])
    assert_fp("combine", out_gpu[rows], comb)

    # end to end from the raw inputs, with the GPU's accepted routed sets
    et = rows if e2e_tokens is None else np.asarray(e2e_tokens)
    need = sorted({int(i) - eb for t in et for i in gpu_idx[t] if eb <= i < eb + ec})
    cache = {e: expert_f64(inp, e, wdtype) for e in need}
    ref = oracle.moe_ffn(x[et], to_f64(inp["gamma"]), w_r, bias,
                         lambda e: cache[e], eb, ec, idx=gpu_idx[et], act_fp8=a8)
    max_abs = 2e-2 if wdtype == "bf16" else None
    assert_fp("FFN output (end to end)", out_gpu[et], ref["out"], rel=rel, max_abs=max_abs)
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
    """RMSNorm + one bf16 TP shard (4096 x 4096, f_s 2048): sampled rows."""
    spec = WORKLOADS["norm_tp_shard_bf16_4096"]
    T, d, f = spec["T"], spec["d"], spec["f"]
    D = make_dense(T, d, f, dtype=torch.bfloat16, norm=True, device=DEV)
    v = g.rmsnorm(D["x"], D["gamma"], 1e-5)
    part, h = g.tp_shard_mlp(v, *(g.pack_weights(D[k]) for k in ("w_gate", "w_up", "w_down")))
    torch.cuda.synchronize()
    rows = np.random.default_rng(0).choice(T, size=192, replace=False)
    rows[:2] = [0, T - 1]
    x = to_f64(D["x"])[rows]
    assert_fp("V", to_f64(v)[rows], oracle.rmsnorm(x, to_f64(D["gamma"]), 1e-5))
    vg = to_f64(v)[rows]
    wg, wu, wd = (to_f64(D[k]).T for k in ("w_gate", "w_up", "w_down"))
    assert_fp("H", to_f64(h)[rows], oracle.silu(vg @ wg) * (vg @ wu), max_abs=None)
    assert_fp("partial", to_f64(part)[rows], oracle.tp_shard_mlp(vg, wg, wu, wd, 1, 0))


@pytest.fixture(scope="module")
def prefill(g):
    spec = WORKLOADS["moe_prefill_8192tok_32exp_bf16"]
    inp = make_moe(spec["T"], spec["d"], spec["f"], spec["E"], spec["e_begin"], spec["e_count"],
                   wdtype="bf16", zipf=spec["zipf"], device=DEV)
    layer = build_layer(g, inp, spec["T"], spec["d"], spec["f"], spec["e_begin"])
    return spec, inp, layer


def test_workload_prefill_8192tok(g, prefill):
    spec, inp, layer = prefill
    T = spec["T"]
    r = np.random.default_rng(1)
    tokens = np.sort(r.choice(T, size=256, replace=False))
    tokens[0], tokens[-1] = 0, T - 1
    res = check_layer(g, layer, inp, T, spec["d"], spec["f"], spec["E"], spec["e_begin"],
                      spec["e_count"], "bf16", token_sample=tokens,
                      col_sample=list(range(96, 128)) + [2047],
                      e2e_tokens=tokens[:12])
    counts = to_i64(layer.counts)
    # the skewed bias gives the local experts uneven loads (0.5x to 3x the mean)
    assert counts.max() > 2 * counts.mean() and counts.min() > 0
    assert res["S"] == counts.sum()


def test_prefill_is_deterministic(g, prefill):
    spec, inp, layer = prefill
    a = layer(inp["x"]).clone()
    b = layer(inp["x"]).clone()
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_workload_decode_64tok_fp8(g):
    spec = WORKLOADS["moe_decode_64tok_256exp_fp8"]
    inp = make_moe(spec["T"], spec["d"], spec["f"], spec["E"], spec["e_begin"], spec["e_count"],
                   wdtype="fp8", device=DEV)
    layer = build_layer(g, inp, spec["T"], spec["d"], spec["f"], spec["e_begin"])
    res = check_layer(g, layer, inp, spec["T"], spec["d"], spec["f"], spec["E"],
                      spec["e_begin"], spec["e_count"], "fp8",
                      col_sample=list(range(256, 288)), e2e_tokens=[0, 63])
    assert res["S"] == 64 * 8


def test_workload_prefill_8192tok_fp8_activations(g):
    spec = WORKLOADS["moe_prefill_8192tok_32exp_fp8act"]
    inp = make_moe(spec["T"], spec["d"], spec["f"], spec["E"], spec["e_begin"], spec["e_count"],
                   wdtype="fp8", zipf=spec["zipf"], device=DEV)
    layer = build_layer(g, inp, spec["T"], spec["d"], spec["f"], spec["e_begin"], act_fp8=True)
    T = spec["T"]
    r = np.random.default_rng(2)
    tokens = np.sort(r.choice(T, size=128, replace=False))
    tokens[0], tokens[-1] = 0, T - 1
    res = check_layer(g, layer, inp, T, spec["d"], spec["f"], spec["E"], spec["e_begin"],
                      spec["e_count"], "fp8", token_sample=tokens,
                      col_sample=list(range(128, 160)) + [2047], e2e_tokens=tokens[:6])
    assert res["S"] == to_i64(layer.counts).sum()


def _masked_twin(g, inp, T, d, f, eb, cap=None):
    return g.MoEFFNLayer(T=T, d=d, f=f, w_r=inp["w_r"], bias=inp["bias"], gamma=inp.get("gamma"),
                         w_gate=inp["w_gate"], w_up=inp["w_up"], w_down=inp["w_down"],
                         e_begin=eb, s_gate=inp.get("s_gate"), s_up=inp.get("s_up"),
                         s_down=inp.get("s_down"), layout="masked", cap=cap)


@pytest.mark.parametrize("wdtype,T,eb,ec", [("bf16", 200, 16, 16), ("fp8", 64, 0, 64)])
def test_masked_layout_equals_contiguous(g, wdtype, T, eb, ec):
    """The masked (fixed-capacity) layout changes where rows live, not their
    arithmetic: the layer output is bit-identical to the contiguous layer's,
    which check_layer ties to the oracle; the dispatch integers are the
    oracle's."""
    d, f, E = 256, 256, 64
    inp = make_moe(T, d, f, E, eb, ec, wdtype=wdtype, seed=T + ec + 9, device=DEV)
    contig = build_layer(g, inp, T, d, f, eb)
    check_layer(g, contig, inp, T, d, f, E, eb, ec, wdtype)
    masked = _masked_twin(g, inp, T, d, f, eb)
    a = contig(inp["x"]).clone()
    b = masked(inp["x"]).clone()
    torch.cuda.synchronize()
    counts, rows, pos = oracle.dispatch_masked(to_i64(masked.idx), eb, ec, T)
    assert np.array_equal(to_i64(masked.counts), counts)
    assert np.array_equal(to_i64(masked.inv_pos), pos)
    used = rows >= 0
    assert np.array_equal(to_i64(masked.row_index)[used], rows[used])
    assert torch.equal(a, b)


def test_workload_decode_64tok_fp8_masked(g):
    spec = WORKLOADS["moe_decode_64tok_256exp_fp8"]
    inp = make_moe(spec["T"], spec["d"], spec["f"], spec["E"], spec["e_begin"], spec["e_count"],
                   wdtype="fp8", device=DEV)
    contig = build_layer(g, inp, spec["T"], spec["d"], spec["f"], spec["e_begin"])
    masked = _masked_twin(g, inp, spec["T"], spec["d"], spec["f"], spec["e_begin"])
    a = contig(inp["x"]).clone()
    b = masked(inp["x"]).clone()
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert int(masked.counts.sum()) == spec["T"] * 8
