"""The FFN sub-block as a HIP graph: MoEFFNLayer.forward captured once
(torch.cuda.CUDAGraph) and replayed.

The forward allocates nothing, synchronises nothing and issues no memset, so
it can be captured. Each replay must reproduce the eager forward bit for bit
(every kernel is deterministic). The replays are separated by eager work of
the program's own (a fill of the output and of the intermediates) and by
device synchronisations. After a replay on new input values written into
the captured input buffer, the output must equal an eager forward on those
values.
"""

import pytest
import torch

from synth.workloads import make_moe

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def g():
    import gated_mlp_transformer_amd as mod
    return mod


def _layer(g, inp, T, d, f, e_begin, **kw):
    return g.MoEFFNLayer(T=T, d=d, f=f, w_r=inp["w_r"], bias=inp["bias"], gamma=inp.get("gamma"),
                         w_gate=inp["w_gate"], w_up=inp["w_up"], w_down=inp["w_down"],
                         e_begin=e_begin, s_gate=inp.get("s_gate"), s_up=inp.get("s_up"),
                         s_down=inp.get("s_down"), **kw)


def _capture(layer, x):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer(x)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out = layer(x)
    torch.cuda.synchronize()
    return graph, out


@pytest.mark.parametrize("T,d,f,E,eb,ec,wdtype,kw", [
    (96, 256, 256, 32, 8, 8, "bf16", {}),                       # contiguous, bf16
    (640, 256, 512, 16, 0, 16, "bf16", {}),                     # several tiles per expert
    (16, 256, 256, 16, 0, 16, "fp8", {}),                       # decode-shaped, fp8 weights
    (16, 256, 256, 16, 0, 16, "fp8", {"layout": "masked"}),     # fixed-capacity layout
    (128, 256, 256, 32, 4, 12, "fp8", {"act_fp8": True}),       # fp8 activations
])
def test_graph_replays_equal_eager(g, T, d, f, E, eb, ec, wdtype, kw):
    inp = make_moe(T, d, f, E, eb, ec, wdtype=wdtype, zipf=0.05, seed=T + ec + 17, device=DEV)
    layer = _layer(g, inp, T, d, f, eb, **kw)
    x = inp["x"].clone()
    ref = layer(x).clone()
    torch.cuda.synchronize()
    graph, out = _capture(layer, x)
    for _ in range(3):
        # the program's own eager work between replays
        layer.out.fill_(float("nan"))
        layer.h.fill_(float("nan"))
        layer.y_perm.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
    # new values in the captured input buffer: the replay computes on them
    x.copy_(make_moe(T, d, f, E, eb, ec, wdtype=wdtype, zipf=0.05, seed=T + ec + 18,
                     device=DEV)["x"])
    graph.replay()
    torch.cuda.synchronize()
    got = out.clone()
    want = layer(x).clone()
    torch.cuda.synchronize()
    assert torch.equal(got, want)
    assert not torch.equal(got, ref)
    del graph
