"""The layer captured into a HIP graph (torch.cuda.CUDAGraph around calls
through the C ABI on the capturing stream) and replayed.

Every entry point launches kernels only, on the stream it is given (no
allocation, memset, copy or host synchronisation), so a graph holds a whole
step.  Each replay must reproduce the eager call bit for bit: the graph is
replayed several times, with the batch in its input buffer changed between
replays (other routing, other row counts per expert, so other tile tables and
claim counters) and with eager work of the library in between."""
import pytest
import torch

import mixture_experts_layer_45_amd as moe
from mixture_experts_layer_45_amd import inputs
from tests import _gpu as G

pytestmark = pytest.mark.gpu

CASES = {
    "top2_drops": ("top2_e8_h4096", dict(T=600, h=512, f=320, capacity_factor=0.8)),
    # E > 64 with T >= 256: the split-K router GEMM path
    "sigmoid_shared_split_route": ("sigmoid_top8_e256_shared", dict(T=512, h=512, f=128)),
    "multihead_wo": ("multihead_h8_e32_top4", dict(T=300, h=512, f=128)),
    "switch_gelu_zipf": ("switch_top1_e64_zipf", dict(T=1000, h=128, f=256)),
}


def _aux(cfg):
    T, H, E, K = cfg["T"], cfg.get("H", 1), cfg["E"], cfg["K"]
    S, Et = T * H, H * E
    i32 = dict(dtype=torch.int32, device=G.DEV)
    f32 = dict(dtype=torch.float32, device=G.DEV)
    return dict(topk_idx=torch.empty((S, K), **i32), topk_w=torch.empty((S, K), **f32),
                dest_row=torch.empty(S * K, **i32), counts=torch.empty(Et, **i32), kept=torch.empty(Et, **i32),
                n_kept=torch.empty(1, **i32), n_dropped=torch.empty(1, **i32), f=torch.empty(Et, **f32),
                P=torch.empty(Et, **f32), l_aux=torch.empty(1, **f32))


def _same(a, b):
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    if a.dtype == torch.float32:
        return torch.equal(a.view(torch.int32), b.view(torch.int32))
    return torch.equal(a, b)


def _capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()  # a warm call on a side stream, as torch's capture recipe asks
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("packed", [0, 1], ids=["row_major", "fragment_order"])
@pytest.mark.parametrize("case", sorted(CASES))
def test_forward_graph_replays_match_eager(case, packed):
    name, over = CASES[case]
    cfg = inputs.variant(name, **over)
    G.log(f"[graph] forward {case} packed={packed}")
    inp = G.dev_inputs(cfg)
    if packed:  # the expert weights in fragment order, as bench.py times the layer
        cfg = dict(cfg, packed=1)
        inp = moe.pack_weights(inp)
        torch.cuda.synchronize()
    x_a = inp["x"].clone()
    x_b = G.dev_inputs(cfg, seed=5)["x"]
    d = moe.desc_from_cfg(cfg)
    ws = moe.workspace(d)

    def eager(x):
        y = torch.empty_like(x)
        aux = _aux(cfg)
        moe.moe_layer_forward(d, inp, x, y, aux, ws)
        torch.cuda.synchronize()
        return y, aux

    ref = {"a": eager(x_a), "b": eager(x_b)}
    assert not torch.equal(ref["a"][1]["topk_idx"], ref["b"][1]["topk_idx"])
    x_in = x_a.clone()
    y = torch.empty_like(x_in)
    aux = _aux(cfg)
    g = _capture(lambda: moe.moe_layer_forward(d, inp, x_in, y, aux, ws))
    for rep, which in enumerate(("a", "b", "a", "b")):
        x_in.copy_(x_a if which == "a" else x_b)
        y.fill_(7.0)
        for t in aux.values():
            t.fill_(-3)
        g.replay()
        torch.cuda.synchronize()
        ry, raux = ref[which]
        assert _same(y, ry), (case, rep, "y")
        for k in aux:
            assert _same(aux[k], raux[k]), (case, rep, k)
        eager(x_b if which == "a" else x_a)  # the library's own eager work between replays


@pytest.mark.parametrize("case", ["top2_drops", "sigmoid_shared_split_route", "multihead_wo"])
def test_training_step_graph_replays_match_eager(case):
    """Training forward and backward in one graph."""
    name, over = CASES[case]
    cfg = inputs.variant(name, **over)
    G.log(f"[graph] training step {case}")
    inp = G.dev_inputs(cfg)
    d = moe.desc_from_cfg(cfg)
    ws_f = moe.workspace(d)
    ws_b = moe.workspace(d, moe.MOE_WS_BACKWARD)
    dy = torch.randn((cfg["T"], cfg["h"]), generator=torch.Generator().manual_seed(4)).to(torch.bfloat16).to(G.DEV)

    def step(y, sv, gr):
        moe.moe_layer_forward_train(d, inp, inp["x"], y, sv, ws=ws_f)
        moe.moe_layer_backward(d, inp, inp["x"], dy, sv, gr, aux_weight=1.0, ws=ws_b)

    def fresh():
        return (torch.empty_like(inp["x"]), moe.alloc_saved(d, G.DEV), moe.alloc_grads(d, inp, inp["x"]))

    ref = fresh()
    step(*ref)
    torch.cuda.synchronize()
    bufs = fresh()
    g = _capture(lambda: step(*bufs))
    y, sv, gr = bufs
    for rep in range(3):
        y.fill_(7.0)
        for t in gr.values():
            t.fill_(7.0)
        g.replay()
        torch.cuda.synchronize()
        assert _same(y, ref[0]), (case, rep, "y")
        for k in gr:
            assert _same(gr[k], ref[2][k]), (case, rep, k)
        other = fresh()
        step(*other)  # eager work between replays
        torch.cuda.synchronize()
