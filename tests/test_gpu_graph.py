"""moe_forward and moe_forward_noalloc captured into a HIP graph (torch.cuda.CUDAGraph) and replayed: every
replay must give the eager call's routing, counts and h bit for bit. Between replays the test does eager
work of its own (an eager forward on another workspace, output poisoning, a new batch copied into the
captured input) with synchronizations, and a replay after the input changed must follow the new input.
The forward clears its counters and flags with fill kernels, never with memset nodes, so a captured
graph replays them like any other kernel."""
import pytest
import torch

import fine_grained_mixture_gemm_amd as moe
from synth import configs
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

W = configs.WORKLOADS
CASES = {
    # the tiled E4M3 kernel (shared block, ragged groups) and the decode-batch kernels, tiled weights
    "fp8_tiled": W["v3_fp8"].replace(name="graph_fp8_tiled", T=300, d=512, E=20, K=4),
    "fp8_decode": W["v3_fp8"].replace(name="graph_fp8_decode", T=64, d=512, E=20, K=4),
    # bf16 on the tiled kernel with two shared experts, softmax gates
    "bf16": W["dsmoe16b_bf16"].replace(name="graph_bf16", T=600, d=512, E=16, K=6, f=384),
}


def _tiled_layer(g):
    t = g.t
    for key, which in (("w13", moe.MOE_PACK_W13), ("w2", moe.MOE_PACK_W2), ("ws13", moe.MOE_PACK_WS13),
                       ("ws2", moe.MOE_PACK_WS2)):
        if key in t:
            src = t[key] if t[key].dtype == torch.uint8 else t[key].view(torch.uint8)
            dst = torch.empty_like(src)
            moe.moe_pack_weights(g.cfg, which, src, dst)
            t[key + "_tiled"] = dst
    torch.cuda.synchronize()
    return moe.make_layer(t["w13_tiled"], t["w2_tiled"], t["wg"], ws13=t.get("ws13_tiled"), ws2=t.get("ws2_tiled"),
                          w13_scale=t.get("w13s"), w2_scale=t.get("w2s"), ws13_scale=t.get("ws13s"),
                          ws2_scale=t.get("ws2s"), logit_offset=t["off"], weight_layout=moe.MOE_LAYOUT_TILED)


def _outputs(g):
    w = g.w
    return (torch.empty_like(g.t["u"]), torch.empty((w.T, w.K), dtype=torch.int32, device=H.DEV),
            torch.empty(w.E, dtype=torch.int32, device=H.DEV))


def _poison(outs):
    h, idx, cnt = outs
    h.fill_(float("nan"))
    idx.fill_(-7)
    cnt.fill_(-7)


def _same(a, b):
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    if a.dtype == torch.float32:
        return torch.equal(a.view(torch.int32), b.view(torch.int32))
    return torch.equal(a, b)


def _eager(g, layer, u, noalloc=False):
    outs = _outputs(g)
    _poison(outs)
    if noalloc:
        moe.moe_forward_noalloc(g.cfg, layer, u, g.t["bias"], *outs)
    else:
        moe.moe_forward(g.cfg, layer, u, g.t["bias"], *outs, H.workspace(g, poison=True))
    torch.cuda.synchronize()
    return outs


def _check(got, ref, label):
    for name, x, y in zip(("h", "topk_idx", "counts"), got, ref):
        assert _same(x, y), f"{label}: {name} of the graph replay differs from the eager forward"


@pytest.mark.parametrize("name", list(CASES) + ["fp8_tiled_noalloc"])
def test_forward_graph_replays_match_eager(name):
    noalloc = name.endswith("_noalloc")
    w = CASES[name.removesuffix("_noalloc")]
    print(f"[case] graph {name} T={w.T}", flush=True)
    g = H.build(w)
    layer = _tiled_layer(g)
    if noalloc:
        assert moe.moe_workspace_size(g.cfg) <= moe.MOE_NOALLOC_SCRATCH_BYTES
    u_static = g.t["u"].clone()
    # a second batch: the same rows in reverse order (other routing per position, same value range)
    u_other = torch.flip(g.t["u"], dims=[0]).contiguous()
    ref = _eager(g, layer, u_static, noalloc)
    ref_other = _eager(g, layer, u_other, noalloc)

    ws = H.workspace(g, poison=True)
    outs = _outputs(g)

    def step():
        if noalloc:
            moe.moe_forward_noalloc(g.cfg, layer, u_static, g.t["bias"], *outs)
        else:
            moe.moe_forward(g.cfg, layer, u_static, g.t["bias"], *outs, ws)

    # warm up on a side stream (kernel attributes are set on first use), then capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    for rep in range(3):
        _poison(outs)
        ws.fill_(0xFF)                 # the captured workspace: nothing may depend on its old contents
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        _check(outs, ref, f"{name} replay {rep}")
        # eager work between replays: a forward of its own on another workspace
        _check(_eager(g, layer, u_other, noalloc), ref_other, f"{name} eager call after replay {rep}")

    # a new batch in the captured input buffer: the replay follows it
    u_static.copy_(u_other)
    _poison(outs)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    _check(outs, ref_other, f"{name} replay on the second batch")
    # and back
    u_static.copy_(g.t["u"])
    graph.replay()
    torch.cuda.synchronize()
    _check(outs, ref, f"{name} replay on the first batch again")


def test_step_with_bias_update_graph_replays_match_eager():
    """The timed step of the decode workload (forward, then a copy of the bias and one bias update into the
    copy) captured as one graph: every replay gives the eager step's h, routing, counts and updated bias bit
    for bit, and the bias the forward reads is never changed by a replay."""
    w = CASES["fp8_decode"].replace(name="graph_fp8_decode_bias", gamma=0.001)
    print(f"[case] graph step with bias update T={w.T}", flush=True)
    g = H.build(w)
    layer = _tiled_layer(g)
    bias = g.t["bias"]
    bias0 = bias.clone()
    ws = H.workspace(g, poison=True)
    outs = _outputs(g)
    bias_next = torch.empty_like(bias)

    def step():
        moe.moe_forward(g.cfg, layer, g.t["u"], bias, *outs, ws)
        bias_next.copy_(bias)
        moe.moe_update_bias(g.cfg, outs[2], w.gamma, bias_next)

    _poison(outs)
    step()
    torch.cuda.synchronize()
    ref = tuple(x.clone() for x in outs)
    ref_bias = bias_next.clone()
    assert not torch.equal(ref_bias, bias0), "the update left every bias unchanged: no load differs from the mean"

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        _poison(outs)
        bias_next.fill_(float("nan"))
        ws.fill_(0xFF)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        _check(outs, ref, f"bias step replay {rep}")
        assert _same(bias_next, ref_bias), f"replay {rep}: updated bias differs from the eager step"
        assert _same(bias, bias0), f"replay {rep}: the forward's bias changed"
