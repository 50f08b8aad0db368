"""GPU parity at the full V3-shaped sizes (T = 8192 and the 64-token decode step), in the launch
configuration bench.py times.

Routing, gates, counts, offsets, the permutation and the bias update are compared on every token, bit
for bit (gates within 1e-5). Expert outputs are compared on samples the oracle can afford one by one:
every routed row and the shared row of token 0, every row of token 0's first expert, and h of token 0,
within 6e-2 max-abs / RMS (E4M3)."""
import functools

import numpy as np
import pytest
import torch

import fine_grained_mixture_gemm_amd as moe
from fine_grained_mixture_gemm_amd import layers
from oracle import moe as omoe
from synth import configs
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

RECHECK_DELTA = 4e-5      # the library's fp32-to-fp64 recheck margin for sigmoid keys


@functools.lru_cache(maxsize=None)
def _oracle_expert(seed: int, e: int):
    # the oracle's own E4M3 weights (config 4 and the decode step share seed and layer)
    return H.oracle_fp8_expert(configs.WORKLOADS["v3_fp8"], e)


def _host_inputs(w):
    u = configs.u_as_f32(w, configs.make_u(w))
    wg, bias, off = configs.make_router(w)
    return u, wg, bias, off


def _run(w):
    L = layers.device_layer(w)
    g = H.GpuLayer(w, L.cfg, L.layer, L.t, None, None, None, None)
    ws = H.workspace(g, poison=True)
    o = H.run_stages(g, ws)
    z = torch.empty((w.T, w.E), dtype=torch.float32, device="cuda")
    moe.moe_router_logits(L.cfg, L.layer, L.t["u"], z, ws)
    torch.cuda.synchronize()
    return L, o, H.to_np(z)


def _check_routing(w, o, z32, u, wg, bias, off):
    z = omoe.router_logits(u, wg, off)
    r = omoe.route(z, w.gate, w.K, bias, w.renorm, w.n_groups, w.topk_groups)
    key32 = 1.0 / (1.0 + np.exp(-z32.astype(np.float64))) if w.gate == "sigmoid_bias" else z32
    key64 = r["key"] - (bias[None, :] if (w.gate == "sigmoid_bias" and bias is not None) else 0.0)
    kerr = float(np.abs(key32 - key64).max())
    print(f"{w.name}: max fp32 key error {kerr:.3e}, min fp64 gap {r['gap'].min():.3e}, "
          f"tokens under the recheck margin {int((r['gap'] < RECHECK_DELTA).sum())}", flush=True)
    assert kerr * 20 <= RECHECK_DELTA, "fp32 keys are not 20x inside the recheck margin"
    assert r["gap"].min() > 1e-9, "an fp64 near-tie would make the selection ill-defined"
    assert np.array_equal(H.to_np(o["idx"]), r["idx"])
    assert np.abs(H.to_np(o["gw"]) - r["w"]).max() < 1e-5
    offsets, perm, row_of = omoe.dispatch(r["idx"], w.E)
    assert np.array_equal(H.to_np(o["counts"]), omoe.expert_counts(r["idx"], w.E))
    assert np.array_equal(H.to_np(o["offsets"]), offsets)
    assert np.array_equal(H.to_np(o["perm"]), perm)
    assert np.array_equal(H.to_np(o["row_of"]), row_of)
    return r, offsets, perm, row_of


def _check_token0(w, o, u, r, row_of):
    ys = omoe.swiglu_ffn_fp8(u[:1], *_oracle_expert(w.seed, -1))[0]
    e_sh = H.err(H.to_np(o["y_s"][:1]), ys)
    ys_all = []
    for k in range(w.K):
        e = int(r["idx"][0, k])
        y = omoe.swiglu_ffn_fp8(u[:1], *_oracle_expert(w.seed, e))[0]
        ys_all.append(y)
    y_ref = np.vstack(ys_all)
    y_gpu = H.to_np(o["y_r"])[row_of[0]]
    e_rows = H.err(y_gpu, y_ref)
    routed_ref = (r["w"][0][:, None] * y_ref).sum(axis=0, keepdims=True)
    h_ref = u[:1] + ys + routed_ref
    e_h = H.err(H.to_np(o["h"][:1]), h_ref)
    e_routed = H.err((H.to_np(o["gw"])[0][:, None] * y_gpu).sum(axis=0, keepdims=True), routed_ref)
    print(f"{w.name} token 0: rows {e_rows:.4f} shared {e_sh:.4f} routed {e_routed:.4f} h {e_h:.4f}", flush=True)
    for v in (e_rows, e_sh, e_routed, e_h):
        assert v <= H.TOL["fp8"]


def test_v3_layer_full_size():
    w = configs.WORKLOADS["v3_fp8"]
    print("[case] v3_fp8 full size", flush=True)
    L, o, z32 = _run(w)
    u, wg, bias, off = _host_inputs(w)
    r, offsets, perm, row_of = _check_routing(w, o, z32, u, wg, bias, off)
    _check_token0(w, o, u, r, row_of)
    # every row of token 0's first expert
    e = int(r["idx"][0, 0])
    a, b = offsets[e], offsets[e + 1]
    y_ref = omoe.swiglu_ffn_fp8(u[perm[a:b]], *_oracle_expert(w.seed, e))[0]
    e_exp = H.err(H.to_np(o["y_r"][a:b]), y_ref)
    print(f"expert {e}: {b - a} rows, err {e_exp:.4f}", flush=True)
    assert e_exp <= H.TOL["fp8"]


def test_v3_node_limited_routing_full_size():
    # the V3 limit of the MoE report (3.2, 3.8): each token's experts on at most 4 of 8 nodes
    w = configs.WORKLOADS["v3_fp8"].replace(name="v3_fp8_node_limited", n_groups=8, topk_groups=4)
    print("[case] v3_fp8 node-limited routing", flush=True)
    L, o, z32 = _run(w)
    u, wg, bias, off = _host_inputs(w)
    r, offsets, perm, row_of = _check_routing(w, o, z32, u, wg, bias, off)
    groups = H.to_np(o["idx"]) // (w.E // w.n_groups)
    assert max(len(set(row)) for row in groups.tolist()) <= w.topk_groups
    _check_token0(w, o, u, r, row_of)


def test_v3_decode_step_and_bias_update():
    w = configs.WORKLOADS["v3_fp8_decode"]
    print("[case] v3_fp8_decode", flush=True)
    L, o, z32 = _run(w)
    u, wg, bias, off = _host_inputs(w)
    r, offsets, perm, row_of = _check_routing(w, o, z32, u, wg, bias, off)
    # the decode tokens are the first 64 tokens of the V3 workload: routing is per token
    _check_token0(w, o, u, r, row_of)
    # one bias update from this step's loads, bit for bit
    b = L.t["bias"].clone()
    moe.moe_update_bias(L.cfg, o["counts"], w.gamma, b)
    torch.cuda.synchronize()
    ref = omoe.bias_update(bias, omoe.expert_counts(r["idx"], w.E), w.gamma, w.T, w.K)
    got = b.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    assert (got != bias).any()


STREAM_DY_R, STREAM_DY_S = 10_000, 10_001     # seeded output gradients of the backward check


def test_v3_backward_sampled_experts():
    """The E4M3 expert backward (input and weight gradients) at the V3 size, in the launch bench.py times,
    checked on the largest, a median and the smallest non-empty expert (the shared block's gradients are
    checked at the smaller sizes of test_gpu_backward.py); experts with no rows get zero weight gradients."""
    from synth import device as sdev, gen
    from tests.test_gpu_backward import _check_wgrad, _transposed_layer
    w = configs.WORKLOADS["v3_fp8"]
    print("[case] v3_fp8 backward, sampled experts", flush=True)
    L = layers.device_layer(w)
    g = H.GpuLayer(w, L.cfg, L.layer, L.t, None, None, None, None)
    ws = H.workspace(g)
    o = H.run_stages(g, ws)
    layer_t, tt = _transposed_layer(g)
    bf = dict(dtype=torch.bfloat16, device="cuda")
    dy_r = sdev.fill_normal(torch.empty((w.T * w.K, w.d), **bf), w.seed, STREAM_DY_R, 1.0)
    dy_s = sdev.fill_normal(torch.empty((w.T, w.d), **bf), w.seed, STREAM_DY_S, 1.0)
    dx_r, dx_s = torch.empty((w.T * w.K, w.d), **bf), torch.empty((w.T, w.d), **bf)
    dw13, dw2 = torch.empty((w.E, 2 * w.f, w.d), **bf), torch.empty((w.E, w.d, w.f), **bf)
    dws13, dws2 = torch.empty((2 * w.fs, w.d), **bf), torch.empty((w.d, w.fs), **bf)
    bws = torch.empty(moe.moe_backward_workspace_size(L.cfg), dtype=torch.uint8, device="cuda")
    moe.moe_expert_ffn_backward(L.cfg, L.layer, layer_t, L.t["u"], o["offsets"], o["perm"], dy_r, dy_s, dx_r, dx_s,
                                dw13, dw2, dws13, dws2, bws)
    torch.cuda.synchronize()
    offsets, perm = H.to_np(o["offsets"]), H.to_np(o["perm"])
    counts = np.diff(offsets)
    for e in np.flatnonzero(counts == 0):
        assert torch.count_nonzero(dw13[e]).item() == 0 and torch.count_nonzero(dw2[e]).item() == 0
    nz = np.flatnonzero(counts)
    sel = sorted({int(np.argmax(counts)), int(nz[np.argmin(counts[nz])]), int(np.argsort(counts)[len(counts) // 2])})
    u = configs.u_as_f32(w, configs.make_u(w))
    for e in sel:
        a, b = int(offsets[e]), int(offsets[e + 1])
        dy = gen.bf16_bits_to_f32(gen.f32_to_bf16_bits(gen.normal_f32(w.seed, STREAM_DY_R, (b - a, w.d), 1.0,
                                                                      start=a * w.d))).astype(np.float64)
        assert np.array_equal(H.to_np(dy_r[a:b]), dy), "device and host gradient generators disagree"
        ex = _oracle_expert(w.seed, e)
        x = u[perm[a:b]]
        e_dx = H.err(H.to_np(dx_r[a:b]), omoe.swiglu_ffn_backward_input_fp8(dy, x, *ex))
        ref13, ref2, ops = omoe.swiglu_ffn_backward_weight_fp8(dy, x, *ex, operands=True)
        worst = _check_wgrad(H.to_np(dw13[e]), H.to_np(dw2[e]), ref13, ref2, ops, b - a, f"expert {e}")
        print(f"expert {e}: {b - a} rows, dx err {e_dx:.4f}, dW plain max-abs/RMS {worst:.4f}", flush=True)
        assert e_dx <= H.TOL["fp8"]
