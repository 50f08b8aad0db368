"""GPU parity at the full V3-shaped sizes (T = 8192 and the 64-token decode step), in the launch
configuration bench.py times.

Routing, gates, counts, offsets, the permutation and the bias update are compared on every token, bit
for bit (gates within 1e-5). Expert outputs are compared on rows the oracle evaluates one expert at a
time (its E4M3 experts rebuilt in parallel on the host cores): at T = 8192 the rows at every 128-row
boundary of every routed expert (the first and last row of each half of every 256-token tile, so every
tile of both grouped launches, and the ragged tails) and of the shared group, and h with its routed and
shared parts for every 64th token; at the decode step every row and every token. All within 6e-2
max-abs / RMS (E4M3)."""
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
    g = H.GpuLayer(w, H.make_cfg(w), None, {}, u, wg, bias, off)
    H.check_key_margins(g, z32, r["key"], r["gap"], w.name)
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


def _boundary_rows(n: int) -> np.ndarray:
    """Rows 128 k - 1 and 128 k of a group of n rows, and its first and last row."""
    r = {0, n - 1}
    for k in range(1, (n + 127) // 128):
        r.update((128 * k - 1, 128 * k))
    return np.array(sorted(x for x in r if 0 <= x < n), dtype=np.int64)


def _gather(tokens_by_expert, e, t):
    tokens_by_expert.setdefault(e, set()).add(int(t))


def test_v3_every_tile_and_decode_step():
    from tests import oracle_pool
    w = configs.WORKLOADS["v3_fp8"]
    wd = configs.WORKLOADS["v3_fp8_decode"]
    print("[case] v3_fp8 full size, every tile sampled; v3_fp8_decode every row", flush=True)
    L, o, z32 = _run(w)
    u, wg, bias, off = _host_inputs(w)
    r, offsets, perm, row_of = _check_routing(w, o, z32, u, wg, bias, off)
    Ld, od, zd = _run(wd)
    ud = u[:wd.T]
    rd, offs_d, perm_d, row_of_d = _check_routing(wd, od, zd, ud, wg, bias, off)
    # (expert, token) pairs the oracle evaluates
    need = {}
    sample_rows = []                       # global routed rows sampled at T = 8192
    for e in range(w.E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        for rr in _boundary_rows(b - a):
            sample_rows.append(a + int(rr))
            _gather(need, e, perm[a + rr])
    sample_rows = np.array(sample_rows)
    shared_tokens = _boundary_rows(w.T)
    h_tokens = np.arange(0, w.T, 64)
    # the device rows compared (only those leave the GPU)
    pick = lambda t, i: H.to_np(t[torch.from_numpy(np.asarray(i, dtype=np.int64)).to(t.device)])
    got = {"y_r": dict(zip(np.concatenate([sample_rows, row_of[h_tokens].ravel()]).tolist(),
                           pick(o["y_r"], np.concatenate([sample_rows, row_of[h_tokens].ravel()])))),
           "y_s": pick(o["y_s"], shared_tokens), "h": pick(o["h"], h_tokens), "gw": H.to_np(o["gw"])}
    got_d = {k: H.to_np(od[k]) for k in ("y_r", "y_s", "h", "gw")}
    del L, o
    for t in np.concatenate([shared_tokens, h_tokens, np.arange(wd.T)]):
        _gather(need, -1, t)
    for t in h_tokens:
        for k in range(w.K):
            _gather(need, int(r["idx"][t, k]), t)
    for t in range(wd.T):
        for k in range(wd.K):
            _gather(need, int(rd["idx"][t, k]), t)
    tok = {e: np.array(sorted(v), dtype=np.int64) for e, v in need.items()}
    ys = oracle_pool.fp8_expert_outputs(w.name, {e: u[t] for e, t in tok.items()}, "v3")
    pos = {e: {int(t): i for i, t in enumerate(ts)} for e, ts in tok.items()}
    y_of = lambda e, t: ys[e][pos[e][int(t)]]

    # every tile: the sampled routed rows, expert by expert, and the sampled shared rows
    worst = 0.0
    for e in range(w.E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        rows = sample_rows[(sample_rows >= a) & (sample_rows < b)]
        if len(rows) == 0:
            continue
        ref = np.vstack([y_of(e, perm[x]) for x in rows])
        worst = max(worst, H.err(np.vstack([got["y_r"][int(x)] for x in rows]), ref))
    e_sh = H.err(got["y_s"], np.vstack([y_of(-1, t) for t in shared_tokens]))
    # h, its routed part (device gates and rows) and its shared part, every 64th token
    y_rows_ref = {int(t): np.vstack([y_of(int(r["idx"][t, k]), t) for k in range(w.K)]) for t in h_tokens}
    routed_ref = np.vstack([(r["w"][t][:, None] * y_rows_ref[int(t)]).sum(0) for t in h_tokens])
    sh_ref = np.vstack([y_of(-1, t) for t in h_tokens])
    h_ref = u[h_tokens] + sh_ref + routed_ref
    routed_got = np.vstack([(got["gw"][t][:, None] * np.vstack([got["y_r"][int(x)] for x in row_of[t]])).sum(0)
                            for t in h_tokens])
    e_h, e_routed = H.err(got["h"], h_ref), H.err(routed_got, routed_ref)
    print(f"v3 T=8192: {len(sample_rows)} sampled routed rows over {int((np.diff(offsets) > 0).sum())} experts, "
          f"worst expert err {worst:.4f}; shared ({len(shared_tokens)} rows) {e_sh:.4f}; "
          f"every 64th token: h {e_h:.4f} routed {e_routed:.4f}", flush=True)
    for v in (worst, e_sh, e_h, e_routed):
        assert v <= H.TOL["fp8"]

    # decode step: every row, every token
    yd_ref = np.vstack([y_of(int(rd["idx"][t, k]), t) for t in range(wd.T) for k in range(wd.K)])
    yd_got = np.vstack([got_d["y_r"][row_of_d[t, k]] for t in range(wd.T) for k in range(wd.K)])
    e_rows = H.err(yd_got, yd_ref)
    e_shd = H.err(got_d["y_s"], np.vstack([y_of(-1, t) for t in range(wd.T)]))
    routed_ref_d = (rd["w"][:, :, None] * yd_ref.reshape(wd.T, wd.K, wd.d)).sum(1)
    h_ref_d = ud + np.vstack([y_of(-1, t) for t in range(wd.T)]) + routed_ref_d
    routed_got_d = (got_d["gw"][:, :, None] * yd_got.reshape(wd.T, wd.K, wd.d)).sum(1)
    e_hd, e_rd = H.err(got_d["h"], h_ref_d), H.err(routed_got_d, routed_ref_d)
    print(f"v3 decode T=64: rows {e_rows:.4f} shared {e_shd:.4f} routed {e_rd:.4f} h {e_hd:.4f}", flush=True)
    for v in (e_rows, e_shd, e_hd, e_rd):
        assert v <= H.TOL["fp8"]


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
        worst = _check_wgrad(H.to_np(dw13[e]), H.to_np(dw2[e]), ref13, ref2, dy, x, ex, ops, b - a, f"expert {e}")
        print(f"expert {e}: {b - a} rows, dx err {e_dx:.4f}, dW plain max-abs/RMS {worst:.4f}", flush=True)
        assert e_dx <= H.TOL["fp8"]
