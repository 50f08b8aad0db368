"""GPU parity of the E4M3 expert input backward (moe_expert_ffn_backward_input) and of the weight
transposition it uses (moe_transpose_fp8_weights), against the oracle's swiglu_ffn_backward_input_fp8
([TR] §3.6: the activation backward GEMMs in FP8 with the forward's 1x128 / 128x128 tiling).

The routed rows of each expert are compared with the oracle run on that expert's own E4M3 weights
(quantized by the oracle from the fp32 masters) and the rows' tokens; the shared block likewise on every
token. The bar is the E4M3 tolerance max|dx - dx_ref| / RMS(dx_ref) <= 6e-2 per expert and per block."""
import numpy as np
import pytest
import torch

import fine_grained_mixture_gemm_amd as moe
from oracle import moe as omoe
from synth import configs, gen
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

W = configs.WORKLOADS
CASES = {
    # V3 expert inner dim f = 2048 (2 f = 4096 channels of [dg | dv]); ragged groups and token tails
    "bwd_fp8_shared": W["v3_fp8"].replace(name="bwd_fp8_shared", T=160, d=512, E=16, K=4),
    "bwd_fp8_no_shared": W["v3_fp8"].replace(name="bwd_fp8_no_shared", T=100, d=256, E=8, Ks=0, K=2),
    "bwd_fp8_one_token": W["v3_fp8"].replace(name="bwd_fp8_one_token", T=1, d=256, E=32, K=8),
    "bwd_fp8_ragged_tail": W["v3_fp8"].replace(name="bwd_fp8_ragged_tail", T=333, d=256, E=12, K=3),
}


def _transposed(q: torch.Tensor, s: torch.Tensor):
    qt = torch.empty(q.shape[:-2] + (q.shape[-1], q.shape[-2]), dtype=torch.uint8, device=H.DEV)
    st = torch.empty(s.shape[:-2] + (s.shape[-1], s.shape[-2]), dtype=torch.float32, device=H.DEV)
    moe.moe_transpose_fp8_weights(q, s, qt, st)
    return qt, st


def _transposed_layer(g):
    t = g.t
    tt = {}
    tt["w13"], tt["w13s"] = _transposed(t["w13"], t["w13s"])
    tt["w2"], tt["w2s"] = _transposed(t["w2"], t["w2s"])
    if g.w.Ks > 0:
        tt["ws13"], tt["ws13s"] = _transposed(t["ws13"], t["ws13s"])
        tt["ws2"], tt["ws2s"] = _transposed(t["ws2"], t["ws2s"])
    torch.cuda.synchronize()
    layer_t = moe.make_layer(tt["w13"], tt["w2"], t["wg"], ws13=tt.get("ws13"), ws2=tt.get("ws2"),
                             w13_scale=tt["w13s"], w2_scale=tt["w2s"], ws13_scale=tt.get("ws13s"),
                             ws2_scale=tt.get("ws2s"))
    return layer_t, tt


def _bf16_normal(rng, shape):
    bits = gen.f32_to_bf16_bits(rng.normal(0, 1, shape).astype(np.float32))
    return H.bf16_tensor(bits).to(H.DEV), gen.bf16_bits_to_f32(bits).astype(np.float64)


def _run_backward(g, seed=7):
    w = g.w
    ws = H.workspace(g)
    o = H.run_stages(g, ws)
    layer_t, tt = _transposed_layer(g)
    rng = np.random.default_rng(seed)
    dy_r, dy_r_host = _bf16_normal(rng, (w.T * w.K, w.d))
    dy_s, dy_s_host = _bf16_normal(rng, (w.T, w.d)) if w.Ks > 0 else (None, None)
    dx_r = torch.empty((w.T * w.K, w.d), dtype=torch.bfloat16, device=H.DEV)
    dx_s = torch.empty((w.T, w.d), dtype=torch.bfloat16, device=H.DEV) if w.Ks > 0 else None
    bws = torch.empty(moe.moe_backward_workspace_size(g.cfg), dtype=torch.uint8, device=H.DEV)
    bws.fill_(0xFF)   # NaN in every float view: nothing may be read before it is written
    moe.moe_expert_ffn_backward_input(g.cfg, g.layer, layer_t, g.t["u"], o["offsets"], o["perm"], dy_r, dy_s, dx_r,
                                      dx_s, bws)
    torch.cuda.synchronize()
    return o, dict(dy_r=dy_r_host, dy_s=dy_s_host, dx_r=H.to_np(dx_r), dx_s=H.to_np(dx_s) if dx_s is not None else None,
                   tt=tt)


@pytest.mark.parametrize("name", list(CASES))
def test_backward_input_matches_oracle(name):
    w = CASES[name]
    print(f"case {name}: T={w.T} d={w.d} E={w.E} K={w.K} Ks={w.Ks} f={w.f}", flush=True)
    g = H.build(w)
    o, r = _run_backward(g)
    off = H.to_np(o["offsets"])
    perm = H.to_np(o["perm"])
    assert np.isfinite(r["dx_r"]).all()
    worst = 0.0
    for e in range(w.E):
        a, b = int(off[e]), int(off[e + 1])
        if a == b:
            continue
        ref = omoe.swiglu_ffn_backward_input_fp8(r["dy_r"][a:b], g.u_host[perm[a:b]], *H.oracle_fp8_expert(w, e))
        err = H.err(r["dx_r"][a:b], ref)
        worst = max(worst, err)
        assert err <= H.TOL["fp8"], f"expert {e} rows {a}:{b} err {err}"
    if w.Ks > 0:
        assert np.isfinite(r["dx_s"]).all()
        ref = omoe.swiglu_ffn_backward_input_fp8(r["dy_s"], g.u_host, *H.oracle_fp8_expert(w, -1))
        err = H.err(r["dx_s"], ref)
        assert err <= H.TOL["fp8"], f"shared err {err}"
        worst = max(worst, err)
    print(f"worst err {worst:.4f}")


def test_transpose_is_bit_exact():
    w = CASES["bwd_fp8_shared"]
    g = H.build(w)
    _, tt = _transposed_layer(g)
    for k in ("w13", "w2", "ws13", "ws2"):
        q = g.t[k].cpu().numpy()
        s = g.t[k + "s"].cpu().numpy()
        assert np.array_equal(tt[k].cpu().numpy(), np.swapaxes(q, -1, -2)), k
        assert np.array_equal(tt[k + "s"].cpu().numpy(), np.swapaxes(s, -1, -2)), k


def test_backward_of_zero_gradient_is_zero():
    # dy = 0: da = 0, [dg | dv] = 0 with unit scales, dx = 0 exactly, whatever u and the weights
    w = CASES["bwd_fp8_no_shared"]
    g = H.build(w)
    ws = H.workspace(g)
    o = H.run_stages(g, ws)
    layer_t, _ = _transposed_layer(g)
    dy = torch.zeros((w.T * w.K, w.d), dtype=torch.bfloat16, device=H.DEV)
    dx = torch.full((w.T * w.K, w.d), 1.0, dtype=torch.bfloat16, device=H.DEV)
    bws = torch.empty(moe.moe_backward_workspace_size(g.cfg), dtype=torch.uint8, device=H.DEV)
    moe.moe_expert_ffn_backward_input(g.cfg, g.layer, layer_t, g.t["u"], o["offsets"], o["perm"], dy, None, dx, None,
                                      bws)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dx).item() == 0
