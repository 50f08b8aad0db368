"""GPU parity of the whole layer against the oracle, stage by stage, on seeded synthetic layers.

Routing (indices), counts, offsets and the permutation must match bit for bit; float outputs within
max|y - y_ref| / RMS(y_ref) <= 1e-5 (fp32), 2e-2 (bf16), 6e-2 (fp8), checked on every per-row expert
output, the shared output, the routed sum and h."""
import numpy as np
import pytest
import torch

from oracle import moe as omoe
from synth import configs
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

W = configs.WORKLOADS
SMALL = {
    "tiny_f32": W["tiny_f32"],
    "bf16_softmax_ragged": W["dsmoe2b_bf16"].replace(name="bf16_softmax_ragged", T=300, d=256, E=12, K=3, f=128),
    "bf16_2shared_zipf": W["dsmoe16b_bf16"].replace(name="bf16_2shared_zipf", T=200, d=512, E=16, K=4, f=256),
    "bf16_no_shared": W["dsmoe2b_bf16"].replace(name="bf16_no_shared", T=130, d=256, E=8, Ks=0, K=2, f=128, zipf=None),
    # E4M3 cases keep the V3 expert inner dim f = 2048: one requantized SwiGLU code that rounds the
    # other way moves a row of y by about 0.3 * 3 / sqrt(f) of its RMS, so small f inflates the error.
    "fp8_sigmoid_ragged": W["v3_fp8"].replace(name="fp8_sigmoid_ragged", T=333, d=512, E=20, K=4),
    "fp8_k_equals_e": W["v3_fp8"].replace(name="fp8_k_equals_e", T=70, d=256, E=4, K=4),
    # no shared experts on the tiled E4M3 path (its scale copy then has no shared part)
    "fp8_no_shared": W["v3_fp8"].replace(name="fp8_no_shared", T=260, d=512, E=16, Ks=0, K=4),
    "fp8_one_token": W["v3_fp8"].replace(name="fp8_one_token", T=1, d=256, E=32, K=8),
    # batches of at most 128 tokens take the E4M3 decode kernels: groups spanning 3 and 4 token tiles,
    # two shared experts (shared inner dim 2 f)
    "fp8_decode_3tiles": W["v3_fp8"].replace(name="fp8_decode_3tiles", T=64, d=512, E=6, K=4),
    "fp8_decode_2shared": W["v3_fp8"].replace(name="fp8_decode_2shared", T=40, d=512, E=16, Ks=2, K=6),
    "fp8_decode_k_equals_e": W["v3_fp8"].replace(name="fp8_decode_k_equals_e", T=64, d=256, E=4, K=4),
    # the largest decode batch: the shared group takes eight 16-token passes, routed groups several
    "fp8_decode_128": W["v3_fp8"].replace(name="fp8_decode_128", T=128, d=512, E=16, K=4),
    # group-limited routing: 4 groups of 4 keeping 2 (softmax), 8 groups of 4 keeping 4 (sigmoid + bias)
    "bf16_group_limited": W["dsmoe2b_bf16"].replace(name="bf16_group_limited", T=300, d=256, E=16, K=3, f=128,
                                                     n_groups=4, topk_groups=2),
    "fp8_node_limited": W["v3_fp8"].replace(name="fp8_node_limited", T=200, d=512, E=32, K=8, n_groups=8,
                                            topk_groups=4),
    "f32_sigmoid_norenorm": W["tiny_f32"].replace(name="f32_sigmoid_norenorm", gate="sigmoid_bias", renorm=False,
                                                  bias_range=0.1, T=77, E=9, K=3),
    # more routed rows per token than the combine holds in registers at once (bf16 outputs), and the
    # largest top-K the library takes
    "bf16_k12": W["dsmoe2b_bf16"].replace(name="bf16_k12", T=150, d=256, E=24, K=12, f=128),
    "bf16_k16_sigmoid": W["dsmoe2b_bf16"].replace(name="bf16_k16_sigmoid", T=90, d=256, E=20, K=16, f=128,
                                                   gate="sigmoid_bias", renorm=True, bias_range=0.1, zipf=None),
    # enough tokens for the MFMA router logits (T * E >= 2^16) with an expert count that is not a multiple
    # of its 64-expert blocks, a ragged last token block, and d = 1024 split into two slices (the expert
    # inner dim 512: with d = 1024 and f = 128 the bf16 rounding of the routed sum reaches the tolerance)
    "bf16_mfma_router_e63": W["dsmoe2b_bf16"].replace(name="bf16_mfma_router_e63", T=2100, d=1024, E=63, K=7,
                                                       f=512),
    # heavy-tailed token rows (about 1 in 16 scaled by 32, 1 in 8 by 8, 1 in 16 with one element scaled by
    # 64): the 1x128 amax, the requantization and the router's recheck margins on outliers; the MFMA
    # router logits and the vector-ALU logits, E4M3 and bf16 experts. Rows then differ in scale by up to
    # 32^2 (SwiGLU is quadratic in u), so the tolerance is applied row by row (H.err_rows).
    "fp8_heavy_tail": W["v3_fp8"].replace(name="fp8_heavy_tail", T=300, d=512, E=20, K=4, u_tail=True),
    "bf16_heavy_tail_mfma_router": W["dsmoe2b_bf16"].replace(name="bf16_heavy_tail_mfma_router", T=2100, d=1024,
                                                             E=63, K=7, f=512, u_tail=True),
    # the largest d_model the library takes (8192: the fp64 recheck holds a whole centroid row, 32 elements
    # per thread): router, recheck, 32 K stages of the tiled bf16 kernel and the combine at that width
    "bf16_max_d": W["dsmoe2b_bf16"].replace(name="bf16_max_d", T=300, d=8192, E=8, K=2, f=512),
}


def _oracle_layer(g):
    w = g.w
    if w.wdt == "fp8":
        experts = [H.oracle_fp8_expert(w, e) for e in range(w.E)]
        shared = H.oracle_fp8_expert(w, -1) if w.Ks > 0 else None
    else:
        experts, shared = g.host_experts, g.host_shared
    return omoe.layer_forward(g.u_host, g.wg, experts, shared, gate=w.gate, K=w.K, bias=g.bias, renorm=w.renorm,
                              logit_offset=g.off, fp8=(w.wdt == "fp8"), n_groups=w.n_groups,
                              topk_groups=w.topk_groups)


def _check_all(g, o, ref):
    w = g.w
    tol = H.TOL[w.wdt]
    y_bf16 = o["y_r"].dtype == torch.bfloat16
    gw = H.to_np(o["gw"])

    def err(y, y_ref, rounding=None):
        # heavy-tailed rows: the tolerance row by row, past the bf16 rounding of each stored element
        if not w.u_tail:
            return H.err(y, y_ref)
        return H.err_rows(y, y_ref, 0.0 if rounding is None else 2.0 ** -8 * rounding)
    assert np.array_equal(H.to_np(o["idx"]), ref["idx"]), "routing differs"
    assert np.array_equal(H.to_np(o["counts"]), ref["counts"])
    assert np.array_equal(H.to_np(o["offsets"]), ref["offsets"])
    assert np.array_equal(H.to_np(o["perm"]), ref["perm_src"])
    assert np.array_equal(H.to_np(o["row_of"]), ref["row_of"])
    gate_err = np.abs(H.to_np(o["gw"]) - ref["w"]).max()
    assert gate_err < 1e-5, gate_err
    e_rows = err(H.to_np(o["y_r"]), ref["y_rows"], np.abs(ref["y_rows"]) if y_bf16 else None)
    assert e_rows <= tol, f"per-row expert outputs err {e_rows}"
    if w.Ks > 0:
        e_sh = err(H.to_np(o["y_s"]), ref["y_shared"], np.abs(ref["y_shared"]) if y_bf16 else None)
        assert e_sh <= tol, f"shared err {e_sh}"
    y = H.to_np(o["y_r"])
    zero = np.zeros_like(g.u_host)
    routed = omoe.combine(zero, zero, y, ref["row_of"], gw)
    routed_mag = omoe.combine(zero, zero, np.abs(ref["y_rows"]), ref["row_of"], np.abs(gw)) if y_bf16 else None
    e_routed = err(routed, ref["routed"], routed_mag)
    assert e_routed <= tol, f"routed sum err {e_routed}"
    h_bf16 = o["h"].dtype == torch.bfloat16
    e_h = err(H.to_np(o["h"]), ref["h"], np.abs(ref["h"]) if h_bf16 else None)
    assert e_h <= tol, f"h err {e_h}"
    return dict(rows=e_rows, h=e_h, routed=e_routed)


@pytest.mark.parametrize("name", list(SMALL))
def test_small_layer_stages_match_oracle(name):
    import fine_grained_mixture_gemm_amd as moe
    print(f"[case] {name}", flush=True)
    g = H.build(SMALL[name])
    ws = H.workspace(g, poison=True)
    o = H.run_stages(g, ws)
    ref = _oracle_layer(g)
    errs = _check_all(g, o, ref)
    z = torch.empty((g.w.T, g.w.E), dtype=torch.float32, device="cuda")
    moe.moe_router_logits(g.cfg, g.layer, g.t["u"], z, ws)
    torch.cuda.synchronize()
    r = omoe.route(ref["z"], g.w.gate, g.w.K, g.bias, g.w.renorm, g.w.n_groups, g.w.topk_groups)
    H.check_key_margins(g, H.to_np(z), r["key"], r["gap"], name)
    print(name, errs)


@pytest.mark.parametrize("name", ["bf16_softmax_ragged", "fp8_sigmoid_ragged", "tiny_f32"])
def test_forward_equals_stages_and_is_deterministic(name):
    import fine_grained_mixture_gemm_amd as moe
    print(f"[case] {name}", flush=True)
    g = H.build(SMALL[name])
    ws = H.workspace(g, poison=True)
    o = H.run_stages(g, ws)
    outs = []
    for rep in range(2):
        ws.fill_(0xFF if rep == 0 else 0x00)
        h = torch.empty_like(o["h"])
        idx = torch.empty_like(o["idx"])
        cnt = torch.empty_like(o["counts"])
        moe.moe_forward(g.cfg, g.layer, g.t["u"], g.t["bias"], h, idx, cnt, ws)
        torch.cuda.synchronize()
        outs.append((h.clone(), idx.clone(), cnt.clone()))
    for h, idx, cnt in outs:
        assert torch.equal(idx, o["idx"]) and torch.equal(cnt, o["counts"])
        assert torch.equal(h.view(torch.int16) if h.dtype == torch.bfloat16 else h,
                           o["h"].view(torch.int16) if h.dtype == torch.bfloat16 else o["h"])


@pytest.mark.parametrize("name", ["tiny_f32", "dsmoe2b_bf16", "dsmoe16b_bf16"])
def test_full_size_float_configs(name):
    import fine_grained_mixture_gemm_amd as moe
    print(f"[case] {name}", flush=True)
    g = H.build(W[name])
    ws = H.workspace(g)
    o = H.run_stages(g, ws)
    ref = _oracle_layer(g)
    # the fp32 logits (softmax keys) stay 20x inside every token's recheck margin
    z = torch.empty((g.w.T, g.w.E), dtype=torch.float32, device="cuda")
    moe.moe_router_logits(g.cfg, g.layer, g.t["u"], z, ws)
    torch.cuda.synchronize()
    r = omoe.route(ref["z"], g.w.gate, g.w.K, g.bias, g.w.renorm, g.w.n_groups, g.w.topk_groups)
    H.check_key_margins(g, H.to_np(z), r["key"], r["gap"], name)
    print(name, _check_all(g, o, ref))


# Batches large enough for the 256-token x 128-expert MFMA logits blocks (about 256 blocks over four slices
# of d), with a ragged last token block (8000 = 31.25 x 256) and an expert count that is not a multiple of
# 128, softmax and sigmoid + bias keys, and heavy-tailed rows for the sigmoid case: routing bit for bit
# against the oracle, the fp32 keys inside the recheck margins.
ROUTER_LARGE = {
    "softmax": W["dsmoe2b_bf16"].replace(name="router_large_softmax", T=8000, d=2048, E=200, K=6, f=128),
    "sigmoid_tail": W["v3_fp8"].replace(name="router_large_sigmoid_tail", T=8000, d=2048, E=200, K=8, f=128,
                                        wdt="bf16", u_tail=True),
}


@pytest.mark.parametrize("name", list(ROUTER_LARGE))
def test_router_large_blocks_ragged(name):
    import fine_grained_mixture_gemm_amd as moe
    w = ROUTER_LARGE[name]
    # the library takes the large blocks when ceil(T / 256) ceil(E / 128) x 4 slices >= 256
    assert -(-w.T // 256) * -(-w.E // 128) * 4 >= 256
    print(f"[case] router large blocks {name}", flush=True)
    g = H.build(w, keep_host_weights=False)
    ws = H.workspace(g, poison=True)
    idx = torch.empty((w.T, w.K), dtype=torch.int32, device="cuda")
    gw = torch.empty((w.T, w.K), dtype=torch.float32, device="cuda")
    moe.moe_route(g.cfg, g.layer, g.t["u"], g.t["bias"], idx, gw, ws)
    z = torch.empty((w.T, w.E), dtype=torch.float32, device="cuda")
    moe.moe_router_logits(g.cfg, g.layer, g.t["u"], z, ws)
    torch.cuda.synchronize()
    zr, r = H.oracle_route(g)
    assert np.array_equal(H.to_np(idx), r["idx"]), "routing differs"
    assert np.abs(H.to_np(gw) - r["w"]).max() < 1e-5
    H.check_key_margins(g, H.to_np(z), r["key"], r["gap"], name)


# E4M3 with the smallest inner dim f = 128: a row of a is one 1x128 tile, so one requantized code of a
# that rounds the other way moves that row of y by about 0.3 * 3 / sqrt(128) = 8 % of its RMS, above the
# 6e-2 bar. Such a code is one whose input window (the gate/up GEMM's fp32 summation bound carried through
# SwiGLU, tests/e4m3_bounds.py) crosses a rounding midpoint or can move its tile's scale; the check
# compares per element |y - y_ref| <= 6e-2 RMS + 2^-8 |y_ref| (bf16 output) + sum_c |W2[i, c]| flip_a[r, c],
# and bounds the rest with the RMS error (<= 1e-2) and the plain maximum (<= 0.25 of the RMS).
F128 = {
    "fp8_f128_tiled": W["v3_fp8"].replace(name="fp8_f128_tiled", T=300, d=512, E=12, K=3, f=128),
    "fp8_f128_decode": W["v3_fp8"].replace(name="fp8_f128_decode", T=64, d=512, E=12, K=3, f=128),
}


def _flip_aware(y_gpu, y_ref, x, ex, what):
    from oracle import quant as oquant
    from tests import e4m3_bounds as EB
    (_, _, _, _), (a32, Da) = EB.forward_windows(x, ex[0], ex[1])
    code, scale = EB.flip(a32, Da, axis_tiles=1, parts=True)                # [n, f]
    flip_a = code + scale
    w2 = np.abs(oquant.dequant_weight(ex[2], ex[3]))                        # [d, f]
    allow = flip_a @ w2.T                                                   # [n, d]
    rms = np.sqrt(np.mean(y_ref ** 2))
    diff = np.abs(y_gpu - y_ref)
    excess = (diff - (H.TOL["fp8"] * rms + 2.0 ** -8 * np.abs(y_ref) + allow)).max() / rms
    rms_err, plain = np.sqrt(np.mean(diff ** 2)) / rms, diff.max() / rms
    assert excess <= 0, f"{what}: exceeds the flip-aware bound by {excess:.4f} RMS (plain {plain:.4f})"
    assert rms_err <= 1e-2 and plain <= 0.25, f"{what}: RMS error {rms_err:.4f}, plain {plain:.4f}"
    return plain, int((code > 0).sum())


@pytest.mark.parametrize("name", list(F128))
def test_fp8_inner_dim_128_flip_aware(name):
    w = F128[name]
    print(f"[case] {name}", flush=True)
    g = H.build(w)
    ws = H.workspace(g, poison=True)
    o = H.run_stages(g, ws)
    z = omoe.router_logits(g.u_host, g.wg, g.off)
    r = omoe.route(z, w.gate, w.K, g.bias, w.renorm)
    assert np.array_equal(H.to_np(o["idx"]), r["idx"]), "routing differs"
    offsets, perm, _ = omoe.dispatch(r["idx"], w.E)
    assert np.array_equal(H.to_np(o["offsets"]), offsets) and np.array_equal(H.to_np(o["perm"]), perm)
    y = H.to_np(o["y_r"])
    worst, flips = 0.0, 0
    for e in range(w.E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if a == b:
            continue
        ex = H.oracle_fp8_expert(w, e)
        x = g.u_host[perm[a:b]]
        p, nf = _flip_aware(y[a:b], omoe.swiglu_ffn_fp8(x, *ex)[0], x, ex, f"{name} expert {e}")
        worst, flips = max(worst, p), flips + nf
    ex = H.oracle_fp8_expert(w, -1)
    p, nf = _flip_aware(H.to_np(o["y_s"]), omoe.swiglu_ffn_fp8(g.u_host, *ex)[0], g.u_host, ex, f"{name} shared")
    worst, flips = max(worst, p), flips + nf
    print(f"{name}: worst plain max-abs/RMS {worst:.4f}, codes of a that may round either way {flips}")
