"""The tiled weight layout (moe_pack_weights): its byte order against the definition in include/moe.h,
and the expert GEMMs on tiled weights bit for bit equal to the same GEMMs on row-major weights: the forward
on the tiled and the decode-batch kernels, bf16 and E4M3, and the E4M3 input backward. The layout changes
where the weight bytes sit, not one operation of the arithmetic, so every result is identical."""
import numpy as np
import pytest
import torch

import fine_grained_mixture_gemm_amd as moe
from synth import configs
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

W = configs.WORKLOADS


def tiled_reference(m: np.ndarray, gateup: bool) -> np.ndarray:
    """uint8 [groups, rows, row_bytes] in the tiled layout, from the header's index formula: tile n of 256
    rows (gate/up: W1 rows 128 n.. then W3 rows rows/2 + 128 n..; else rows 256 n..), K stage k, 16-row
    block b, chunk c of row r at byte (n * stages + k) * 32768 + 2048 b + 16 (64 (c / 4) + 16 (c % 4) + r)."""
    G, R, C = m.shape
    stages, ntiles = C // 128, R // 256
    # destination order: (n, k, b, c // 4, c % 4, r), C-contiguous
    n, k, b, h, q, r = np.meshgrid(np.arange(ntiles), np.arange(stages), np.arange(16), np.arange(2), np.arange(4),
                                   np.arange(16), indexing="ij")
    if gateup:
        row = np.where(b < 8, 128 * n + 16 * b, R // 2 + 128 * n + 16 * (b - 8)) + r
    else:
        row = 256 * n + 16 * b + r
    chunk = k * 8 + 4 * h + q                    # 16-byte chunk index within the row
    out = np.stack([m[g].reshape(R, C // 16, 16)[row.ravel(), chunk.ravel()] for g in range(G)])
    return out.reshape(G, R, C)


def _tiled_copy(cfg, which, src):
    dst = torch.empty_like(src)
    moe.moe_pack_weights(cfg, which, src, dst)
    return dst


@pytest.mark.parametrize("wdt", ["fp8", "bf16"])
def test_pack_matches_definition(wdt):
    w = (W["v3_fp8"].replace(name="pack_fp8", T=8, d=512, E=3, Ks=2, K=2, f=256) if wdt == "fp8" else
         W["dsmoe16b_bf16"].replace(name="pack_bf16", T=8, d=256, E=2, Ks=1, K=2, f=384))
    print(f"[case] pack {wdt}", flush=True)
    cfg = H.make_cfg(w)
    esz = 1 if wdt == "fp8" else 2
    rng = np.random.default_rng(5)
    shapes = {moe.MOE_PACK_W13: (w.E, 2 * w.f, w.d), moe.MOE_PACK_W2: (w.E, w.d, w.f),
              moe.MOE_PACK_WS13: (1, 2 * w.fs, w.d), moe.MOE_PACK_WS2: (1, w.d, w.fs)}
    if wdt == "fp8":
        # the backward's transposed weights, in plain 256-row tiles
        shapes.update({moe.MOE_PACK_W13T: (w.E, w.d, 2 * w.f), moe.MOE_PACK_W2T: (w.E, w.f, w.d),
                       moe.MOE_PACK_WS13T: (1, w.d, 2 * w.fs), moe.MOE_PACK_WS2T: (1, w.fs, w.d)})
    for which, (G, R, C) in shapes.items():
        host = rng.integers(0, 256, size=(G, R, C * esz), dtype=np.uint8)
        src = torch.from_numpy(host).to(H.DEV)
        dst = _tiled_copy(cfg, which, src)
        torch.cuda.synchronize()
        gateup = which in (moe.MOE_PACK_W13, moe.MOE_PACK_WS13)
        assert np.array_equal(dst.cpu().numpy(), tiled_reference(host, gateup)), f"layout of matrix {which}"


def _tiled_layer(g):
    """g's layer with its expert weights copied into the tiled layout (tensors kept in g.t)."""
    t = g.t
    for key, which in (("w13", moe.MOE_PACK_W13), ("w2", moe.MOE_PACK_W2), ("ws13", moe.MOE_PACK_WS13),
                       ("ws2", moe.MOE_PACK_WS2)):
        if key in t:
            src = t[key] if t[key].dtype == torch.uint8 else t[key].view(torch.uint8)
            t[key + "_tiled"] = _tiled_copy(g.cfg, which, src)
    torch.cuda.synchronize()
    return moe.make_layer(t["w13_tiled"], t["w2_tiled"], t["wg"], ws13=t.get("ws13_tiled"), ws2=t.get("ws2_tiled"),
                          w13_scale=t.get("w13s"), w2_scale=t.get("w2s"), ws13_scale=t.get("ws13s"),
                          ws2_scale=t.get("ws2s"), logit_offset=t["off"], weight_layout=moe.MOE_LAYOUT_TILED)


FORWARD = {
    # the tiled kernel (E4M3, 300 tokens; shared block; ragged groups), the decode-batch kernel (64 tokens)
    "fp8_tiled": W["v3_fp8"].replace(name="fp8_tiled", T=300, d=512, E=20, K=4),
    "fp8_decode": W["v3_fp8"].replace(name="fp8_decode", T=64, d=512, E=20, K=4),
    # bf16 on the tiled kernel: two shared experts (fs = 512) and f = 384 (N tiles of the shared block
    # and of the routed experts differ), and the 2B shape with f = 128
    "bf16_2shared": W["dsmoe16b_bf16"].replace(name="bf16_2shared", T=600, d=512, E=16, K=6, f=384),
    "bf16_f128": W["dsmoe2b_bf16"].replace(name="bf16_f128", T=300, d=256, E=12, K=3, f=128),
}


@pytest.mark.parametrize("name", list(FORWARD))
def test_tiled_forward_is_bit_identical(name):
    w = FORWARD[name]
    print(f"[case] {name}", flush=True)
    g = H.build(w, keep_host_weights=False)
    layer_tiled = _tiled_layer(g)
    ws = H.workspace(g)
    out = {}
    for lay, layer in (("rows", g.layer), ("tiled", layer_tiled)):
        g.layer = layer
        o = H.run_stages(g, ws)
        h2 = torch.empty_like(o["h"])
        idx = torch.empty_like(o["idx"])
        counts = torch.empty_like(o["counts"])
        moe.moe_forward(g.cfg, layer, g.t["u"], g.t["bias"], h2, idx, counts, ws)
        torch.cuda.synchronize()
        out[lay] = {k: v.cpu() for k, v in o.items() if v is not None}
        out[lay]["h_forward"] = h2.cpu()
    for k in out["rows"]:
        a, b = out["rows"][k].contiguous().view(torch.uint8), out["tiled"][k].contiguous().view(torch.uint8)
        assert torch.equal(a, b), f"{name}: {k} differs between the row and the tiled layout"


def _tiled_transposed_layer(g, tt):
    """The transposed weights of the backward (tt, row layout) copied into the tiled layout."""
    out = {}
    for key, which in (("w13", moe.MOE_PACK_W13T), ("w2", moe.MOE_PACK_W2T), ("ws13", moe.MOE_PACK_WS13T),
                       ("ws2", moe.MOE_PACK_WS2T)):
        if key in tt:
            out[key] = _tiled_copy(g.cfg, which, tt[key])
    torch.cuda.synchronize()
    layer = moe.make_layer(out["w13"], out["w2"], g.t["wg"], ws13=out.get("ws13"), ws2=out.get("ws2"),
                           w13_scale=tt["w13s"], w2_scale=tt["w2s"], ws13_scale=tt.get("ws13s"),
                           ws2_scale=tt.get("ws2s"), weight_layout=moe.MOE_LAYOUT_TILED)
    return layer, out


def test_tiled_backward_is_bit_identical():
    """Input and weight gradients with the forward and the transposed weights tiled, against both in rows."""
    from tests.test_gpu_backward import _bf16_normal, _transposed_layer
    w = W["v3_fp8"].replace(name="bwd_tiled", T=160, d=512, E=16, K=4)
    print("[case] bwd_tiled", flush=True)
    g = H.build(w, keep_host_weights=False)
    layer_tiled = _tiled_layer(g)
    ws = H.workspace(g)
    o = H.run_stages(g, ws)
    layer_t, tt = _transposed_layer(g)
    layer_t_tiled, _keep = _tiled_transposed_layer(g, tt)
    rng = np.random.default_rng(11)
    dy_r, _ = _bf16_normal(rng, (w.T * w.K, w.d))
    dy_s, _ = _bf16_normal(rng, (w.T, w.d))
    bws = torch.empty(moe.moe_backward_workspace_size(g.cfg), dtype=torch.uint8, device=H.DEV)
    bf = dict(dtype=torch.bfloat16, device=H.DEV)
    res = []
    for layer, lt in ((g.layer, layer_t), (layer_tiled, layer_t_tiled), (layer_tiled, layer_t)):
        out = [torch.empty((w.T * w.K, w.d), **bf), torch.empty((w.T, w.d), **bf),
               torch.empty((w.E, 2 * w.f, w.d), **bf), torch.empty((w.E, w.d, w.f), **bf),
               torch.empty((2 * w.fs, w.d), **bf), torch.empty((w.d, w.fs), **bf)]
        moe.moe_expert_ffn_backward(g.cfg, layer, lt, g.t["u"], o["offsets"], o["perm"], dy_r, dy_s, *out, bws)
        torch.cuda.synchronize()
        res.append([x.view(torch.int16).cpu() for x in out])
    for k in (1, 2):
        for i, nm in enumerate(("dx_r", "dx_s", "dw13", "dw2", "dws13", "dws2")):
            assert torch.equal(res[0][i], res[k][i]), f"{nm} differs between the layouts (case {k})"
