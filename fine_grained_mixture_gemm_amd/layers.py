"""Device-side set-up of a seeded synthetic layer (plumbing around libmoe, used by bench.py and smoke()).

Inputs come from ``synth`` (the same counter-based generator the oracle side uses): u and the expert
weights are filled on the device, the router tensors are made on the host. E4M3 weights are produced
from their fp32 masters by libmoe's own 128x128 block quantizer, a few experts at a time.
"""
from __future__ import annotations

import dataclasses

import torch

from synth import configs, device as sdev

from . import (MOE_BF16, MOE_F32, MOE_FP8_E4M3, MOE_GATE_SIGMOID_BIAS, MOE_GATE_SOFTMAX, MOE_LAYOUT_ROWS,
               MOE_LAYOUT_TILED, MOE_PACK_W13, MOE_PACK_W2, MOE_PACK_WS13, MOE_PACK_WS2, make_config, make_layer,
               moe_pack_weights, moe_quantize_weights)


@dataclasses.dataclass
class DeviceLayer:
    w: configs.Workload
    cfg: object
    layer: object
    t: dict     # device tensors kept alive for `layer`; w13, w2, ws13, ws2 always in the row layout


def workload_config(w: configs.Workload):
    return make_config(w.T, w.d, w.E, w.Ks, w.K, w.f, MOE_GATE_SOFTMAX if w.gate == "softmax" else MOE_GATE_SIGMOID_BIAS,
                       w.renorm, MOE_F32 if w.act == "f32" else MOE_BF16,
                       {"f32": MOE_F32, "bf16": MOE_BF16, "fp8": MOE_FP8_E4M3}[w.wdt], w.n_groups, w.topk_groups)


def _fill_w13(dst, w, e, rows):
    """dst [2*rows, d]: W1 (gate) rows then W3 (up) rows of routed expert e (e < 0: the shared block)."""
    s1 = configs.STREAM_SH_W1 if e < 0 else configs.stream_routed(e, 0)
    s3 = configs.STREAM_SH_W3 if e < 0 else configs.stream_routed(e, 1)
    sdev.fill_normal(dst[:rows], w.seed, s1, configs.sigma_in(w))
    sdev.fill_normal(dst[rows:], w.seed, s3, configs.sigma_in(w))


def _fill_w2(dst, w, e):
    sdev.fill_normal(dst, w.seed, configs.STREAM_SH_W2 if e < 0 else configs.stream_routed(e, 2), configs.sigma_down(w))


def _tiled(cfg, t, layer_args):
    """Copies of the expert weights in the tiled layout (the form the expert GEMMs stream fastest); the
    row-layout tensors stay in t for callers that need them (the backward's transposed weights)."""
    for key, which in (("w13", MOE_PACK_W13), ("w2", MOE_PACK_W2), ("ws13", MOE_PACK_WS13), ("ws2", MOE_PACK_WS2)):
        if key in t:
            t[key + "_tiled"] = torch.empty_like(t[key])
            moe_pack_weights(cfg, which, t[key], t[key + "_tiled"])
    for key in ("w13", "w2", "ws13", "ws2"):
        if key in t:
            layer_args[key] = t[key + "_tiled"]
    layer_args["weight_layout"] = MOE_LAYOUT_TILED


def device_layer(w: configs.Workload, device: str = "cuda", chunk: int = 16, tiled: bool = True) -> DeviceLayer:
    """The workload's layer on the device. tiled: bf16 / fp8 expert weights in the tiled layout (the
    layer struct points at those copies); fp32 weights are always row-major."""
    t = {}
    adt = torch.float32 if w.act == "f32" else torch.bfloat16
    t["u"] = sdev.fill_normal(torch.empty((w.T, w.d), dtype=adt, device=device), w.seed, configs.STREAM_U, 1.0)
    wg, bias, off = configs.make_router(w)
    t["wg"] = torch.from_numpy(wg).to(device)
    t["bias"] = torch.from_numpy(bias).to(device) if bias is not None else None
    t["off"] = torch.from_numpy(off).to(device) if off is not None else None
    if w.wdt in ("f32", "bf16"):
        wdt = torch.float32 if w.wdt == "f32" else torch.bfloat16
        t["w13"] = torch.empty((w.E, 2 * w.f, w.d), dtype=wdt, device=device)
        t["w2"] = torch.empty((w.E, w.d, w.f), dtype=wdt, device=device)
        for e in range(w.E):
            _fill_w13(t["w13"][e], w, e, w.f)
            _fill_w2(t["w2"][e], w, e)
        if w.Ks > 0:
            t["ws13"] = torch.empty((2 * w.fs, w.d), dtype=wdt, device=device)
            t["ws2"] = torch.empty((w.d, w.fs), dtype=wdt, device=device)
            _fill_w13(t["ws13"], w, -1, w.fs)
            _fill_w2(t["ws2"], w, -1)
        args = dict(w13=t["w13"], w2=t["w2"], w_gate=t["wg"], ws13=t.get("ws13"), ws2=t.get("ws2"),
                    logit_offset=t["off"], weight_layout=MOE_LAYOUT_ROWS)
        if tiled and w.wdt == "bf16":
            _tiled(workload_config(w), t, args)
        layer = make_layer(**args)
    else:
        t["w13"] = torch.empty((w.E, 2 * w.f, w.d), dtype=torch.uint8, device=device)
        t["w13s"] = torch.empty((w.E, 2 * w.f // 128, w.d // 128), dtype=torch.float32, device=device)
        t["w2"] = torch.empty((w.E, w.d, w.f), dtype=torch.uint8, device=device)
        t["w2s"] = torch.empty((w.E, w.d // 128, w.f // 128), dtype=torch.float32, device=device)
        tmp13 = torch.empty((chunk, 2 * w.f, w.d), dtype=torch.float32, device=device)
        tmp2 = torch.empty((chunk, w.d, w.f), dtype=torch.float32, device=device)
        for e0 in range(0, w.E, chunk):
            n = min(chunk, w.E - e0)
            for i in range(n):
                _fill_w13(tmp13[i], w, e0 + i, w.f)
                _fill_w2(tmp2[i], w, e0 + i)
            moe_quantize_weights(tmp13[:n], t["w13"][e0:e0 + n], t["w13s"][e0:e0 + n])
            moe_quantize_weights(tmp2[:n], t["w2"][e0:e0 + n], t["w2s"][e0:e0 + n])
        del tmp13, tmp2
        if w.Ks > 0:
            s13 = torch.empty((2 * w.fs, w.d), dtype=torch.float32, device=device)
            s2 = torch.empty((w.d, w.fs), dtype=torch.float32, device=device)
            _fill_w13(s13, w, -1, w.fs)
            _fill_w2(s2, w, -1)
            t["ws13"] = torch.empty((2 * w.fs, w.d), dtype=torch.uint8, device=device)
            t["ws13s"] = torch.empty((2 * w.fs // 128, w.d // 128), dtype=torch.float32, device=device)
            t["ws2"] = torch.empty((w.d, w.fs), dtype=torch.uint8, device=device)
            t["ws2s"] = torch.empty((w.d // 128, w.fs // 128), dtype=torch.float32, device=device)
            moe_quantize_weights(s13, t["ws13"], t["ws13s"])
            moe_quantize_weights(s2, t["ws2"], t["ws2s"])
            del s13, s2
        args = dict(w13=t["w13"], w2=t["w2"], w_gate=t["wg"], ws13=t.get("ws13"), ws2=t.get("ws2"),
                    w13_scale=t["w13s"], w2_scale=t["w2s"], ws13_scale=t.get("ws13s"), ws2_scale=t.get("ws2s"),
                    logit_offset=t["off"], weight_layout=MOE_LAYOUT_ROWS)
        if tiled:
            _tiled(workload_config(w), t, args)
        layer = make_layer(**args)
    torch.cuda.synchronize()
    return DeviceLayer(w, workload_config(w), layer, t)
