"""Shared set-up of the GPU parity tests: one seeded synthetic layer, built twice from ``synth`` alone,
once on the device through libmoe (for the kernels) and once on the host (for the oracle).

The oracle never sees a value produced by the HIP path: fp8 weights are quantized independently on
both sides from the same fp32 masters (the quantizers are compared bit for bit in the tests)."""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

import fine_grained_mixture_gemm_amd as moe
from oracle import moe as omoe, quant as oquant
from synth import configs, gen

DEV = "cuda"
TOL = {"f32": 1e-5, "bf16": 2e-2, "fp8": 6e-2}


def err(y, y_ref) -> float:
    """max |y - y_ref| / RMS(y_ref)."""
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    rms = np.sqrt(np.mean(y_ref ** 2))
    return float(np.abs(y - y_ref).max() / max(rms, 1e-300))


def err_rows(y, y_ref, slack=0.0) -> float:
    """max over rows of max(|y_r - y_ref_r| - slack_r) / RMS(y_ref_r): the tolerance applied row by row, for
    inputs whose rows differ in scale by orders of magnitude (heavy-tailed tokens), where one global RMS
    would let the large rows hide the small ones and hold the large ones to the small ones' scale. slack
    (per element, or 0) is the output format's own rounding, which an element far above its row's RMS
    carries in full (bf16 rounds by up to 2^-9 of the value)."""
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    rms = np.sqrt(np.mean(y_ref ** 2, axis=1))
    return float((np.maximum(np.abs(y - y_ref) - slack, 0.0).max(axis=1) / np.maximum(rms, 1e-300)).max())


def to_np(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.float().numpy().astype(np.float64)
    return t.numpy()


def bf16_tensor(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)


@dataclasses.dataclass
class GpuLayer:
    w: configs.Workload
    cfg: moe.moe_config
    layer: moe.moe_layer
    t: dict                      # device tensors, kept alive
    u_host: np.ndarray           # u as stored (fp32 values)
    wg: np.ndarray
    bias: Optional[np.ndarray]
    off: Optional[np.ndarray]
    host_experts: Optional[list] = None   # float path: [(w1, w3, w2)] stored values
    host_shared: Optional[tuple] = None


def make_cfg(w: configs.Workload) -> moe.moe_config:
    return moe.make_config(w.T, w.d, w.E, w.Ks, w.K, w.f,
                           moe.MOE_GATE_SOFTMAX if w.gate == "softmax" else moe.MOE_GATE_SIGMOID_BIAS, w.renorm,
                           moe.MOE_F32 if w.act == "f32" else moe.MOE_BF16,
                           {"f32": moe.MOE_F32, "bf16": moe.MOE_BF16, "fp8": moe.MOE_FP8_E4M3}[w.wdt],
                           w.n_groups, w.topk_groups)


def _store(x32: np.ndarray, wdt: str) -> tuple[torch.Tensor, np.ndarray]:
    """Device tensor in the weight dtype and the stored values as fp32 on the host."""
    if wdt == "f32":
        return torch.from_numpy(np.ascontiguousarray(x32)), x32
    bits = gen.f32_to_bf16_bits(x32)
    return bf16_tensor(bits), gen.bf16_bits_to_f32(bits)


def build(w: configs.Workload, keep_host_weights: bool = True) -> GpuLayer:
    """Float weights (f32 / bf16) are generated on the host and uploaded; fp8 weights are generated on
    the device by the synth fill and quantized there by libmoe (and independently by the oracle)."""
    u = configs.make_u(w)
    u_host = configs.u_as_f32(w, u)
    wg, bias, off = configs.make_router(w)
    t = {}
    t["u"] = (torch.from_numpy(u) if w.act == "f32" else bf16_tensor(u)).to(DEV)
    t["wg"] = torch.from_numpy(wg).to(DEV)
    t["bias"] = torch.from_numpy(bias).to(DEV) if bias is not None else None
    t["off"] = torch.from_numpy(off).to(DEV) if off is not None else None
    host_experts, host_shared = None, None
    if w.wdt in ("f32", "bf16"):
        dt = torch.float32 if w.wdt == "f32" else torch.bfloat16
        w13 = torch.empty((w.E, 2 * w.f, w.d), dtype=dt)
        w2 = torch.empty((w.E, w.d, w.f), dtype=dt)
        host_experts = []
        for e in range(w.E):
            a1, h1 = _store(configs.master_w1(w, e), w.wdt)
            a3, h3 = _store(configs.master_w3(w, e), w.wdt)
            a2, h2 = _store(configs.master_w2(w, e), w.wdt)
            w13[e, :w.f], w13[e, w.f:], w2[e] = a1, a3, a2
            if keep_host_weights:
                host_experts.append((h1, h3, h2))
        t["w13"], t["w2"] = w13.to(DEV), w2.to(DEV)
        if w.Ks > 0:
            a1, h1 = _store(configs.master_w1(w, -1), w.wdt)
            a3, h3 = _store(configs.master_w3(w, -1), w.wdt)
            a2, h2 = _store(configs.master_w2(w, -1), w.wdt)
            t["ws13"] = torch.cat([a1, a3], 0).to(DEV)
            t["ws2"] = a2.to(DEV)
            host_shared = (h1, h3, h2)
        layer = moe.make_layer(t["w13"], t["w2"], t["wg"], ws13=t.get("ws13"), ws2=t.get("ws2"),
                               logit_offset=t["off"])
    else:
        t.update(quantize_fp8_weights_on_device(w))
        layer = moe.make_layer(t["w13"], t["w2"], t["wg"], ws13=t.get("ws13"), ws2=t.get("ws2"),
                               w13_scale=t["w13s"], w2_scale=t["w2s"], ws13_scale=t.get("ws13s"),
                               ws2_scale=t.get("ws2s"), logit_offset=t["off"])
    return GpuLayer(w, make_cfg(w), layer, t, u_host, wg, bias, off, host_experts, host_shared)


def quantize_fp8_weights_on_device(w: configs.Workload, chunk: int = 16) -> dict:
    """fp32 masters filled on the device, E4M3 + 128x128 scales by libmoe, `chunk` experts at a time."""
    from synth import device as sdev
    out = {
        "w13": torch.empty((w.E, 2 * w.f, w.d), dtype=torch.uint8, device=DEV),
        "w13s": torch.empty((w.E, 2 * w.f // 128, w.d // 128), dtype=torch.float32, device=DEV),
        "w2": torch.empty((w.E, w.d, w.f), dtype=torch.uint8, device=DEV),
        "w2s": torch.empty((w.E, w.d // 128, w.f // 128), dtype=torch.float32, device=DEV),
    }
    tmp13 = torch.empty((chunk, 2 * w.f, w.d), dtype=torch.float32, device=DEV)
    tmp2 = torch.empty((chunk, w.d, w.f), dtype=torch.float32, device=DEV)
    for e0 in range(0, w.E, chunk):
        n = min(chunk, w.E - e0)
        for i in range(n):
            e = e0 + i
            sdev.fill_normal(tmp13[i, :w.f], w.seed, configs.stream_routed(e, 0), configs.sigma_in(w))
            sdev.fill_normal(tmp13[i, w.f:], w.seed, configs.stream_routed(e, 1), configs.sigma_in(w))
            sdev.fill_normal(tmp2[i], w.seed, configs.stream_routed(e, 2), configs.sigma_down(w))
        moe.moe_quantize_weights(tmp13[:n], out["w13"][e0:e0 + n], out["w13s"][e0:e0 + n])
        moe.moe_quantize_weights(tmp2[:n], out["w2"][e0:e0 + n], out["w2s"][e0:e0 + n])
    del tmp13, tmp2
    if w.Ks > 0:
        s13 = torch.empty((2 * w.fs, w.d), dtype=torch.float32, device=DEV)
        sdev.fill_normal(s13[:w.fs], w.seed, configs.STREAM_SH_W1, configs.sigma_in(w))
        sdev.fill_normal(s13[w.fs:], w.seed, configs.STREAM_SH_W3, configs.sigma_in(w))
        s2 = torch.empty((w.d, w.fs), dtype=torch.float32, device=DEV)
        sdev.fill_normal(s2, w.seed, configs.STREAM_SH_W2, configs.sigma_down(w))
        out["ws13"] = torch.empty((2 * w.fs, w.d), dtype=torch.uint8, device=DEV)
        out["ws13s"] = torch.empty((2 * w.fs // 128, w.d // 128), dtype=torch.float32, device=DEV)
        out["ws2"] = torch.empty((w.d, w.fs), dtype=torch.uint8, device=DEV)
        out["ws2s"] = torch.empty((w.d // 128, w.fs // 128), dtype=torch.float32, device=DEV)
        moe.moe_quantize_weights(s13, out["ws13"], out["ws13s"])
        moe.moe_quantize_weights(s2, out["ws2"], out["ws2s"])
    torch.cuda.synchronize()
    return out


def oracle_fp8_expert(w: configs.Workload, e: int):
    """The oracle's own E4M3 weights of routed expert e (or the shared block for e < 0)."""
    w13q, w13s = oquant.quantize_weight_128x128(np.vstack([configs.master_w1(w, e), configs.master_w3(w, e)]))
    w2q, w2s = oquant.quantize_weight_128x128(configs.master_w2(w, e))
    return w13q, w13s, w2q, w2s


def workspace(g: GpuLayer, poison: bool = False) -> torch.Tensor:
    n = moe.moe_workspace_size(g.cfg)
    ws = torch.empty(n, dtype=torch.uint8, device=DEV)
    if poison:
        ws.fill_(0xFF)           # NaN in every float view, -1 in every int view
    return ws


def y_dtype(w: configs.Workload):
    return torch.bfloat16 if w.wdt == "fp8" else torch.float32


def run_stages(g: GpuLayer, ws: torch.Tensor) -> dict:
    """moe_route -> moe_dispatch -> moe_expert_ffn -> moe_combine, every intermediate returned."""
    w = g.w
    T, K, E, d = w.T, w.K, w.E, w.d
    o = {
        "idx": torch.empty((T, K), dtype=torch.int32, device=DEV),
        "gw": torch.empty((T, K), dtype=torch.float32, device=DEV),
        "counts": torch.empty(E, dtype=torch.int32, device=DEV),
        "offsets": torch.empty(E + 1, dtype=torch.int32, device=DEV),
        "perm": torch.empty(T * K, dtype=torch.int32, device=DEV),
        "row_of": torch.empty((T, K), dtype=torch.int32, device=DEV),
        "y_r": torch.empty((T * K, d), dtype=y_dtype(w), device=DEV),
        "y_s": torch.empty((T, d), dtype=y_dtype(w), device=DEV) if w.Ks > 0 else None,
        "h": torch.empty((T, d), dtype=g.t["u"].dtype, device=DEV),
    }
    moe.moe_route(g.cfg, g.layer, g.t["u"], g.t["bias"], o["idx"], o["gw"], ws)
    moe.moe_dispatch(g.cfg, o["idx"], o["counts"], o["offsets"], o["perm"], o["row_of"], ws)
    moe.moe_expert_ffn(g.cfg, g.layer, g.t["u"], o["offsets"], o["perm"], o["y_r"], o["y_s"], ws)
    moe.moe_combine(g.cfg, g.t["u"], o["y_r"], o["y_s"], o["row_of"], o["gw"], o["h"])
    torch.cuda.synchronize()
    return o


def oracle_route(g: GpuLayer):
    w = g.w
    z = omoe.router_logits(g.u_host, g.wg, g.off)
    return z, omoe.route(z, w.gate, w.K, g.bias, w.renorm)


def token_margins(cfg, u_host: np.ndarray, wg: np.ndarray) -> np.ndarray:
    """The router's recheck margin of every token, as the header states it:
    delta * max(1, |u_t| max_i |e_i| / sqrt(d)), delta from the library (moe_route_margin)."""
    delta = moe.moe_route_margin(cfg)
    un = np.sqrt((np.asarray(u_host, dtype=np.float64) ** 2).sum(axis=1))
    wn = np.sqrt((np.asarray(wg, dtype=np.float64) ** 2).sum(axis=1)).max()
    return delta * np.maximum(1.0, un * wn / np.sqrt(u_host.shape[1]))


def check_key_margins(g, z32: np.ndarray, ref_key: np.ndarray, gap: np.ndarray, label: str = "") -> None:
    """The fp32 keys the router compares stay 20x inside each token's recheck margin (so every token whose
    selection the fp32 keys could get wrong is decided again in fp64), and no fp64 near-tie makes the
    selection ill-defined."""
    w = g.w
    bias = g.bias if (w.gate == "sigmoid_bias" and g.bias is not None) else None
    key32 = 1.0 / (1.0 + np.exp(-z32.astype(np.float64))) if w.gate == "sigmoid_bias" else z32.astype(np.float64)
    key64 = ref_key - (bias[None, :] if bias is not None else 0.0)
    kerr = np.abs(key32 - key64).max(axis=1)
    margin = token_margins(g.cfg, g.u_host, g.wg)
    worst = float((kerr * 20 / margin).max())
    print(f"{label}: max fp32 key error {kerr.max():.3e}, worst 20 x error / margin {worst:.3f}, margin "
          f"{margin.min():.2e}..{margin.max():.2e}, min fp64 gap {gap.min():.3e}, tokens under their margin "
          f"{int((gap < margin).sum())}", flush=True)
    assert worst <= 1.0, "fp32 keys are not 20x inside the recheck margin"
    assert gap.min() > 1e-9, "an fp64 near-tie would make the selection ill-defined"

