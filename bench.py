#!/usr/bin/env python3
"""Throughput of the DeepSeekMoE layer forward on one MI355X.

One step = the whole hot path on one batch of seeded synthetic tokens: router (logits, gating, top-K),
dispatch, the grouped expert GEMMs (gate/up + SwiGLU, down), combine, and the bias update when the
workload has one. Inputs and weights are resident in HBM before timing starts. The default workload is
the V3-shaped layer: T = 8192 tokens, d = 7168, 1 shared + 256 routed SwiGLU experts of inner dim 2048,
sigmoid affinity + selection bias, top-8, renormalised gates, E4M3 experts with 1x128 / 128x128 scales.

The step is captured once into a HIP graph and the timed steps are replays of it (`launch`; the eager
time of the same steps is `eager_ms_per_step`). Prints ONE JSON line. `roofline` covers the dominant kernel
(the gate/up grouped GEMM), timed live with HIP events on the launch stream over the eager timed steps; `configs` holds the same record for the other
configurations (the 2B and 16B bf16 layers and the 64-token V3 decode step), each timed in a run of its
own after the headline; `cpu_baseline` times the float64 CPU oracle on a bounded sample of the headline
workload on this host, scaled to the whole batch.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE layer tokens/sec + grouped-GEMM TFLOPS (% MFMA peak), V3-shaped layer, 1 GPU"
PEAK = {"fp8": 5.0e15, "bf16": 2.5e15, "f32": 157.3e12, "hbm": 8.0e12}


def note(msg):
    """Progress on stderr (stdout carries only the JSON line)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="v3_fp8")
    ap.add_argument("--tokens", type=int, default=0,
                    help="run the workload's layer with this many tokens instead (a sweep over batch sizes; the "
                         "workload name gains a _t<T> suffix and no profiled traffic is attached)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true", help="skip timing the E4M3 expert backward")
    ap.add_argument("--no-subconfigs", action="store_true",
                    help="skip the timed runs of the other configurations (2B / 16B bf16 layers, V3 decode step)")
    ap.add_argument("--no-graph", action="store_true",
                    help="time the eager steps only (no HIP-graph capture; for profiler runs)")
    ap.add_argument("--sub-steps", type=int, default=300)
    ap.add_argument("--sub-warmup", type=int, default=20)
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="first run one plain device copy of this many MiB (a known-size kernel that profiler "
                         "counters of HBM traffic are scaled against)")
    return ap.parse_args()


def kernel_work(w, counts):
    """Algorithmic FLOPs and HBM bytes of the two grouped GEMM launches (each input and output once,
    weights of the experts that received tokens)."""
    touched = int((counts > 0).sum())
    rows = w.T * w.K
    ew = {"f32": 4, "bf16": 2, "fp8": 1}[w.wdt]
    ex = 1 if w.wdt == "fp8" else (4 if w.act == "f32" else 2)     # activation bytes fed to gate/up
    ea = {"f32": 4, "bf16": 2, "fp8": 1}[w.wdt]                       # SwiGLU output bytes
    ey = 2 if w.wdt == "fp8" else 4                                    # expert output bytes
    sc = 4 if w.wdt == "fp8" else 0
    g = {
        "flops": 2.0 * w.d * 2 * w.f * rows + 2.0 * w.d * 2 * w.fs * w.T,
        "bytes": (touched * 2 * w.f * w.d * ew + touched * (2 * w.f // 128) * (w.d // 128) * sc
                  + 2 * w.fs * w.d * ew + (2 * w.fs // 128) * (w.d // 128) * sc * (w.Ks > 0)
                  + w.T * w.d * ex + w.T * (w.d // 128) * sc
                  + (rows * w.f + w.T * w.fs) * ea + (rows * (w.f // 128) + w.T * (w.fs // 128)) * sc),
    }
    dn = {
        "flops": 2.0 * w.f * w.d * rows + 2.0 * w.fs * w.d * w.T,
        "bytes": (touched * w.d * w.f * ew + touched * (w.d // 128) * (w.f // 128) * sc
                  + w.d * w.fs * ew + (w.d // 128) * (w.fs // 128) * sc * (w.Ks > 0)
                  + (rows * w.f + w.T * w.fs) * ea + (rows * (w.f // 128) + w.T * (w.fs // 128)) * sc
                  + (rows + w.T * (w.Ks > 0)) * w.d * ey),
    }
    return g, dn, touched


def roofline(work, ms, peak_mfma):
    t = ms * 1e-3
    t_mfma = work["flops"] / peak_mfma
    t_hbm = work["bytes"] / PEAK["hbm"]
    if t_hbm >= t_mfma:
        ach = work["bytes"] / t / 1e9
        return {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK["hbm"] / 1e9, "unit": "GB/s",
                "frac": round(ach / (PEAK["hbm"] / 1e9), 4), "traffic": None}
    ach = work["flops"] / t / 1e12
    return {"bound": "mfma", "achieved": round(ach, 1), "peak": peak_mfma / 1e12, "unit": "TFLOP/s",
            "frac": round(ach / (peak_mfma / 1e12), 4), "traffic": None}


def gateup_kernel_name(w):
    """The kernel that runs the gate/up projection of workload w (the library picks it from the config)."""
    if w.wdt == "f32":
        return "grouped_gemm_simt gate/up"
    if w.wdt == "fp8" and w.T <= 128:
        return "grouped_gemm_decode gate/up+SwiGLU"
    return "grouped_gemm_mfma gate/up+SwiGLU"


def profiled_traffic(workload):
    """HBM bytes per launch of the two grouped GEMM kernels from the committed counter profile of this
    workload (profiles/traffic_<workload>.json), or None when the kernel source changed since."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    src = open(os.path.join(ROOT, rec["kernel_source"]), "rb").read()
    if hashlib.sha256(src).hexdigest() != rec["source_sha256"]:
        return None
    return rec


def time_balance_stats(moe, L, w, ws, reps=20):
    """Time moe_balance_stats (f, P, expert-level and sequence-wise losses) on the router outputs of the
    workload; not part of the step. Sequences of 4096 tokens when they divide T, else one sequence."""
    import torch
    seq = 4096 if w.T % 4096 == 0 else w.T
    z = torch.empty((w.T, w.E), dtype=torch.float32, device="cuda")
    idx = torch.empty((w.T, w.K), dtype=torch.int32, device="cuda")
    gw = torch.empty((w.T, w.K), dtype=torch.float32, device="cuda")
    moe.moe_router_logits(L.cfg, L.layer, L.t["u"], z, ws)
    moe.moe_route(L.cfg, L.layer, L.t["u"], L.t["bias"], idx, gw, ws)
    f = torch.empty(w.E, dtype=torch.float32, device="cuda")
    P = torch.empty_like(f)
    loss = torch.empty(2, dtype=torch.float32, device="cuda")
    run = lambda: moe.moe_balance_stats(L.cfg, z, idx, seq, 0.003, 0.0001, f, P, loss, ws)
    run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        run()
    e1.record()
    torch.cuda.synchronize()
    return {"ms": round(e0.elapsed_time(e1) / reps, 4), "seq_len": seq,
            "loss_expert": float(loss[0]), "loss_seq": float(loss[1])}


def time_backward(moe, L, w, ws, reps=5):
    """Time the E4M3 expert backward on the workload's routing with a seeded bf16 gradient (not part of
    the step): moe_expert_ffn_backward_input, and moe_expert_ffn_backward with the weight gradients too.
    Algorithmic FLOPs per row (routed and shared): input 10 d f (g/v recompute 4 d f, da 2 d f, dx 4 d f),
    weights 6 d f (dW2 2 d f, d[W1; W3] 4 d f)."""
    import torch
    dev = "cuda"
    t = L.t

    def tr(q, s):
        qt = torch.empty(q.shape[:-2] + (q.shape[-1], q.shape[-2]), dtype=torch.uint8, device=dev)
        st = torch.empty(s.shape[:-2] + (s.shape[-1], s.shape[-2]), dtype=torch.float32, device=dev)
        moe.moe_transpose_fp8_weights(q, s, qt, st)
        return qt, st

    tt = {}
    tt["w13"], tt["w13s"] = tr(t["w13"], t["w13s"])
    tt["w2"], tt["w2s"] = tr(t["w2"], t["w2s"])
    if w.Ks > 0:
        tt["ws13"], tt["ws13s"] = tr(t["ws13"], t["ws13s"])
        tt["ws2"], tt["ws2s"] = tr(t["ws2"], t["ws2s"])
    # the transposed weights in the tiled layout, like the forward's
    for key, which in (("w13", moe.MOE_PACK_W13T), ("w2", moe.MOE_PACK_W2T), ("ws13", moe.MOE_PACK_WS13T),
                       ("ws2", moe.MOE_PACK_WS2T)):
        if key in tt:
            tiled = torch.empty_like(tt[key])
            moe.moe_pack_weights(L.cfg, which, tt[key], tiled)
            tt[key] = tiled
    layer_t = moe.make_layer(tt["w13"], tt["w2"], t["wg"], ws13=tt.get("ws13"), ws2=tt.get("ws2"),
                             w13_scale=tt["w13s"], w2_scale=tt["w2s"], ws13_scale=tt.get("ws13s"),
                             ws2_scale=tt.get("ws2s"), weight_layout=moe.MOE_LAYOUT_TILED)
    idx = torch.empty((w.T, w.K), dtype=torch.int32, device=dev)
    gw = torch.empty((w.T, w.K), dtype=torch.float32, device=dev)
    counts = torch.empty(w.E, dtype=torch.int32, device=dev)
    offsets = torch.empty(w.E + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(w.T * w.K, dtype=torch.int32, device=dev)
    row_of = torch.empty((w.T, w.K), dtype=torch.int32, device=dev)
    moe.moe_route(L.cfg, L.layer, t["u"], t["bias"], idx, gw, ws)
    moe.moe_dispatch(L.cfg, idx, counts, offsets, perm, row_of, ws)
    g = torch.Generator(device=dev)
    g.manual_seed(w.seed)
    bf = dict(dtype=torch.bfloat16, device=dev)
    dy_r = torch.randn((w.T * w.K, w.d), generator=g, device=dev).to(torch.bfloat16)
    dy_s = torch.randn((w.T, w.d), generator=g, device=dev).to(torch.bfloat16) if w.Ks > 0 else None
    dx_r = torch.empty((w.T * w.K, w.d), **bf)
    dx_s = torch.empty((w.T, w.d), **bf) if w.Ks > 0 else None
    dw13 = torch.empty((w.E, 2 * w.f, w.d), **bf)
    dw2 = torch.empty((w.E, w.d, w.f), **bf)
    dws13 = torch.empty((2 * w.fs, w.d), **bf) if w.Ks > 0 else None
    dws2 = torch.empty((w.d, w.fs), **bf) if w.Ks > 0 else None
    bws = torch.empty(moe.moe_backward_workspace_size(L.cfg), dtype=torch.uint8, device=dev)
    run_in = lambda: moe.moe_expert_ffn_backward_input(L.cfg, L.layer, layer_t, t["u"], offsets, perm, dy_r, dy_s,
                                                       dx_r, dx_s, bws)
    run_all = lambda: moe.moe_expert_ffn_backward(L.cfg, L.layer, layer_t, t["u"], offsets, perm, dy_r, dy_s, dx_r,
                                                  dx_s, dw13, dw2, dws13, dws2, bws)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    ms_in, ms_all = timed(run_in), timed(run_all)
    rows = w.T * w.K + (w.T if w.Ks > 0 else 0)
    f_in, f_w = 10.0 * w.d * w.f * rows, 6.0 * w.d * w.f * rows
    out = {"ms_input": round(ms_in, 3), "ms_input_and_weight": round(ms_all, 3),
           "input_tflops": round(f_in / (ms_in * 1e-3) / 1e12, 1),
           "input_and_weight_tflops": round((f_in + f_w) / (ms_all * 1e-3) / 1e12, 1),
           "weight_grad_bytes_bf16": int(2 * 3 * w.d * w.f * (w.E + (1 if w.Ks > 0 else 0)))}
    del tt, layer_t, dy_r, dy_s, dx_r, dx_s, dw13, dw2, dws13, dws2, bws
    torch.cuda.empty_cache()
    return out


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor()


def cpu_baseline(w, repeats=3):
    """The float64 oracle on a bounded sample of the workload's layer, scaled to the whole batch.

    Timed on the host, median of `repeats` runs: the router (logits, gating, top-K) and dispatch on all T
    tokens, four routed experts on their own rows (the fewest rows, the most, and two between, by rank
    in load), and the combine on all T tokens. The oracle's expert costs a fixed part (turning E4M3
    weights into float64) plus a part per row; the least-squares line through the four timed experts gives
    every other routed expert's time and the shared block's (inner dim Ks*f, scaled by Ks). Weight
    generation and quantization are set-up, not timed."""
    import numpy as np
    from oracle import moe as omoe, quant as oquant
    from synth import configs, gen
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = 1
    u = configs.u_as_f32(w, configs.make_u(w))
    wg, bias, off = configs.make_router(w)

    def weights(e):
        w1, w3, w2 = configs.master_w1(w, e), configs.master_w3(w, e), configs.master_w2(w, e)
        if w.wdt == "fp8":
            return (*oquant.quantize_weight_128x128(np.vstack([w1, w3])), *oquant.quantize_weight_128x128(w2))
        if w.wdt == "bf16":
            st = lambda x: gen.bf16_bits_to_f32(gen.f32_to_bf16_bits(x))
            return st(w1), st(w3), st(w2)
        return w1, w3, w2

    def ffn(x, ex):
        if w.wdt == "fp8":
            return omoe.swiglu_ffn_fp8(x, *ex)[0]
        return omoe.swiglu_ffn(x, *ex)

    r = omoe.route(omoe.router_logits(u, wg, off), w.gate, w.K, bias, w.renorm)
    offsets, perm, row_of = omoe.dispatch(r["idx"], w.E)
    rows = np.diff(offsets)
    touched = np.flatnonzero(rows)
    by_load = touched[np.argsort(rows[touched], kind="stable")]
    sample = [int(by_load[round(q * (len(by_load) - 1))]) for q in (0.0, 1 / 3, 2 / 3, 1.0)]
    ex = {e: weights(e) for e in sample}
    y_rows = np.zeros((w.T * w.K, w.d))
    runs = []
    for _ in range(repeats):
        t = {}
        t0 = time.perf_counter()
        r = omoe.route(omoe.router_logits(u, wg, off), w.gate, w.K, bias, w.renorm)
        offsets, perm, row_of = omoe.dispatch(r["idx"], w.E)
        t["route"] = time.perf_counter() - t0
        for e in sample:
            t0 = time.perf_counter()
            y_rows[offsets[e]:offsets[e + 1]] = ffn(u[perm[offsets[e]:offsets[e + 1]]], ex[e])
            t[e] = time.perf_counter() - t0
        t0 = time.perf_counter()
        omoe.combine(u, np.zeros_like(u), y_rows, row_of, r["w"])
        t["combine"] = time.perf_counter() - t0
        per_row, fixed = np.polyfit([float(rows[e]) for e in sample], [t[e] for e in sample], 1)
        per_row, fixed = max(float(per_row), 0.0), max(float(fixed), 0.0)
        routed = fixed * len(touched) + per_row * float(rows.sum())
        shared = w.Ks * (fixed + per_row * w.T) if w.Ks > 0 else 0.0
        total = t["route"] + routed + shared + t["combine"]
        runs.append((total, t["route"] + sum(t[e] for e in sample) + t["combine"], fixed, per_row))
        note(f"cpu baseline run {len(runs)}/{repeats}: {runs[-1][1]:.1f} s timed, {total:.0f} s for the batch")
    runs.sort()
    total, timed, fixed, per_row = runs[len(runs) // 2]
    return {"value": round(w.T / total, 3), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": (f"{w.name} (T = {w.T}) through the float64 oracle, median of {repeats} runs: router and "
                       f"dispatch on all tokens, routed experts "
                       f"{', '.join(f'{e} ({int(rows[e])} rows)' for e in sample)} on their rows, combine on "
                       f"all tokens ({timed:.1f} s timed per run); the other {len(touched) - len(sample)} "
                       f"touched experts and the shared block from the least-squares line through those "
                       f"({fixed:.2f} s + {per_row * 1e3:.2f} ms per row), {total:.0f} s "
                       f"for the whole batch; weight generation/quantization untimed; host: {cpu_model()}")}


def library_record(moe):
    import hashlib
    return {"path": os.path.relpath(moe.LIB_PATH, ROOT),
            "sha256": hashlib.sha256(open(moe.LIB_PATH, "rb").read()).hexdigest()[:16]}


def time_graph_replays(step, stream, steps, warmup):
    """The same step captured once into a HIP graph (torch.cuda.CUDAGraph) and replayed `steps` times after
    `warmup` untimed replays: every kernel of the step runs on every replay, on the same resident inputs;
    what the graph removes is the host's per-launch cost, which bounds small layers (the 2B layer's ~20
    launches per step take longer on the host than its kernels on the device). Returns (ms per step,
    None), or (None, message) when capture is not possible, in which case the eager time stands."""
    import torch
    try:
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            step()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
    except Exception as e:                       # capture refused: report it and keep the eager timing
        torch.cuda.synchronize()
        return None, f"{type(e).__name__}: {e}"[:300]
    with torch.cuda.stream(stream):
        for _ in range(warmup):
            graph.replay()
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for _ in range(steps):
            graph.replay()
        t1.record(stream)
        torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    del graph
    return ms, None


def measure(moe, layers, w, steps, warmup, graph=True):
    """Build workload w on the device and time `steps` steps after `warmup` untimed ones. Returns the
    record (step time, per-stage times from HIP events on the launch stream, grouped-GEMM rates and
    rooflines) and the device layer, workspace and step outputs for further timings."""
    import ctypes
    import torch
    t_setup = time.time()
    L = layers.device_layer(w)
    setup_s = time.time() - t_setup
    ws = torch.empty(moe.moe_workspace_size(L.cfg), dtype=torch.uint8, device="cuda")
    h = torch.empty_like(L.t["u"])
    idx = torch.empty((w.T, w.K), dtype=torch.int32, device="cuda")
    counts = torch.empty(w.E, dtype=torch.int32, device="cuda")
    bias = L.t["bias"]
    bias_next = bias.clone() if w.gamma is not None else None
    stream = torch.cuda.current_stream()

    def step():
        # every step routes with the workload's bias and makes one update of it (into bias_next), so the
        # routing, and with it the work, is the same in every step
        moe.moe_forward(L.cfg, L.layer, L.t["u"], bias, h, idx, counts, ws)
        if w.gamma is not None:
            bias_next.copy_(bias)
            moe.moe_update_bias(L.cfg, counts, w.gamma, bias_next)

    # stage events: one set per timed step, created by recording them once
    marks = []
    for _ in range(steps):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(moe.MOE_NUM_MARKS)]
        for e in evs:
            e.record(stream)
        marks.append(evs)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_start.record(stream)
    for i in range(steps):
        arr = (ctypes.c_void_p * moe.MOE_NUM_MARKS)(*[e.cuda_event for e in marks[i]])
        moe.moe_set_timing_events(arr)
        step()
    moe.moe_set_timing_events(None)
    t_end.record(stream)
    torch.cuda.synchronize()
    eager_ms = t_start.elapsed_time(t_end) / steps
    graph_ms, graph_err = time_graph_replays(step, stream, steps, warmup) if graph else (None, None)
    ms = graph_ms if graph_ms is not None else eager_ms
    stage = {}
    for a, b in zip(moe.MARK_NAMES[:-1], moe.MARK_NAMES[1:]):
        ia, ib = moe.MARK_NAMES.index(a), moe.MARK_NAMES.index(b)
        stage[b.replace("_end", "")] = sum(m[ia].elapsed_time(m[ib]) for m in marks) / steps
    gwork, dwork, touched = kernel_work(w, counts.cpu().numpy())
    peak = PEAK[w.wdt]
    gemm_ms = stage["gateup"] + stage["down"]
    gemm_tflops = (gwork["flops"] + dwork["flops"]) / (gemm_ms * 1e-3) / 1e12
    rec = {
        "value": round(w.T / (ms * 1e-3), 1), "unit": "tokens/s", "steps": steps, "warmup": warmup,
        "ms_per_step": round(ms, 4), "launch": "hip_graph" if graph_ms is not None else "eager",
        "eager_ms_per_step": round(eager_ms, 4), "dtype": {"fp8": "fp8_e4m3", "bf16": "bf16", "f32": "f32"}[w.wdt],
        "config": {"workload": w.name, "T": w.T, "d_model": w.d, "routed": w.E, "shared": w.Ks, "top_k": w.K,
                   "inter_dim": w.f, "gate": w.gate, "renorm": w.renorm, "weights": w.wdt, "act": w.act,
                   "bias_update": w.gamma is not None},
        "roofline": dict(kernel=gateup_kernel_name(w), **roofline(gwork, stage["gateup"], peak)),
        "algorithmic_bytes": {"gateup": int(gwork["bytes"]), "down": int(dwork["bytes"])},
        "algorithmic_flops": {"gateup": gwork["flops"], "down": dwork["flops"]},
        "grouped_gemm_tflops": round(gemm_tflops, 1),
        "grouped_gemm_mfma_frac": round(gemm_tflops * 1e12 / peak, 4),
        "grouped_gemm_hbm_gbps": round((gwork["bytes"] + dwork["bytes"]) / (gemm_ms * 1e-3) / 1e9, 1),
        "grouped_gemm_hbm_frac": round((gwork["bytes"] + dwork["bytes"]) / (gemm_ms * 1e-3) / PEAK["hbm"], 4),
        "down_roofline": roofline(dwork, stage["down"], peak),
        "stages_ms": {k: round(v, 4) for k, v in stage.items()},
        "touched_experts": touched,
        "setup_s": round(setup_s, 1),
    }
    if graph_err is not None:
        rec["graph_error"] = graph_err
    prof = profiled_traffic(w.name)
    if prof is not None:
        rec["roofline"]["traffic"] = round(prof["gateup"]["traffic_bytes"])
        rec["down_roofline"]["traffic"] = round(prof["down"]["traffic_bytes"])
    note(f"{w.name}: {ms:.3f} ms per step over {steps} steps ({rec['launch']}; eager {eager_ms:.3f}), gate/up {stage['gateup']:.3f} ms, "
         f"down {stage['down']:.3f} ms (set-up {setup_s:.0f} s)")
    return rec, L, ws


SUB_WORKLOADS = ("dsmoe2b_bf16", "dsmoe16b_bf16", "v3_fp8_decode")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (this layer's multi-GPU "
              f"sharding is a design note, not a code path)", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU (HIP device)", file=sys.stderr)
        sys.exit(1)
    import fine_grained_mixture_gemm_amd as moe
    from fine_grained_mixture_gemm_amd import layers
    from synth import configs

    w = configs.WORKLOADS[args.workload]
    if args.tokens > 0:
        w = w.replace(name=f"{w.name}_t{args.tokens}", T=args.tokens)
    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    rec, L, ws = measure(moe, layers, w, args.steps, args.warmup, graph=not args.no_graph)
    out = {"metric": METRIC, "value": rec.pop("value"), "unit": rec.pop("unit"), "n_gpus": 1,
           "steps": rec.pop("steps"), "warmup": rec.pop("warmup"), "ms_per_step": rec.pop("ms_per_step"),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": rec.pop("dtype"),
           "data": "synthetic", "config": rec.pop("config")}
    out.update(rec)
    out["library"] = library_record(moe)
    out["balance_stats"] = time_balance_stats(moe, L, w, ws)
    if w.wdt == "fp8" and not args.no_backward:
        out["backward"] = time_backward(moe, L, w, ws)
        note(f"expert backward: input {out['backward']['ms_input']} ms, input + weight "
             f"{out['backward']['ms_input_and_weight']} ms")
    del L, ws
    torch.cuda.empty_cache()
    if not args.no_subconfigs and args.tokens == 0:
        # the other configurations the headline is quoted beside: the 2B and 16B bf16 layers (matrix-core
        # bound at large batch) and the 64-token V3 decode step (a weight stream), each its own timed run
        out["configs"] = {}
        for name in SUB_WORKLOADS:
            if name == w.name:
                continue
            sub, Ls, wss = measure(moe, layers, configs.WORKLOADS[name], args.sub_steps, args.sub_warmup,
                                   graph=not args.no_graph)
            out["configs"][name] = sub
            del Ls, wss
            torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
