"""Host-parallel oracle evaluations for the full-size parity tests (test infrastructure).

At the V3 shape one expert's E4M3 weights take the oracle several seconds to rebuild from their synthetic
fp32 masters, so the tests that sample rows of every expert spread the experts over the host's cores:
each task rebuilds one expert's weights and evaluates the oracle's E4M3 SwiGLU expert on the token rows
given for it. Workers are fresh interpreters (spawn) running one BLAS thread each; they touch no GPU.
"""
from __future__ import annotations

import concurrent.futures as cf
import multiprocessing as mp
import os
import sys
import time

import numpy as np

_ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _init():
    if _ROOT not in sys.path:
        sys.path.insert(0, _ROOT)


def _expert_task(args):
    name, e, x = args
    _init()
    from oracle import moe as omoe, quant as oquant
    from synth import configs
    w = configs.WORKLOADS[name]
    w13q, w13s = oquant.quantize_weight_128x128(np.vstack([configs.master_w1(w, e), configs.master_w3(w, e)]))
    w2q, w2s = oquant.quantize_weight_128x128(configs.master_w2(w, e))
    return e, omoe.swiglu_ffn_fp8(x, w13q, w13s, w2q, w2s)[0]


def workers() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


def fp8_expert_outputs(workload: str, rows: dict[int, np.ndarray], label: str = "") -> dict[int, np.ndarray]:
    """{expert e (-1: the shared block): x [n, d] float64} -> {e: the oracle's E4M3 FFN_e(x) [n, d]}."""
    tasks = [(workload, e, np.ascontiguousarray(x)) for e, x in rows.items() if len(x)]
    out, t0, n = {}, time.time(), workers()
    saved = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS")}
    os.environ["OMP_NUM_THREADS"] = os.environ["OPENBLAS_NUM_THREADS"] = "1"
    try:
        # a worker that dies raises BrokenProcessPool here instead of being replaced
        with cf.ProcessPoolExecutor(n, mp_context=mp.get_context("spawn"), initializer=_init) as pool:
            futs = [pool.submit(_expert_task, t) for t in tasks]
            for i, fut in enumerate(cf.as_completed(futs)):
                e, y = fut.result()
                out[e] = y
                if (i + 1) % 32 == 0 or i + 1 == len(tasks):
                    print(f"{label} oracle experts {i + 1}/{len(tasks)} ({n} workers, {time.time() - t0:.0f} s)",
                          flush=True)
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    return out
