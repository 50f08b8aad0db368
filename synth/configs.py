"""The five seeded synthetic DeepSeekMoE layer workloads and their host-side inputs.

Shapes follow the pages: the DeepSeekMoE 2B / 16B scale table and the V3 MoE configuration
(256 routed + 1 shared SwiGLU experts, top-8, expert inner dim 2048, hidden 7168).
Only the recipe lives here (shapes, seeds, distributions); every step of the method is elsewhere.

Tensor streams of one layer (see ``synth.gen``): u = 0, W_g = 1, bias = 2, Zipf permutation = 3,
shared W1 / W3 / W2 = 4 / 5 / 6, routed expert e W1 / W3 / W2 = 16 + 3e + 0 / 1 / 2.
Shared experts are generated as one concatenated expert of inner dim Ks * f.
Distributions: u ~ N(0, 1); W1, W3, W_g ~ N(0, 1/d); W2 ~ N(0, 1/f); bias ~ U(-0.1, 0.1);
Zipf(1.1) logit offsets -1.1 * ln(r_e) with r a seeded permutation of 1..E.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

from . import gen

STREAM_U, STREAM_WG, STREAM_BIAS, STREAM_ZIPF = 0, 1, 2, 3
STREAM_SH_W1, STREAM_SH_W3, STREAM_SH_W2 = 4, 5, 6
STREAM_U_TAIL = 7


def stream_routed(e: int, which: int) -> int:
    """which: 0 = W1 (gate), 1 = W3 (up), 2 = W2 (down)."""
    return 16 + 3 * e + which


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    d: int
    E: int          # routed experts
    Ks: int         # shared experts
    K: int          # routed experts per token
    f: int          # routed expert inner dim
    gate: str       # "softmax" or "sigmoid_bias"
    renorm: bool
    act: str        # dtype of u and h: "f32" or "bf16"
    wdt: str        # expert weight dtype: "f32", "bf16" or "fp8"
    seed: int
    zipf: Optional[float] = None
    bias_range: Optional[float] = None
    gamma: Optional[float] = None   # bias update speed, when the workload includes one
    n_groups: int = 0               # group-limited routing: experts in n_groups groups, topk_groups kept
    topk_groups: int = 0
    u_tail: bool = False            # heavy-tailed token rows (see tail_factors)

    @property
    def fs(self) -> int:
        return self.Ks * self.f

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    def expert_flops(self) -> float:
        """Algorithmic expert FLOPs: 6 d f per routed row plus 6 d f_s per token."""
        return 6.0 * self.d * self.f * self.T * self.K + 6.0 * self.d * self.fs * self.T


WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", T=128, d=256, E=16, Ks=1, K=2, f=64, gate="softmax",
                         renorm=False, act="f32", wdt="f32", seed=0),
    "dsmoe2b_bf16": Workload("dsmoe2b_bf16", T=2048, d=1024, E=63, Ks=1, K=7, f=1024,
                             gate="softmax", renorm=False, act="bf16", wdt="bf16", seed=1, zipf=1.1),
    "dsmoe16b_bf16": Workload("dsmoe16b_bf16", T=4096, d=2048, E=64, Ks=2, K=6, f=1408,
                              gate="softmax", renorm=False, act="bf16", wdt="bf16", seed=2, zipf=1.1),
    "v3_fp8": Workload("v3_fp8", T=8192, d=7168, E=256, Ks=1, K=8, f=2048, gate="sigmoid_bias",
                       renorm=True, act="bf16", wdt="fp8", seed=3, bias_range=0.1),
    "v3_fp8_decode": Workload("v3_fp8_decode", T=64, d=7168, E=256, Ks=1, K=8, f=2048,
                              gate="sigmoid_bias", renorm=True, act="bf16", wdt="fp8", seed=3,
                              bias_range=0.1, gamma=0.001),
}


def sigma_in(w: Workload) -> float:
    return 1.0 / math.sqrt(w.d)


def sigma_down(w: Workload) -> float:
    return 1.0 / math.sqrt(w.f)


def tail_factors(w: Workload) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Heavy tails for the token rows: word t of stream (seed, STREAM_U_TAIL) picks c = word % 16; c = 0
    scales row t by 32, c = 1 or 2 by 8, and c = 3 scales the single element (word >> 8) % d by 64.
    Returns (row factor [T] fp32, spiked rows, their spiked column)."""
    wd = gen.words(gen.tensor_key(w.seed, STREAM_U_TAIL), 0, w.T)
    c = (wd % np.uint64(16)).astype(np.int64)
    row = np.where(c == 0, 32.0, np.where((c == 1) | (c == 2), 8.0, 1.0)).astype(np.float32)
    spikes = np.flatnonzero(c == 3)
    cols = ((wd[spikes] >> np.uint64(8)) % np.uint64(w.d)).astype(np.int64)
    return row, spikes, cols


def make_u(w: Workload) -> np.ndarray:
    """u [T, d]: fp32 array for act f32, uint16 bf16 bit patterns for act bf16 (heavy-tailed rows when
    w.u_tail: the fp32 values scaled by tail_factors before the storage rounding)."""
    x = gen.normal_f32(w.seed, STREAM_U, (w.T, w.d), 1.0)
    if w.u_tail:
        row, spikes, cols = tail_factors(w)
        x = (x * row[:, None]).astype(np.float32)
        x[spikes, cols] = (x[spikes, cols] * np.float32(64.0)).astype(np.float32)
    return x if w.act == "f32" else gen.f32_to_bf16_bits(x)


def u_as_f32(w: Workload, u: np.ndarray) -> np.ndarray:
    return u if w.act == "f32" else gen.bf16_bits_to_f32(u)


def make_router(w: Workload):
    """(W_g [E, d] fp32, bias [E] fp32 or None, logit_offset [E] fp32 or None)."""
    wg = gen.normal_f32(w.seed, STREAM_WG, (w.E, w.d), sigma_in(w))
    bias = None
    if w.bias_range is not None:
        bias = gen.uniform_f32(w.seed, STREAM_BIAS, (w.E,), -w.bias_range, w.bias_range)
    off = None
    if w.zipf is not None:
        r = 1.0 + gen.random_permutation(w.seed, STREAM_ZIPF, w.E).astype(np.float64)
        off = (-w.zipf * np.log(r)).astype(np.float32)
    return wg, bias, off


def master_w1(w: Workload, e: int) -> np.ndarray:
    """fp32 master W1 (gate) of routed expert e, or of the shared group when e < 0: [f or fs, d]."""
    if e < 0:
        return gen.normal_f32(w.seed, STREAM_SH_W1, (w.fs, w.d), sigma_in(w))
    return gen.normal_f32(w.seed, stream_routed(e, 0), (w.f, w.d), sigma_in(w))


def master_w3(w: Workload, e: int) -> np.ndarray:
    if e < 0:
        return gen.normal_f32(w.seed, STREAM_SH_W3, (w.fs, w.d), sigma_in(w))
    return gen.normal_f32(w.seed, stream_routed(e, 1), (w.f, w.d), sigma_in(w))


def master_w2(w: Workload, e: int) -> np.ndarray:
    """fp32 master W2 (down) [d, f or fs]."""
    if e < 0:
        return gen.normal_f32(w.seed, STREAM_SH_W2, (w.d, w.fs), sigma_down(w))
    return gen.normal_f32(w.seed, stream_routed(e, 2), (w.d, w.f), sigma_down(w))


def weight_streams(w: Workload):
    """(stream, rows, cols, sigma) of every master weight matrix, shared group first."""
    out = [(STREAM_SH_W1, w.fs, w.d, sigma_in(w)), (STREAM_SH_W3, w.fs, w.d, sigma_in(w)),
           (STREAM_SH_W2, w.d, w.fs, sigma_down(w))]
    for e in range(w.E):
        out += [(stream_routed(e, 0), w.f, w.d, sigma_in(w)), (stream_routed(e, 1), w.f, w.d, sigma_in(w)),
                (stream_routed(e, 2), w.d, w.f, sigma_down(w))]
    return out
