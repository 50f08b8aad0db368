"""Bounds on how far E4M3 quantizer inputs computed on the GPU may be from the float64 oracle's, derived
from the arithmetic alone (test infrastructure for the E4M3 parity tests).

The kernels form g, v (and in the backward da) with block-scaled E4M3 GEMMs summed in fp32. Summed with
rounding to nearest, such a GEMM is off by at most
    (gamma_127 + gamma_nkb + 2 u) * sum_kb |s_x s_w| sum_k |q_x q_w|,   u = 2^-24, gamma_n = n u / (1 - n u)
(every 128-term partial sum, the scale product and the fused promotion into the running sum). These bounds
are carried through SwiGLU and its derivative to first order (times 1.1 for the higher orders, plus 1e-6
relative for the fp32 evaluation of SiLU with the hardware exponential and reciprocal). A quantized code
whose input window crosses a rounding midpoint may come out either way, and a window at a tile's largest
magnitude may move the tile's scale: flip() gives the largest change of the quantized value these allow.
"""
from __future__ import annotations

import numpy as np

from oracle import formats as oformats, quant as oquant

U32 = 2.0 ** -24


def gamma(n):
    return n * U32 / (1 - n * U32)


def gemm_bound(xq, xs, wq, ws):
    """Worst-case |fp32 result - exact| of the block-scaled E4M3 GEMM (rounding to nearest)."""
    mag = oquant.gemm_blockscaled(xq & np.uint8(0x7F), xs, wq & np.uint8(0x7F), ws)   # sum |s_x s_w q_x q_w|
    return (gamma(127) + gamma(xq.shape[1] // 128) + 2 * U32) * mag


def _silu_parts(g):
    sig = 1.0 / (1.0 + np.exp(-g))
    return sig, g * sig, sig * (1.0 + g * (1.0 - sig)), sig * (1.0 - sig) * (2.0 + g * (1.0 - 2.0 * sig))


def forward_windows(x, w13q, w13s):
    """(g, v, their bounds) of the gate/up GEMM and (a = SiLU(g) v, its bound) for the token rows x."""
    f = w13q.shape[0] // 2
    xq, xs = oquant.quantize_act_1x128(x)
    gv, dgv = oquant.gemm_blockscaled(xq, xs, w13q, w13s), gemm_bound(xq, xs, w13q, w13s)
    g, v, Dg, Dv = gv[:, :f], gv[:, f:], dgv[:, :f], dgv[:, f:]
    _, silu, d1, _ = _silu_parts(g)
    Da = 1.1 * (np.abs(d1 * v) * Dg + np.abs(silu) * Dv) + 1e-6 * np.abs(silu * v)
    return (g, v, Dg, Dv), (silu * v, Da)


def backward_windows(dy, x, w13q, w13s, w2q, w2s):
    """Bounds of a = SiLU(g) v [n, f] and of [dg | dv] [n, 2f] (dy quantized 1x128 along d, da = dy W2)."""
    (g, v, Dg, Dv), (_, Da) = forward_windows(x, w13q, w13s)
    dyq, dys = oquant.quantize_act_1x128(np.asarray(dy).astype(np.float32))
    w2t, w2st = np.ascontiguousarray(w2q.T), np.ascontiguousarray(w2s.T)
    da, Dda = oquant.gemm_blockscaled(dyq, dys, w2t, w2st), gemm_bound(dyq, dys, w2t, w2st)
    _, silu, d1, d2 = _silu_parts(g)
    Ddg = 1.1 * (np.abs(v * d1) * Dda + np.abs(da * d1) * Dv + np.abs(da * v * d2) * Dg) + 1e-6 * np.abs(da * v * d1)
    Ddv = 1.1 * (np.abs(silu) * Dda + np.abs(da * d1) * Dg) + 1e-6 * np.abs(da * silu)
    return Da, np.hstack([Ddg, Ddv])


def _round_e4m3(y):
    return oformats.e4m3_decode(oformats.e4m3_encode(np.clip(y, -448.0, 448.0)))


def _tile_max(a, axis_tiles):
    """Largest value of a over its 128-wide tiles along `axis_tiles` (0: rows, 1: columns), broadcast back."""
    a = np.asarray(a, dtype=np.float64)
    if axis_tiles == 1:
        n, c = a.shape
        return np.repeat(a.reshape(n, c // 128, 128).max(axis=2), 128, axis=1)
    n = a.shape[0]
    pad = -n % 128
    ap = np.vstack([a, np.zeros((pad, a.shape[1]))])
    return np.repeat(ap.reshape(-1, 128, a.shape[1]).max(axis=1), 128, axis=0)[:n]


def flip(v, win, axis_tiles, parts=False):
    """Largest change (value units) of the E4M3 tile-quantized v when every input may move by `win`: a code
    whose window crosses a rounding midpoint, and a tile scale moved as far as the tile's largest magnitude
    can move (it stays within [max(|v| - win), max(|v| + win)] over the tile). parts=True returns the two
    terms apart: (the code changes, the scale change)."""
    v = np.asarray(v, dtype=np.float64)
    win = np.asarray(win, dtype=np.float64)
    amax = _tile_max(np.abs(v), axis_tiles)
    up = _tile_max(np.abs(v) + win, axis_tiles) - amax
    down = amax - _tile_max(np.maximum(np.abs(v) - win, 0.0), axis_tiles)
    s = np.where(amax > 0, amax / 448.0, 1.0)
    rel = np.where(amax > 0, np.maximum(up, down) / np.maximum(amax, 1e-300), 0.0)   # relative scale change
    y = v / s
    w = win / s + np.abs(y) * rel
    code = np.abs(_round_e4m3(y + w) - _round_e4m3(y - w)) * s
    return (code, np.abs(v) * rel) if parts else code + np.abs(v) * rel
