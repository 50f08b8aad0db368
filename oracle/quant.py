"""Fine-grained FP8 quantization, [TR] §3.6 ("quantization strategy") and [YJ] §4.2.2.

Activations get one scale per row per 128 consecutive columns (1x128 tiles); weights get one scale per
128x128 block. The pages fix the tile shapes and the E4M3 format but not how a scale is derived; the
reading taken here (the plainest one) maps each tile's largest magnitude onto the largest E4M3 value:

    amax = max |x| over the tile          (x taken in fp32)
    s    = fl32(amax / 448)               (s = 1 when amax = 0)
    inv  = fl32(448 / amax)               (inv = 1 when amax = 0)
    q    = E4M3(fl32(x * inv))            (nearest-even, saturating)

so that x is approximately s * q. Every operation above is a single correctly rounded fp32 operation,
which numpy's float32 arithmetic performs.
"""
from __future__ import annotations

import numpy as np

from .formats import e4m3_encode, e4m3_decode

TILE = 128
_448 = np.float32(448.0)


def _scales(amax32: np.ndarray):
    amax32 = amax32.astype(np.float32)
    zero = amax32 == 0
    safe = np.where(zero, np.float32(1.0), amax32).astype(np.float32)
    s = np.where(zero, np.float32(1.0), safe / _448).astype(np.float32)
    inv = np.where(zero, np.float32(1.0), _448 / safe).astype(np.float32)
    return s, inv


def quantize_act_1x128(x) -> tuple[np.ndarray, np.ndarray]:
    """x [rows, cols] (cols % 128 == 0) -> (E4M3 codes uint8 [rows, cols], scales fp32 [rows, cols/128])."""
    x32 = np.asarray(x).astype(np.float32)
    rows, cols = x32.shape
    assert cols % TILE == 0
    g = x32.reshape(rows, cols // TILE, TILE)
    amax = np.abs(g).max(axis=2)
    s, inv = _scales(amax)
    prod = (g * inv[:, :, None]).astype(np.float32)
    q = e4m3_encode(prod.astype(np.float64)).reshape(rows, cols)
    return q, s


def quantize_weight_128x128(w) -> tuple[np.ndarray, np.ndarray]:
    """w [rows, cols] (both % 128 == 0) -> (codes uint8 [rows, cols], scales fp32 [rows/128, cols/128])."""
    w32 = np.asarray(w).astype(np.float32)
    rows, cols = w32.shape
    assert rows % TILE == 0 and cols % TILE == 0
    g = w32.reshape(rows // TILE, TILE, cols // TILE, TILE)
    amax = np.abs(g).max(axis=(1, 3))
    s, inv = _scales(amax)
    prod = (g * inv[:, None, :, None]).astype(np.float32)
    q = e4m3_encode(prod.astype(np.float64)).reshape(rows, cols)
    return q, s


def dequant_act(q, s) -> np.ndarray:
    """float64 s * q per 1x128 tile."""
    v = e4m3_decode(q)
    rows, cols = v.shape
    return (v.reshape(rows, cols // TILE, TILE) * s.astype(np.float64)[:, :, None]).reshape(rows, cols)


def dequant_weight(q, s) -> np.ndarray:
    v = e4m3_decode(q)
    rows, cols = v.shape
    g = v.reshape(rows // TILE, TILE, cols // TILE, TILE) * s.astype(np.float64)[:, None, :, None]
    return g.reshape(rows, cols)


def gemm_blockscaled(xq, xs, wq, ws) -> np.ndarray:
    """out[m, n] = sum_kb xs[m, kb] * ws[n // 128, kb] * sum_{k in block kb} q_x[m, k] q_w[n, k].

    [TR] §3.6: FP8 products with FP32 accumulation promoted every Nc = 128 elements, each partial sum
    multiplied by its tile's activation scale and its block's weight scale. Evaluated in float64: the
    inner 128-term sums of E4M3 products are exact (all terms are multiples of 2^-18 below 2^25), so the
    only rounding is in the scale products and the sum over blocks.
    """
    xv = e4m3_decode(xq)
    wv = e4m3_decode(wq)
    m, k = xv.shape
    n = wv.shape[0]
    out = np.zeros((m, n), dtype=np.float64)
    for kb in range(k // TILE):
        sl = slice(kb * TILE, (kb + 1) * TILE)
        p = xv[:, sl] @ wv[:, sl].T
        sw = np.repeat(ws[:, kb].astype(np.float64), TILE)[None, :]
        out += (xs[:, kb].astype(np.float64)[:, None] * sw) * p
    return out


def quantize_act_along_rows(x) -> tuple[np.ndarray, np.ndarray]:
    """1x128 tiles that run down the columns: the operand of a GEMM whose contraction is over the rows
    (the weight-gradient GEMMs, where the contraction is over tokens).

    x [rows, cols] (cols % 128 == 0) is padded with zero rows to a multiple of 128 and every column is
    quantized in blocks of 128 consecutive rows with the rule above. Returns the codes transposed, so the
    contraction runs along the last axis: (codes uint8 [cols, rows_pad], scales fp32 [cols, rows_pad/128]).
    """
    x32 = np.asarray(x).astype(np.float32)
    rows, cols = x32.shape
    pad = -rows % TILE
    xp = np.vstack([x32, np.zeros((pad, cols), dtype=np.float32)])
    return quantize_act_1x128(np.ascontiguousarray(xp.T))


def gemm_rowscaled(aq, as_, bq, bs) -> np.ndarray:
    """out[m, n] = sum_kb as_[m, kb] * bs[n, kb] * sum_{k in block kb} q_a[m, k] q_b[n, k].

    Both operands carry one scale per row per 128 contraction elements (quantize_act_along_rows), so each
    128-term partial sum is promoted with the product of its two tile scales ([TR] §3.6 promotion every
    128 elements). float64; the inner sums are exact as in gemm_blockscaled.
    """
    av = e4m3_decode(aq)
    bv = e4m3_decode(bq)
    m, k = av.shape
    out = np.zeros((m, bv.shape[0]), dtype=np.float64)
    for kb in range(k // TILE):
        sl = slice(kb * TILE, (kb + 1) * TILE)
        out += (as_[:, kb].astype(np.float64)[:, None] * bs[:, kb].astype(np.float64)[None, :]) * (av[:, sl] @ bv[:, sl].T)
    return out
