"""Pins of the oracle's fine-grained FP8 quantizers and block-scaled GEMM."""
import numpy as np
import pytest

from oracle import formats, quant


def _representable(rng, shape):
    codes = rng.integers(0, 0x7E, size=shape).astype(np.uint8) | (rng.integers(0, 2, size=shape) << 7).astype(np.uint8)
    return formats.e4m3_decode(codes)


def test_act_tiles_with_amax_448_are_exact():
    rng = np.random.default_rng(0)
    x = _representable(rng, (8, 512))
    x[:, ::128] = 448.0
    q, s = quant.quantize_act_1x128(x)
    assert np.all(s == 1.0)
    assert np.array_equal(formats.e4m3_decode(q), x)


def test_zero_tile_scale_one():
    x = np.zeros((2, 256))
    x[1, 128:] = 3.0
    q, s = quant.quantize_act_1x128(x)
    assert s[0, 0] == 1.0 and s[0, 1] == 1.0 and s[1, 0] == 1.0
    assert np.all(q[0] == 0) and np.all(q[1, :128] == 0)
    assert s[1, 1] == np.float32(3.0) / np.float32(448.0)
    assert np.all(formats.e4m3_decode(q[1, 128:]) == 448.0)


def test_act_scale_is_per_row_per_128_columns():
    rng = np.random.default_rng(1)
    x = rng.normal(size=(3, 384)) * np.array([1.0, 10.0, 0.01])[None, :].repeat(128, axis=1)
    _, s = quant.quantize_act_1x128(x)
    amax = np.abs(x.astype(np.float32)).reshape(3, 3, 128).max(axis=2)
    assert np.array_equal(s, (amax / np.float32(448)).astype(np.float32))


def test_act_relative_error_bound():
    # E4M3 has 3 mantissa bits: nearest rounding is within 2^-4 relative in the normal range
    # and within half a subnormal step (2^-10 * s) below it.
    rng = np.random.default_rng(2)
    x = rng.standard_t(3, size=(64, 1024))
    q, s = quant.quantize_act_1x128(x)
    xd = quant.dequant_act(q, s)
    x32 = x.astype(np.float32).astype(np.float64)
    srep = np.repeat(s.astype(np.float64), 128, axis=1)
    bound = np.maximum(np.abs(x32) * 2.0 ** -4, srep * 2.0 ** -10) * (1 + 1e-6)
    assert np.all(np.abs(xd - x32) <= bound)
    # the tile maximum maps to exactly 448 up to the two fp32 roundings of the scale
    g = np.abs(x32).reshape(64, 8, 128).max(axis=2)
    assert np.allclose(g / s, 448.0, rtol=2e-7)


def test_weight_blocks_are_128x128():
    w = np.ones((256, 384), dtype=np.float32)
    mult = np.array([[1.0, 2.0, 4.0], [8.0, 16.0, 32.0]])
    w = w * np.kron(mult, np.ones((128, 128)))
    w[5, 7] = 0.5
    q, s = quant.quantize_weight_128x128(w)
    assert s.shape == (2, 3)
    assert np.array_equal(s, (mult.astype(np.float32) / np.float32(448)).astype(np.float32))
    wd = quant.dequant_weight(q, s)
    assert np.allclose(wd, w, rtol=2.0 ** -4)
    assert formats.e4m3_decode(q[5:6, 7:8])[0, 0] == 224.0


def test_blockscaled_gemm_integer_exact():
    # integer-valued operands that E4M3 represents exactly, unit scales: the result is an int64 matmul.
    rng = np.random.default_rng(3)
    xi = rng.integers(-16, 17, size=(37, 512))
    wi = rng.integers(-16, 17, size=(256, 512))
    xq = formats.e4m3_encode(xi.astype(np.float64))
    wq = formats.e4m3_encode(wi.astype(np.float64))
    out = quant.gemm_blockscaled(xq, np.ones((37, 4), np.float32), wq, np.ones((2, 4), np.float32))
    assert np.array_equal(out, (xi @ wi.T).astype(np.float64))


def test_blockscaled_gemm_applies_each_scale_to_its_block():
    rng = np.random.default_rng(4)
    xi = rng.integers(-8, 9, size=(5, 256))
    wi = rng.integers(-8, 9, size=(256, 256))
    xs = np.array([[2.0, 0.5]] * 5, dtype=np.float32) * np.arange(1, 6, dtype=np.float32)[:, None]
    ws = np.array([[4.0, 0.25], [1.0, 8.0]], dtype=np.float32)
    out = quant.gemm_blockscaled(formats.e4m3_encode(xi.astype(float)), xs,
                                 formats.e4m3_encode(wi.astype(float)), ws)
    ref = np.zeros((5, 256))
    for kb in range(2):
        sl = slice(128 * kb, 128 * kb + 128)
        for nb in range(2):
            nsl = slice(128 * nb, 128 * nb + 128)
            ref[:, nsl] += xs[:, kb:kb + 1] * ws[nb, kb] * (xi[:, sl] @ wi[nsl, sl].T)
    assert np.array_equal(out, ref)


@pytest.mark.parametrize("m", [1, 130])
def test_blockscaled_gemm_equals_dequantized_product(m):
    rng = np.random.default_rng(5)
    x = rng.normal(size=(m, 384))
    w = rng.normal(size=(256, 384)) * 0.05
    xq, xs = quant.quantize_act_1x128(x)
    wq, ws = quant.quantize_weight_128x128(w)
    out = quant.gemm_blockscaled(xq, xs, wq, ws)
    ref = quant.dequant_act(xq, xs) @ quant.dequant_weight(wq, ws).T
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)
