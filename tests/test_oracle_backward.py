"""Pins of the expert FFN input backward in the oracle (oracle.moe.swiglu_backward,
swiglu_ffn_backward_input, swiglu_ffn_backward_input_fp8): finite differences, torch autograd in float64
on the CPU (an independent library routine), and the E4M3 error bound ([TR] §3.6)."""
import numpy as np
import pytest
import torch

from oracle import moe, quant


def test_swiglu_backward_matches_central_differences():
    rng = np.random.default_rng(0)
    g, v, da = (rng.normal(0, 2, 500) for _ in range(3))
    dg, dv = moe.swiglu_backward(da, g, v)
    eps = 1e-6
    a = lambda gg, vv: moe.silu(gg) * vv
    assert np.allclose(dg, da * (a(g + eps, v) - a(g - eps, v)) / (2 * eps), rtol=1e-7, atol=1e-8)
    assert np.allclose(dv, da * (a(g, v + eps) - a(g, v - eps)) / (2 * eps), rtol=1e-7, atol=1e-8)


def _weights(rng, d, f):
    return rng.normal(0, d ** -0.5, (f, d)), rng.normal(0, d ** -0.5, (f, d)), rng.normal(0, f ** -0.5, (d, f))


def test_ffn_backward_input_matches_torch_autograd():
    rng = np.random.default_rng(1)
    d, f, n = 48, 40, 7
    w1, w3, w2 = _weights(rng, d, f)
    x, dy = rng.normal(0, 1, (n, d)), rng.normal(0, 1, (n, d))
    xt = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    T = lambda w: torch.tensor(w, dtype=torch.float64)
    y = (torch.nn.functional.silu(xt @ T(w1).T) * (xt @ T(w3).T)) @ T(w2).T
    y.backward(T(dy))
    assert np.allclose(moe.swiglu_ffn_backward_input(dy, x, w1, w3, w2), xt.grad.numpy(), rtol=1e-12, atol=1e-12)


def test_ffn_backward_input_directional_difference():
    rng = np.random.default_rng(2)
    d, f, n = 32, 24, 5
    w1, w3, w2 = _weights(rng, d, f)
    x, dy, dx_dir = (rng.normal(0, 1, (n, d)) for _ in range(3))
    eps = 1e-6
    lhs = np.sum(moe.swiglu_ffn_backward_input(dy, x, w1, w3, w2) * dx_dir)
    L = lambda xx: np.sum(dy * moe.swiglu_ffn(xx, w1, w3, w2))
    assert np.isclose(lhs, (L(x + eps * dx_dir) - L(x - eps * dx_dir)) / (2 * eps), rtol=1e-7, atol=1e-9)


def _fp8_expert(rng, d, f):
    w1, w3, w2 = _weights(rng, d, f)
    w13q, w13s = quant.quantize_weight_128x128(np.vstack([w1, w3]))
    w2q, w2s = quant.quantize_weight_128x128(w2)
    return w13q, w13s, w2q, w2s


def test_fp8_backward_of_zero_gradient_is_zero():
    rng = np.random.default_rng(3)
    d, f = 256, 256
    w = _fp8_expert(rng, d, f)
    x = rng.normal(0, 1, (6, d))
    assert np.array_equal(moe.swiglu_ffn_backward_input_fp8(np.zeros((6, d)), x, *w), np.zeros((6, d)))


def test_fp8_backward_within_the_e4m3_bound_of_the_float_backward():
    # The float backward on the same (dequantized) weights differs from the E4M3 path only by three
    # 1x128 quantizations (x, dy, [dg | dv]), each a rounding of relative size <= 2^-4 (3 mantissa
    # bits); their combined RMS is then at most sqrt(3) * 2^-4 = 0.108 of the result's RMS.
    rng = np.random.default_rng(4)
    d, f, n = 384, 256, 24
    w13q, w13s, w2q, w2s = _fp8_expert(rng, d, f)
    w13 = quant.dequant_weight(w13q, w13s)
    w2 = quant.dequant_weight(w2q, w2s)
    x, dy = rng.normal(0, 1, (n, d)), rng.normal(0, 1, (n, d))
    ref = moe.swiglu_ffn_backward_input(dy, x, w13[:f], w13[f:], w2)
    got = moe.swiglu_ffn_backward_input_fp8(dy, x, w13q, w13s, w2q, w2s)
    rel = np.sqrt(np.mean((got - ref) ** 2) / np.mean(ref ** 2))
    assert rel <= np.sqrt(3) * 2.0 ** -4, rel
    assert rel > 1e-3          # the quantization is really applied


def test_transposed_block_grid_is_the_transposed_matrix():
    # a weight used transposed keeps its codes and the transposed 128x128 scale grid: the block-scaled
    # product equals the product with the transposed dequantized matrix
    rng = np.random.default_rng(5)
    wq, ws = quant.quantize_weight_128x128(rng.normal(0, 1, (256, 384)))
    xq, xs = quant.quantize_act_1x128(rng.normal(0, 1, (9, 256)))
    got = quant.gemm_blockscaled(xq, xs, np.ascontiguousarray(wq.T), np.ascontiguousarray(ws.T))
    ref = quant.dequant_act(xq, xs) @ quant.dequant_weight(wq, ws)
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------------------ weight gradients
def test_ffn_backward_weight_matches_torch_autograd():
    rng = np.random.default_rng(6)
    d, f, n = 40, 24, 9
    w1, w3, w2 = _weights(rng, d, f)
    x, dy = rng.normal(0, 1, (n, d)), rng.normal(0, 1, (n, d))
    T = lambda w: torch.tensor(w, dtype=torch.float64, requires_grad=True)
    t1, t3, t2 = T(w1), T(w3), T(w2)
    xt = torch.tensor(x, dtype=torch.float64)
    y = (torch.nn.functional.silu(xt @ t1.T) * (xt @ t3.T)) @ t2.T
    y.backward(torch.tensor(dy, dtype=torch.float64))
    for got, ref in zip(moe.swiglu_ffn_backward_weight(dy, x, w1, w3, w2), (t1.grad, t3.grad, t2.grad)):
        assert got.shape == ref.shape
        assert np.allclose(got, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_quantize_along_rows_exact_tiles_and_padding():
    # columns built from E4M3 values whose 128-row blocks each reach 448: scale 1, codes exact; the
    # ragged last block is padded with zero rows (code 0), its scale from the valid rows only
    rng = np.random.default_rng(7)
    vals = quant.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))      # non-negative finite codes
    n, c = 200, 256
    x = rng.choice(vals, (n, c)) * rng.choice([-1.0, 1.0], (n, c))
    x[0, :] = 448.0
    x[128, :] = -448.0
    q, s = quant.quantize_act_along_rows(x)
    assert q.shape == (c, 256) and s.shape == (c, 2)
    assert np.array_equal(s, np.ones((c, 2), dtype=np.float32))
    assert np.array_equal(quant.e4m3_decode(q)[:, :n], x.T)
    assert not q[:, n:].any()


def test_quantize_along_rows_scales_per_column_block():
    x = np.zeros((130, 128))
    x[5, 3] = 7.0          # column 3, block 0
    x[129, 3] = -0.5       # column 3, block 1 (ragged, 2 valid rows)
    q, s = quant.quantize_act_along_rows(x)
    assert s[3, 0] == np.float32(7.0) / np.float32(448.0) and s[3, 1] == np.float32(0.5) / np.float32(448.0)
    assert s[0, 0] == 1.0 and s[0, 1] == 1.0                          # all-zero tiles get scale 1
    assert quant.e4m3_decode(q)[3, 5] == 448.0 and quant.e4m3_decode(q)[3, 129] == -448.0


def test_rowscaled_gemm_is_an_exact_integer_product_on_unit_scale_tiles():
    # integer E4M3 values with every tile reaching 448 (scale 1): the promoted product equals int64 matmul
    rng = np.random.default_rng(8)
    ints = np.array([0, 1, 2, 3, 4, 5, 6, 7, 8, 10, 12, 14, 16, 20, 24, 28, 32])
    m, n, k = 24, 40, 256
    a = rng.choice(ints, (m, k)) * rng.choice([-1, 1], (m, k))
    b = rng.choice(ints, (n, k)) * rng.choice([-1, 1], (n, k))
    a[:, ::128] = 448
    b[:, ::128] = 448
    aq, as_ = quant.quantize_act_1x128(a)
    bq, bs = quant.quantize_act_1x128(b)
    assert (as_ == 1).all() and (bs == 1).all()
    got = quant.gemm_rowscaled(aq, as_, bq, bs)
    assert np.array_equal(got, (a.astype(np.int64) @ b.astype(np.int64).T).astype(np.float64))


def test_rowscaled_gemm_promotes_each_block_with_both_scales():
    # one nonzero per 128-element block: the result is the sum of the scaled code products
    aq = np.zeros((1, 256), dtype=np.uint8)
    bq = np.zeros((1, 256), dtype=np.uint8)
    aq[0, 3], bq[0, 3] = quant.e4m3_encode(np.array([2.0]))[0], quant.e4m3_encode(np.array([3.0]))[0]
    aq[0, 200], bq[0, 200] = quant.e4m3_encode(np.array([-1.0]))[0], quant.e4m3_encode(np.array([5.0]))[0]
    as_ = np.array([[0.5, 4.0]], dtype=np.float32)
    bs = np.array([[0.25, 2.0]], dtype=np.float32)
    assert quant.gemm_rowscaled(aq, as_, bq, bs)[0, 0] == 0.5 * 0.25 * 6.0 + 4.0 * 2.0 * -5.0


def test_fp8_weight_gradient_of_zero_gradient_is_zero():
    rng = np.random.default_rng(9)
    w = _fp8_expert(rng, 256, 256)
    x = rng.normal(0, 1, (70, 256))
    dw13, dw2 = moe.swiglu_ffn_backward_weight_fp8(np.zeros((70, 256)), x, *w)
    assert not dw13.any() and not dw2.any()
    assert dw13.shape == (512, 256) and dw2.shape == (256, 256)


def test_fp8_weight_gradient_within_the_e4m3_bound_of_the_float_gradient():
    # Against the float gradient on the same (dequantized) weights: dW2 = dy^T a sees the roundings of dy
    # along the rows, x along d (through a), a along f and a along the rows (4); d[W1; W3] = [dg | dv]^T x
    # sees x along d (twice: in x and through g, v), x along the rows, dy along d, [dg | dv] along the
    # rows (5). Each is <= 2^-4 relative; their combined RMS is at most sqrt(count) * 2^-4.
    rng = np.random.default_rng(10)
    d, f, n = 384, 256, 300                  # three row blocks, the last one ragged
    w13q, w13s, w2q, w2s = _fp8_expert(rng, d, f)
    w13 = quant.dequant_weight(w13q, w13s)
    w2 = quant.dequant_weight(w2q, w2s)
    x, dy = rng.normal(0, 1, (n, d)), rng.normal(0, 1, (n, d))
    r1, r3, r2 = moe.swiglu_ffn_backward_weight(dy, x, w13[:f], w13[f:], w2)
    dw13, dw2 = moe.swiglu_ffn_backward_weight_fp8(dy, x, w13q, w13s, w2q, w2s)
    rel = lambda got, ref: np.sqrt(np.mean((got - ref) ** 2) / np.mean(ref ** 2))
    e2, e13 = rel(dw2, r2), rel(dw13, np.vstack([r1, r3]))
    assert e2 <= np.sqrt(4) * 2.0 ** -4, e2
    assert e13 <= np.sqrt(5) * 2.0 ** -4, e13
    assert e2 > 1e-3 and e13 > 1e-3
