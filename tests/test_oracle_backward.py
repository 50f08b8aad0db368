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
