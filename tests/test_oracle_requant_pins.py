"""Exact pins of the oracle's E4M3 requantization steps ("DeepSeek Technical Report: MoE Architecture"
§3.6, quantization strategy: 1x128 activation tiles, 128x128 weight blocks; low-precision storage: the
activations cached for the Linear backward are kept in FP8).

Each case is built by hand so that every quantity is exact, except the one value a step must round: a
value that E4M3 cannot hold (324, 280, 17) sits in a 1x128 tile whose largest magnitude fixes the scale.
The expected results below are derived in the comments from the scale rule (s = amax / 448, q = E4M3 of
x * 448 / amax, nearest-even) and nothing else, so that dropping or misplacing a requantization changes
them:
* the SwiGLU output a is requantized before it meets W2 (324 reaches W2 as 320);
* [dg | dv] is quantized before dx = [dg | dv] [W1; W3] (280 enters as 288);
* the weight gradients take a and x as the values of their forward E4M3 copies (a_1 = 320 enters as
  288 * s with s = fl32(512 / 448); x = 17 enters as 16).
SiLU(g) = g and SiLU'(g) = 1 hold exactly in float64 for g >= 40 (exp(-g) < 2^-57 vanishes beside 1).
"""
import numpy as np

from oracle import moe, quant

D = F = 128


def _w13(entries):
    """[W1; W3] of one expert (f = d = 128) with the given (row, col) -> value entries (rows >= 128 are
    W3). Rows 2 and 130 carry 448 in column 2, where x is 0, so that both 128x128 blocks have scale 1."""
    w = np.zeros((2 * F, D))
    w[2, 2] = w[F + 2, 2] = 448.0
    for (r, c), v in entries.items():
        w[r, c] = v
    q, s = quant.quantize_weight_128x128(w)
    assert np.all(s == 1.0) and np.array_equal(quant.dequant_weight(q, s), w)   # exact E4M3 values
    return q, s


def _w2(entries):
    """W2 [d, f] with the given entries, 448 at (1, 5) for a unit block scale (a_5 and dy_1 are 0)."""
    w = np.zeros((D, F))
    w[1, 5] = 448.0
    for (r, c), v in entries.items():
        w[r, c] = v
    q, s = quant.quantize_weight_128x128(w)
    assert np.all(s == 1.0) and np.array_equal(quant.dequant_weight(q, s), w)
    return q, s


def test_swiglu_output_is_requantized_before_w2():
    # x = [256, 448, 0, ...]: amax 448, scale 1, codes exact.
    x = np.zeros((1, D))
    x[0, 0], x[0, 1] = 256.0, 448.0
    # g_0 = 256 * 0.25 = 64, v_0 = 256 * 7/256 = 7     -> a_0 = SiLU(64) * 7 = 448
    # g_1 = 256 * 0.28125 = 72, v_1 = 256 * 1.125/64 = 4.5 -> a_1 = SiLU(72) * 4.5 = 324
    w13q, w13s = _w13({(0, 0): 0.25, (1, 0): 0.28125, (F + 0, 0): 7 / 256, (F + 1, 0): 1.125 / 64})
    # y_0 = a_1 (W2[0, 1] = 1), y_1 = a_0 (W2[1, 0] = 1)
    w2q, w2s = _w2({(0, 1): 1.0, (1, 0): 1.0})
    y, a = moe.swiglu_ffn_fp8(x, w13q, w13s, w2q, w2s)
    assert a[0, 0] == 448.0 and a[0, 1] == 324.0 and not a[0, 2:].any()
    # a's tile [448, 324, 0, ...]: scale 1; 324 lies between the E4M3 neighbours 320 and 352 -> 320
    expected = np.zeros(D)
    expected[0], expected[1] = 320.0, 448.0
    assert np.array_equal(y[0], expected), y[0, :4]


def _backward_case():
    # x = [256, 448, 0, 17, 0, ...]: scale 1; 17 (between 16 and 18, a tie) quantizes to 16 (even).
    x = np.zeros((1, D))
    x[0, 0], x[0, 1], x[0, 3] = 256.0, 448.0, 17.0
    # g = [64, 64, 0, ...] (W1 column 0 = 0.25), v = [8, 5, 0, ...] (W3 column 0 = 1/32, 1.25/64);
    # column 3 of W1 and W3 is 0, so the rounding of x_3 does not reach g and v.
    w13q, w13s = _w13({(0, 0): 0.25, (1, 0): 0.25, (F + 0, 0): 1 / 32, (F + 1, 0): 1.25 / 64})
    # dy = [448, 0, ...] (scale 1); da_j = sum_i dy_i W2[i, j] = 448 * W2[0, j] = [56, 56, 0, ...]
    w2q, w2s = _w2({(0, 0): 0.125, (0, 1): 0.125})
    dy = np.zeros((1, D))
    dy[0, 0] = 448.0
    return dy, x, w13q, w13s, w2q, w2s


def test_dg_dv_are_quantized_before_the_dx_gemm():
    dy, x, *w = _backward_case()
    # dg = da * v * SiLU'(g) = [56 * 8, 56 * 5] = [448, 280]; dv = da * SiLU(g) = [3584, 3584].
    # dg's tile [448, 280, 0, ...]: scale 1, 280 -> 288 (nearest of 256, 288).
    # dv's tile: amax 3584 = 8 * 448: scale 8, codes 448 -> exactly 3584 again.
    # dx_0 = 448 * 0.25 + 288 * 0.25 + 3584 / 32 + 3584 * 1.25 / 64 = 112 + 72 + 112 + 70 = 366
    # (unquantized dg would give 364); dx_2 = (dg_2 + dv_2) * 448 = 0, every other column 0.
    dx = moe.swiglu_ffn_backward_input_fp8(dy, x, *w)
    expected = np.zeros(D)
    expected[0] = 366.0
    assert np.array_equal(dx[0], expected), dx[0, :4]


def test_weight_gradients_use_the_forward_e4m3_copies_of_a_and_x():
    dy, x, *w = _backward_case()
    dw13, dw2 = moe.swiglu_ffn_backward_weight_fp8(dy, x, *w)
    # a = SiLU(g) * v = [512, 320, 0, ...]. Its forward 1x128 copy: amax 512, s = fl32(512 / 448),
    # inv = 448 / 512 = 0.875 exactly, codes E4M3([448, 280]) = [448, 288], so the copy holds
    # [448 s, 288 s] = 8/7 * [448, 288] = [512, 329.142857...] up to the fp32 rounding of s.
    s = float(np.float32(512.0) / np.float32(448.0))
    a_copy = np.array([448.0 * s, 288.0 * s])
    # With one token, the along-rows quantization of a column of value c gives scale fl32(c / 448) and
    # code 448: c back to about 1e-7 relative. dW2[i, j] = dy_i * a_copy_j: row 0 only.
    assert np.allclose(dw2[0, :2], 448.0 * a_copy, rtol=1e-6, atol=0), dw2[0, :2]
    assert abs(dw2[0, 1] - 448.0 * 320.0) > 1e3            # the uncached a would give 143360
    assert not dw2[1:].any() and not dw2[0, 2:].any()
    # x's forward copy is [256, 448, 0, 16, 0, ...]; dW1[j, k] = dg_j x_copy_k with dg = [448, 280]
    # (fp32, not requantized along 2f for this product), dW3[j, k] = dv_j x_copy_k with dv = [3584, 3584].
    x_copy = np.zeros(D)
    x_copy[0], x_copy[1], x_copy[3] = 256.0, 448.0, 16.0
    exp13 = np.zeros((2 * F, D))
    exp13[0], exp13[1] = 448.0 * x_copy, 280.0 * x_copy
    exp13[F], exp13[F + 1] = 3584.0 * x_copy, 3584.0 * x_copy
    assert np.allclose(dw13, exp13, rtol=1e-6, atol=0), (dw13[0, :4], dw13[1, :4])
