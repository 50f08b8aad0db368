"""GPU quantizers and the device input fill, bit for bit against the oracle and the host generator."""
import numpy as np
import pytest
import torch

import fine_grained_mixture_gemm_amd as moe
from oracle import quant as oquant
from synth import device as sdev, gen
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


def _gpu_quant_act(x32: np.ndarray, as_bf16: bool):
    if as_bf16:
        bits = gen.f32_to_bf16_bits(x32)
        xt = H.bf16_tensor(bits).cuda()
        x32 = gen.bf16_bits_to_f32(bits)
    else:
        xt = torch.from_numpy(x32).cuda()
    q = torch.empty(x32.shape, dtype=torch.uint8, device="cuda")
    s = torch.empty((x32.shape[0], x32.shape[1] // 128), dtype=torch.float32, device="cuda")
    moe.moe_quantize_act(xt, moe.MOE_BF16 if as_bf16 else moe.MOE_F32, q, s)
    torch.cuda.synchronize()
    return x32, q.cpu().numpy(), s.cpu().numpy()


@pytest.mark.parametrize("as_bf16", [True, False])
def test_act_quantizer_bit_exact_random(as_bf16):
    rng = np.random.default_rng(0)
    x = (rng.standard_normal((257, 1024)) * np.exp(rng.uniform(-12, 12, (257, 1)))).astype(np.float32)
    x[3, :128] = 0.0
    x[4, 128:256] = 448.0
    x32, q, s = _gpu_quant_act(x, as_bf16)
    rq, rs = oquant.quantize_act_1x128(x32)
    assert np.array_equal(s, rs)
    assert np.array_equal(q, rq)


def test_act_quantizer_every_bf16_value():
    # every finite bf16 bit pattern, in rows of 128 whose maximum is pinned to 448 (unit scale) or left free
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    finite = ((bits >> 7) & 0xFF) != 0xFF
    vals = gen.bf16_bits_to_f32(bits[finite])
    vals = vals[np.abs(vals) <= 448.0]
    n = (len(vals) // 127) * 127
    rows = vals[:n].reshape(-1, 127)
    x = np.concatenate([rows, np.full((rows.shape[0], 1), 448.0, np.float32)], axis=1)
    x = np.concatenate([x, np.random.default_rng(1).permutation(x.reshape(-1)).reshape(x.shape)], axis=0)
    x32, q, s = _gpu_quant_act(x.astype(np.float32), True)
    rq, rs = oquant.quantize_act_1x128(x32)
    assert np.array_equal(s, rs) and np.array_equal(q, rq)


def test_weight_quantizer_bit_exact():
    rng = np.random.default_rng(2)
    w = (rng.standard_normal((3, 256, 384)) / 30).astype(np.float32)
    w[1, :128, :128] = 0.0
    # a block whose maximum is 448: its codes are the plain E4M3 rounding of a wide fp32 sample
    b = rng.integers(0, 2**32, size=(128, 128), dtype=np.uint64).astype(np.uint32).view(np.float32)
    b = np.where(np.isfinite(b) & (np.abs(b) <= 448.0), b, np.float32(1.5)).astype(np.float32)
    b[0, 0] = 448.0
    w[2, 128:, 256:] = b
    wt = torch.from_numpy(w).cuda()
    q = torch.empty(w.shape, dtype=torch.uint8, device="cuda")
    s = torch.empty((3, 2, 3), dtype=torch.float32, device="cuda")
    moe.moe_quantize_weights(wt, q, s)
    torch.cuda.synchronize()
    for i in range(3):
        rq, rs = oquant.quantize_weight_128x128(w[i])
        assert np.array_equal(s[i].cpu().numpy(), rs)
        assert np.array_equal(q[i].cpu().numpy(), rq)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_device_fill_matches_host_generator(dtype):
    n = 1 << 20
    t = torch.empty(n, dtype=dtype, device="cuda")
    sdev.fill_normal(t, 3, 77, 0.01, start=12345)
    torch.cuda.synchronize()
    ref = gen.normal_f32(3, 77, (n,), 0.01, start=12345)
    if dtype == torch.bfloat16:
        got = t.view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(got, gen.f32_to_bf16_bits(ref))
    else:
        assert np.array_equal(t.cpu().numpy(), ref)


def test_act_quantizer_every_fp32_value_in_range():
    """Every fp32 value of magnitude in [2^-11, 448] (20 binades, both signs; below 2^-11 all round to zero)
    through the device quantizer in rows of 127 values plus a 448, so the tile scale is exactly 1 and each
    code is the plain E4M3 rounding of the fp32 input: the conversion is pinned at full fp32 resolution,
    ties and subnormals included."""
    m = np.arange(1 << 23, dtype=np.uint32)
    for e in range(-11, 9):
        x = ((np.uint32(127 + e) << 23) | m).view(np.float32)
        x = x[np.abs(x) <= 448.0]
        n = (len(x) // 127) * 127
        # rows of 127; the last, partial row is filled up with values from the start of the binade
        tail = [np.concatenate([x[n:], x[:127 - (len(x) - n)]])[None]] if len(x) > n else []
        rows = np.concatenate([x[:n].reshape(-1, 127)] + tail, axis=0)
        rows[1::2] = -rows[1::2]
        tile = np.concatenate([rows, np.full((rows.shape[0], 1), 448.0, np.float32)], axis=1)
        x32, q, s = _gpu_quant_act(np.ascontiguousarray(tile), False)
        rq, rs = oquant.quantize_act_1x128(x32)
        assert np.all(s == 1.0) and np.array_equal(rs, s), f"binade 2^{e}: scales"
        bad = np.nonzero(q != rq)
        assert bad[0].size == 0, f"binade 2^{e}: {bad[0].size} codes differ, first at {x32[bad][:4]}"
