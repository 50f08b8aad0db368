"""Pins of the oracle's E4M3 format code against the format definition and torch's converter."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import formats

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3fn_codes.json")


def test_decode_golden_codes():
    g = json.load(open(GOLDEN))
    for code, val in g["codes"].items():
        v = formats.e4m3_decode(np.array([int(code, 16)], dtype=np.uint8))[0]
        assert v == val and np.signbit(v) == np.signbit(val), code
    for code in g["nan_codes"]:
        assert np.isnan(formats.e4m3_decode(np.array([int(code, 16)], dtype=np.uint8))[0])


def test_decode_matches_torch_for_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = formats.e4m3_decode(codes)
    same = (ours == ref) | (np.isnan(ours) & np.isnan(ref))
    assert same.all()


def test_encode_roundtrips_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(formats.e4m3_encode(formats.e4m3_decode(codes)), codes)


def _torch_e4m3(x32):
    return torch.from_numpy(x32).to(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_round_matches_torch_in_range():
    # torch rounds to nearest even and does not saturate; compare where no saturation is involved.
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 2**32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x) & (np.abs(x) < 440.0)]
    assert np.array_equal(formats.e4m3_round(x.astype(np.float64)), _torch_e4m3(x))


def test_ties_and_neighbours_of_every_midpoint():
    vals = np.unique(np.abs(formats.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))))
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)     # exact in fp32
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(0))
    for x in (mids, up, dn, -mids, -up, -dn):
        assert np.array_equal(formats.e4m3_round(x.astype(np.float64)), _torch_e4m3(x))
    # a tie goes to the even mantissa
    lo_codes = formats.e4m3_encode(formats.e4m3_round(mids.astype(np.float64)))
    assert np.all(lo_codes % 2 == 0)


def test_saturation():
    x = np.array([448.0, 450.0, 463.99, 464.0, 465.0, 1e6, 3.4e38, -500.0])
    assert np.array_equal(formats.e4m3_round(x), np.array([448.0] * 7 + [-448.0]))
    assert list(formats.e4m3_encode(x)) == [0x7E] * 7 + [0xFE]


def test_subnormals_and_zero():
    q = 2.0 ** -9
    x = np.array([0.0, -0.0, q * 0.5, q * 0.50001, q * 1.5, q * 2.5, 2 ** -6 - q / 2])
    r = formats.e4m3_round(x)
    assert list(r) == [0.0, -0.0, 0.0, q, 2 * q, 2 * q, 2 ** -6]
    assert np.signbit(r[1])


@pytest.mark.parametrize("seed", [1, 2])
def test_monotone(seed):
    x = np.sort(np.random.default_rng(seed).normal(0, 50, 100_000))
    assert np.all(np.diff(formats.e4m3_round(x)) >= 0)
