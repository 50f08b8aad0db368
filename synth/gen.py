"""Seeded synthetic inputs for the DeepSeekMoE layer, shared by the oracle side and the HIP side.

This module holds no step of the MoE method: only random numbers and their storage format.
Both sides receive the same stored bits from here.

Generator (counter-based, so any slice of any tensor can be regenerated without the rest):

* ``mix64`` is the SplitMix64 output function (Steele, Lea & Flood, "Fast splittable
  pseudorandom number generators", OOPSLA 2014).
* A tensor is named by ``(seed, stream)``. Its key is ``mix64(mix64(seed + G) + G * (stream + 1))``,
  where G = 0x9E3779B97F4A7C15, and its i-th 64-bit word is ``mix64(key + G * (i + 1))``
  (all arithmetic modulo 2^64).
* "Normal" values use the four 16-bit fields c0..c3 of a word:
  S = sum_j (2 c_j - 65535), an even integer in [-262140, 262140] that is exact in fp32,
  mean 0 and variance 4 (65536^2 - 1) / 3 (Irwin-Hall with n = 4, bounded at about 3.46 sigma).
  The value is fl32(fl32(S) * scale) with scale = fl32(sigma / sqrt(4 (65536^2 - 1) / 3)).
* Uniform values on [lo, hi) use the top 24 bits: lo + (hi - lo) * (w >> 40 + 0.5) / 2^24, in fp64,
  then rounded to fp32.
* Storage in bf16 rounds the fp32 value to nearest, ties to even.

The device fill kernels in ``synth/csrc/synth_dev.hip`` implement the same definitions for the
expert weights, which are too large to generate on the host.
"""
from __future__ import annotations

import math

import numpy as np

GOLDEN = 0x9E3779B97F4A7C15
M1 = 0xBF58476D1CE4E5B9
M2 = 0x94D049BB133111EB
MASK64 = (1 << 64) - 1

# Standard deviation of S = sum of four (2c - 65535), c uniform on 0..65535.
IH4_STD = math.sqrt(4.0 * (65536.0 ** 2 - 1.0) / 3.0)

_U = np.uint64


def mix64_int(z: int) -> int:
    """SplitMix64 output function on a Python int (mod 2^64)."""
    z &= MASK64
    z = ((z ^ (z >> 30)) * M1) & MASK64
    z = ((z ^ (z >> 27)) * M2) & MASK64
    return z ^ (z >> 31)


def tensor_key(seed: int, stream: int) -> int:
    """64-bit key of the tensor (seed, stream)."""
    return mix64_int((mix64_int((seed + GOLDEN) & MASK64) + GOLDEN * (stream + 1)) & MASK64)


def _mix64_arr(z: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        z = z ^ (z >> _U(30))
        z = z * _U(M1)
        z = z ^ (z >> _U(27))
        z = z * _U(M2)
        z = z ^ (z >> _U(31))
    return z


def words(key: int, start: int, count: int) -> np.ndarray:
    """Words i = start .. start+count-1 of the stream with this key, as uint64."""
    idx = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = _U(key) + idx * _U(GOLDEN)
    return _mix64_arr(z)


def normal_scale(sigma: float) -> np.float32:
    """fp32 multiplier that maps the integer sum S to standard deviation sigma."""
    return np.float32(sigma / IH4_STD)


def normal_from_words(w: np.ndarray, sigma: float) -> np.ndarray:
    """fp32 values of the Irwin-Hall(4) approximate normal with standard deviation sigma."""
    s = np.zeros(w.shape, dtype=np.int64)
    for j in range(4):
        c = ((w >> _U(16 * j)) & _U(0xFFFF)).astype(np.int64)
        s += 2 * c - 65535
    return (s.astype(np.float32) * normal_scale(sigma)).astype(np.float32)


def normal_f32(seed: int, stream: int, shape, sigma: float, start: int = 0) -> np.ndarray:
    """fp32 tensor of the given shape: elements start .. start+prod(shape)-1 of (seed, stream)."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    key = tensor_key(seed, stream)
    chunk = 1 << 24
    for a in range(0, n, chunk):
        b = min(n, a + chunk)
        out[a:b] = normal_from_words(words(key, start + a, b - a), sigma)
    return out.reshape(shape)


def uniform_f32(seed: int, stream: int, shape, lo: float, hi: float) -> np.ndarray:
    n = int(np.prod(shape))
    w = words(tensor_key(seed, stream), 0, n)
    u = ((w >> _U(40)).astype(np.float64) + 0.5) / float(1 << 24)
    return (lo + (hi - lo) * u).astype(np.float32).reshape(shape)


def random_permutation(seed: int, stream: int, n: int) -> np.ndarray:
    """A permutation of 0..n-1: the stable argsort of the stream's first n words."""
    w = words(tensor_key(seed, stream), 0, n)
    return np.argsort(w, kind="stable").astype(np.int64)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); returns the uint16 bit patterns. No NaN inputs."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (b + _U(0x7FFF) + ((b >> _U(16)) & _U(1))) >> _U(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
