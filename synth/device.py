"""Device fill of the synthetic inputs (same definitions as ``synth.gen``), for tensors too large to
generate on the host. Loads ``synth/libmoe_synth.so``; raises if it has not been built."""
from __future__ import annotations

import ctypes
import os

import torch

from . import gen

_LIB = None


def lib():
    global _LIB
    if _LIB is None:
        path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_synth.so")
        if not os.path.exists(path):
            raise ImportError(f"{path} is missing: run __graft_entry__.build() first")
        _LIB = ctypes.CDLL(path)
        _LIB.synth_fill_normal.argtypes = [ctypes.c_void_p, ctypes.c_longlong, ctypes.c_ulonglong, ctypes.c_longlong,
                                           ctypes.c_float, ctypes.c_int, ctypes.c_void_p]
        _LIB.synth_fill_normal.restype = ctypes.c_int
    return _LIB


def fill_normal(dst: torch.Tensor, seed: int, stream_id: int, sigma: float, start: int = 0) -> torch.Tensor:
    """Fill a contiguous float32 or bfloat16 CUDA tensor with elements start.. of (seed, stream_id)."""
    assert dst.is_cuda and dst.is_contiguous() and dst.dtype in (torch.float32, torch.bfloat16)
    rc = lib().synth_fill_normal(ctypes.c_void_p(dst.data_ptr()), dst.numel(), gen.tensor_key(seed, stream_id), start,
                                 float(gen.normal_scale(sigma)), 1 if dst.dtype == torch.bfloat16 else 0,
                                 ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    if rc != 0:
        raise RuntimeError(f"synth_fill_normal failed with HIP error {rc}")
    return dst
