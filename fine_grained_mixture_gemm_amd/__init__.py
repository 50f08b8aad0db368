"""DeepSeekMoE layer forward on one MI355X: thin ctypes binding of ``libmoe.so`` (see include/moe.h).

Every function has the name and argument order of its C entry point and only marshals arguments:
tensors become device pointers, the stream defaults to torch's current stream. All computation runs in
the HIP kernels of the library; there is no fallback. Importing raises if the library is not built.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "MOE_F32", "MOE_BF16", "MOE_FP8_E4M3", "MOE_GATE_SOFTMAX", "MOE_GATE_SIGMOID_BIAS", "MoeError",
    "moe_config", "moe_layer", "make_config", "make_layer", "moe_workspace_size", "moe_route", "moe_router_logits", "moe_dispatch",
    "moe_expert_ffn", "moe_combine", "moe_forward", "moe_update_bias", "moe_quantize_weights",
    "moe_quantize_act", "moe_last_error", "moe_set_timing_events", "MOE_NUM_MARKS", "MARK_NAMES", "LIB_PATH",
    "moe_balance_stats", "moe_backward_workspace_size", "moe_expert_ffn_backward_input", "moe_transpose_fp8_weights",
    "moe_expert_ffn_backward", "moe_forward_noalloc", "MOE_NOALLOC_SCRATCH_BYTES", "moe_route_margin",
    "moe_pack_weights", "MOE_LAYOUT_ROWS", "MOE_LAYOUT_TILED", "MOE_PACK_W13", "MOE_PACK_W2", "MOE_PACK_WS13",
    "MOE_PACK_WS2", "MOE_PACK_W13T", "MOE_PACK_W2T", "MOE_PACK_WS13T", "MOE_PACK_WS2T",
]

# always the in-tree build, next to this file
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe.so")
if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python fine_grained_mixture_gemm_amd/build.py`")
_lib = ctypes.CDLL(LIB_PATH)

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_F32, MOE_BF16, MOE_FP8_E4M3 = range(3)
MOE_GATE_SOFTMAX, MOE_GATE_SIGMOID_BIAS = range(2)
MOE_LAYOUT_ROWS, MOE_LAYOUT_TILED = range(2)
MOE_PACK_W13, MOE_PACK_W2, MOE_PACK_WS13, MOE_PACK_WS2, MOE_PACK_W13T, MOE_PACK_W2T, MOE_PACK_WS13T, MOE_PACK_WS2T = range(8)
MARK_NAMES = ("route_begin", "route_end", "dispatch_end", "quant_end", "gateup_end", "down_end", "combine_end")
MOE_NUM_MARKS = len(MARK_NAMES)
STATUS_NAMES = {0: "MOE_OK", 1: "MOE_ERR_INVALID_ARG", 2: "MOE_ERR_UNSUPPORTED", 3: "MOE_ERR_WORKSPACE",
                4: "MOE_ERR_HIP"}


class moe_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("T", "d_model", "n_routed", "n_shared", "top_k", "inter_dim", "gate",
                                                "renorm", "act_dtype", "w_dtype", "n_groups", "topk_groups")]


class moe_layer(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("w13", "w2", "w13_scale", "w2_scale", "ws13", "ws2", "ws13_scale",
                                                 "ws2_scale", "w_gate", "logit_offset")] + [("weight_layout", ctypes.c_int32)]


class MoeError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn}: {STATUS_NAMES.get(status, status)}: {moe_last_error()}")


_vp, _sz, _i32, _f32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_float
_CP, _LP = ctypes.POINTER(moe_config), ctypes.POINTER(moe_layer)
_SIGS = {
    "moe_workspace_size": [_CP, ctypes.POINTER(_sz)],
    "moe_route_margin": [_CP, ctypes.POINTER(_f32)],
    "moe_route": [_CP, _LP, _vp, _vp, _vp, _vp, _vp, _sz, _vp],
    "moe_router_logits": [_CP, _LP, _vp, _vp, _vp, _sz, _vp],
    "moe_dispatch": [_CP, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp],
    "moe_expert_ffn": [_CP, _LP, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp],
    "moe_combine": [_CP, _vp, _vp, _vp, _vp, _vp, _vp, _vp],
    "moe_forward": [_CP, _LP, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp],
    "moe_forward_noalloc": [_CP, _LP, _vp, _vp, _vp, _vp, _vp, _vp],
    "moe_update_bias": [_CP, _vp, _f32, _vp, _vp],
    "moe_balance_stats": [_CP, _vp, _vp, _i32, _f32, _f32, _vp, _vp, _vp, _vp, _sz, _vp],
    "moe_backward_workspace_size": [_CP, ctypes.POINTER(_sz)],
    "moe_expert_ffn_backward_input": [_CP, _LP, _LP, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp],
    "moe_expert_ffn_backward": [_CP, _LP, _LP] + [_vp] * 12 + [_sz, _vp],
    "moe_transpose_fp8_weights": [_vp, _vp, _i32, _i32, _i32, _vp, _vp, _vp],
    "moe_pack_weights": [_CP, _i32, _vp, _vp, _vp],
    "moe_quantize_weights": [_vp, _i32, _i32, _i32, _vp, _vp, _vp],
    "moe_quantize_act": [_vp, _i32, _i32, _i32, _vp, _vp, _vp],
    "moe_set_timing_events": [_vp, _i32],
}
for _name, _args in _SIGS.items():
    getattr(_lib, _name).argtypes = _args
    getattr(_lib, _name).restype = ctypes.c_int
_lib.moe_last_error.argtypes = []
_lib.moe_last_error.restype = ctypes.c_char_p


def moe_last_error() -> str:
    return _lib.moe_last_error().decode()


def _dev(t):
    """Device pointer of a CUDA tensor (None -> NULL)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("libmoe takes device tensors only")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _call(name, *args):
    st = getattr(_lib, name)(*args)
    if st != MOE_OK:
        raise MoeError(name, st)


def make_config(T, d_model, n_routed, n_shared, top_k, inter_dim, gate, renorm, act_dtype, w_dtype, n_groups=0,
                topk_groups=0) -> moe_config:
    return moe_config(T, d_model, n_routed, n_shared, top_k, inter_dim, gate, int(renorm), act_dtype, w_dtype,
                      n_groups, topk_groups)


def make_layer(w13, w2, w_gate, ws13=None, ws2=None, w13_scale=None, w2_scale=None, ws13_scale=None,
               ws2_scale=None, logit_offset=None, weight_layout=0) -> moe_layer:
    """Build the weight struct; the caller keeps the tensors alive while the struct is used."""
    return moe_layer(_dev(w13), _dev(w2), _dev(w13_scale), _dev(w2_scale), _dev(ws13), _dev(ws2), _dev(ws13_scale),
                     _dev(ws2_scale), _dev(w_gate), _dev(logit_offset), int(weight_layout))


def moe_pack_weights(cfg, which, src, dst, stream=None):
    _call("moe_pack_weights", ctypes.byref(cfg), int(which), _dev(src), _dev(dst), _stream(stream))


def moe_workspace_size(cfg) -> int:
    n = _sz(0)
    _call("moe_workspace_size", ctypes.byref(cfg), ctypes.byref(n))
    return n.value


def moe_route_margin(cfg) -> float:
    d = _f32(0)
    _call("moe_route_margin", ctypes.byref(cfg), ctypes.byref(d))
    return d.value


def moe_route(cfg, layer, u, bias, topk_idx, topk_w, ws, stream=None):
    _call("moe_route", ctypes.byref(cfg), ctypes.byref(layer), _dev(u), _dev(bias), _dev(topk_idx), _dev(topk_w),
          _dev(ws), ws.numel() * ws.element_size() if ws is not None else 0, _stream(stream))


def moe_router_logits(cfg, layer, u, z, ws, stream=None):
    _call("moe_router_logits", ctypes.byref(cfg), ctypes.byref(layer), _dev(u), _dev(z), _dev(ws),
          ws.numel() * ws.element_size() if ws is not None else 0, _stream(stream))


def moe_dispatch(cfg, topk_idx, counts, offsets, perm_src, row_of, ws, stream=None):
    _call("moe_dispatch", ctypes.byref(cfg), _dev(topk_idx), _dev(counts), _dev(offsets), _dev(perm_src),
          _dev(row_of), _dev(ws), ws.numel() * ws.element_size() if ws is not None else 0, _stream(stream))


def moe_expert_ffn(cfg, layer, u, offsets, perm_src, y_routed, y_shared, ws, stream=None):
    _call("moe_expert_ffn", ctypes.byref(cfg), ctypes.byref(layer), _dev(u), _dev(offsets), _dev(perm_src),
          _dev(y_routed), _dev(y_shared), _dev(ws), ws.numel() * ws.element_size() if ws is not None else 0,
          _stream(stream))


def moe_combine(cfg, u, y_routed, y_shared, row_of, topk_w, h, stream=None):
    _call("moe_combine", ctypes.byref(cfg), _dev(u), _dev(y_routed), _dev(y_shared), _dev(row_of), _dev(topk_w),
          _dev(h), _stream(stream))


def moe_forward(cfg, layer, u, bias, h, topk_idx, counts, ws, stream=None):
    _call("moe_forward", ctypes.byref(cfg), ctypes.byref(layer), _dev(u), _dev(bias), _dev(h), _dev(topk_idx),
          _dev(counts), _dev(ws), ws.numel() * ws.element_size() if ws is not None else 0, _stream(stream))


MOE_NOALLOC_SCRATCH_BYTES = 64 << 20


def moe_forward_noalloc(cfg, layer, u, bias, h, topk_idx, counts, stream=None):
    _call("moe_forward_noalloc", ctypes.byref(cfg), ctypes.byref(layer), _dev(u), _dev(bias), _dev(h), _dev(topk_idx),
          _dev(counts), _stream(stream))


def moe_update_bias(cfg, counts, gamma, bias, stream=None):
    _call("moe_update_bias", ctypes.byref(cfg), _dev(counts), float(gamma), _dev(bias), _stream(stream))


def moe_balance_stats(cfg, z, topk_idx, seq_len, alpha_expert, alpha_seq, f, P, loss, ws, stream=None):
    _call("moe_balance_stats", ctypes.byref(cfg), _dev(z), _dev(topk_idx), int(seq_len), float(alpha_expert),
          float(alpha_seq), _dev(f), _dev(P), _dev(loss), _dev(ws), ws.numel() * ws.element_size() if ws is not None else 0,
          _stream(stream))


def moe_backward_workspace_size(cfg) -> int:
    n = _sz(0)
    _call("moe_backward_workspace_size", ctypes.byref(cfg), ctypes.byref(n))
    return n.value


def moe_expert_ffn_backward_input(cfg, layer, layer_t, u, offsets, perm_src, dy_routed, dy_shared, dx_routed,
                                  dx_shared, ws, stream=None):
    _call("moe_expert_ffn_backward_input", ctypes.byref(cfg), ctypes.byref(layer), ctypes.byref(layer_t), _dev(u),
          _dev(offsets), _dev(perm_src), _dev(dy_routed), _dev(dy_shared), _dev(dx_routed), _dev(dx_shared), _dev(ws),
          ws.numel() * ws.element_size() if ws is not None else 0, _stream(stream))


def moe_expert_ffn_backward(cfg, layer, layer_t, u, offsets, perm_src, dy_routed, dy_shared, dx_routed, dx_shared,
                            dw13, dw2, dws13, dws2, ws, stream=None):
    _call("moe_expert_ffn_backward", ctypes.byref(cfg), ctypes.byref(layer), ctypes.byref(layer_t), _dev(u),
          _dev(offsets), _dev(perm_src), _dev(dy_routed), _dev(dy_shared), _dev(dx_routed), _dev(dx_shared),
          _dev(dw13), _dev(dw2), _dev(dws13), _dev(dws2), _dev(ws),
          ws.numel() * ws.element_size() if ws is not None else 0, _stream(stream))


def moe_transpose_fp8_weights(q, scales, qt, scales_t, stream=None):
    """q [batch, rows, cols] uint8 (or [rows, cols]), scales [batch, rows/128, cols/128] -> transposed copies."""
    batch = q.shape[0] if q.dim() == 3 else 1
    rows, cols = q.shape[-2], q.shape[-1]
    _call("moe_transpose_fp8_weights", _dev(q), _dev(scales), batch, rows, cols, _dev(qt), _dev(scales_t),
          _stream(stream))


def moe_quantize_weights(w, q, scales, stream=None):
    """w: float32 [batch, rows, cols] (or [rows, cols]) -> q uint8 same shape, scales [.., rows/128, cols/128]."""
    shape = w.shape if w.dim() == 3 else (1,) + tuple(w.shape)
    _call("moe_quantize_weights", _dev(w), shape[0], shape[1], shape[2], _dev(q), _dev(scales), _stream(stream))


def moe_quantize_act(x, x_dtype, q, scales, stream=None):
    rows, cols = x.shape
    _call("moe_quantize_act", _dev(x), x_dtype, rows, cols, _dev(q), _dev(scales), _stream(stream))


def moe_set_timing_events(events):
    """events: a ctypes array of MOE_NUM_MARKS hipEvent_t handles (host), or None to switch marks off."""
    if events is None:
        _call("moe_set_timing_events", None, 0)
    else:
        _call("moe_set_timing_events", ctypes.cast(events, ctypes.c_void_p), len(events))
