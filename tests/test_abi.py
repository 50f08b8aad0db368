"""The C ABI without a GPU: every declared entry point is exported, and argument validation returns the
documented status before anything is launched (these calls never reach the HIP runtime)."""
import ctypes
import os
import re
import subprocess

import pytest

import fine_grained_mixture_gemm_amd as moe

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "moe.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:moe_status|const char\*)\s+(moe_\w+)\s*\(", text, flags=re.M)))


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert "moe_forward" in names and len(names) >= 10
    out = subprocess.run(["nm", "-D", "--defined-only", moe.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (\w+)$", out, flags=re.M))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    lib = ctypes.CDLL(moe.LIB_PATH)
    for n in names:
        getattr(lib, n)


def _cfg(**kw):
    base = dict(T=64, d_model=256, n_routed=16, n_shared=1, top_k=4, inter_dim=128, gate=moe.MOE_GATE_SIGMOID_BIAS,
                renorm=1, act_dtype=moe.MOE_BF16, w_dtype=moe.MOE_FP8_E4M3)
    base.update(kw)
    return moe.make_config(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(top_k=17, n_routed=32), moe.MOE_ERR_UNSUPPORTED),
    (dict(top_k=20), moe.MOE_ERR_INVALID_ARG),
    (dict(n_routed=300, top_k=4), moe.MOE_ERR_UNSUPPORTED),
    (dict(T=-1), moe.MOE_ERR_INVALID_ARG),
    (dict(d_model=0), moe.MOE_ERR_INVALID_ARG),
    (dict(gate=7), moe.MOE_ERR_INVALID_ARG),
    (dict(renorm=2), moe.MOE_ERR_INVALID_ARG),
    (dict(act_dtype=moe.MOE_FP8_E4M3), moe.MOE_ERR_INVALID_ARG),
    (dict(act_dtype=moe.MOE_F32, w_dtype=moe.MOE_BF16), moe.MOE_ERR_UNSUPPORTED),
    (dict(d_model=384), moe.MOE_ERR_UNSUPPORTED),          # bf16 / fp8 experts need d % 256 == 0
    (dict(inter_dim=100), moe.MOE_ERR_UNSUPPORTED),
    (dict(d_model=8448), moe.MOE_ERR_UNSUPPORTED),         # fp64 recheck holds d <= 8192
    (dict(n_groups=3, topk_groups=1), moe.MOE_ERR_INVALID_ARG),    # 16 experts do not split into 3 groups
    (dict(n_groups=4, topk_groups=0), moe.MOE_ERR_INVALID_ARG),
    (dict(n_groups=4, topk_groups=5), moe.MOE_ERR_INVALID_ARG),
    (dict(n_groups=0, topk_groups=2), moe.MOE_ERR_INVALID_ARG),
    (dict(n_groups=16, topk_groups=2), moe.MOE_ERR_INVALID_ARG),   # K = 4 > 2 groups x 1 expert
    (dict(n_routed=64, n_groups=32, topk_groups=8), moe.MOE_ERR_UNSUPPORTED),
])
def test_invalid_configs(kw, status):
    with pytest.raises(moe.MoeError) as e:
        moe.moe_workspace_size(_cfg(**kw))
    assert e.value.status == status
    assert moe.moe_last_error()


def test_workspace_size_and_valid_configs():
    assert moe.moe_workspace_size(_cfg()) > 0
    assert moe.moe_workspace_size(_cfg(n_groups=4, topk_groups=2)) > 0
    assert moe.moe_workspace_size(_cfg(T=0)) > 0
    assert moe.moe_workspace_size(_cfg(act_dtype=moe.MOE_F32, w_dtype=moe.MOE_F32, d_model=100, inter_dim=30)) > 0
    big = moe.moe_workspace_size(_cfg(T=8192, d_model=7168, n_routed=256, top_k=8, inter_dim=2048))
    assert 1e9 < big < 2e9


def test_null_pointers_and_workspace_errors():
    cfg = _cfg()
    layer = moe.moe_layer()
    lib = ctypes.CDLL(moe.LIB_PATH)
    lib.moe_route.argtypes = [ctypes.POINTER(moe.moe_config), ctypes.POINTER(moe.moe_layer)] + [ctypes.c_void_p] * 5 + [ctypes.c_size_t, ctypes.c_void_p]
    # layer without w_gate
    assert lib.moe_route(ctypes.byref(cfg), ctypes.byref(layer), 1, None, 1, 1, 1, 1 << 30, None) == moe.MOE_ERR_INVALID_ARG
    layer.w_gate = 16
    # u missing
    assert lib.moe_route(ctypes.byref(cfg), ctypes.byref(layer), None, None, 16, 16, 16, 1 << 30, None) == moe.MOE_ERR_INVALID_ARG
    # workspace too small or missing
    assert lib.moe_route(ctypes.byref(cfg), ctypes.byref(layer), 16, None, 16, 16, 16, 1024, None) == moe.MOE_ERR_WORKSPACE
    assert lib.moe_route(ctypes.byref(cfg), ctypes.byref(layer), 16, None, 16, 16, None, 1 << 30, None) == moe.MOE_ERR_WORKSPACE
    # expert weights: fp8 needs scales
    lib.moe_expert_ffn.argtypes = [ctypes.POINTER(moe.moe_config), ctypes.POINTER(moe.moe_layer)] + [ctypes.c_void_p] * 6 + [ctypes.c_size_t, ctypes.c_void_p]
    layer.w13, layer.w2 = 16, 16
    assert lib.moe_expert_ffn(ctypes.byref(cfg), ctypes.byref(layer), 16, 16, 16, 16, 16, 16, 1 << 30, None) == moe.MOE_ERR_INVALID_ARG
    assert "scale" in moe.moe_last_error()
    # quantizers
    lib.moe_quantize_weights.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    assert lib.moe_quantize_weights(16, 1, 100, 128, 16, 16, None) == moe.MOE_ERR_UNSUPPORTED
    assert lib.moe_quantize_weights(None, 1, 128, 128, 16, 16, None) == moe.MOE_ERR_INVALID_ARG
    lib.moe_quantize_act.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    assert lib.moe_quantize_act(16, moe.MOE_FP8_E4M3, 4, 128, 16, 16, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_quantize_act(16, moe.MOE_BF16, 4, 100, 16, 16, None) == moe.MOE_ERR_UNSUPPORTED
    # timing marks need the full set of events
    lib.moe_set_timing_events.argtypes = [ctypes.c_void_p, ctypes.c_int32]
    assert lib.moe_set_timing_events(16, 3) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_set_timing_events(None, 0) == moe.MOE_OK


def test_balance_stats_argument_errors():
    # every check runs before any launch: non-null dummy pointers are never dereferenced
    cfg = _cfg(T=256)
    lib = ctypes.CDLL(moe.LIB_PATH)
    lib.moe_balance_stats.argtypes = ([ctypes.POINTER(moe.moe_config), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                       ctypes.c_float, ctypes.c_float] + [ctypes.c_void_p] * 4 + [ctypes.c_size_t, ctypes.c_void_p])
    call = lambda seq, z=16, ws=16, nbytes=1 << 31: lib.moe_balance_stats(ctypes.byref(cfg), z, 16, seq, 0.003, 1e-4, 16, 16, 16, ws, nbytes, None)
    assert call(0) == moe.MOE_ERR_INVALID_ARG
    assert call(100) == moe.MOE_ERR_INVALID_ARG          # does not divide T
    assert call(32) == moe.MOE_ERR_UNSUPPORTED           # divides T, not a multiple of 64
    assert call(64, z=None) == moe.MOE_ERR_INVALID_ARG
    assert call(64, nbytes=1024) == moe.MOE_ERR_WORKSPACE
    assert call(256, ws=None) == moe.MOE_ERR_WORKSPACE


def test_binding_rejects_host_tensors():
    import torch
    with pytest.raises(ValueError):
        moe.moe_quantize_act(torch.zeros(4, 128), moe.MOE_F32, torch.zeros(4, 128, dtype=torch.uint8), torch.zeros(4, 1))


def test_backward_argument_errors():
    # every check runs before any launch: non-null dummy pointers are never dereferenced
    with pytest.raises(moe.MoeError) as e:
        moe.moe_backward_workspace_size(_cfg(act_dtype=moe.MOE_BF16, w_dtype=moe.MOE_BF16))
    assert e.value.status == moe.MOE_ERR_UNSUPPORTED
    with pytest.raises(moe.MoeError) as e:
        moe.moe_backward_workspace_size(_cfg(n_shared=2))
    assert e.value.status == moe.MOE_ERR_UNSUPPORTED
    with pytest.raises(moe.MoeError) as e:
        moe.moe_backward_workspace_size(_cfg(inter_dim=128))      # da tiles are 256 channels wide
    assert e.value.status == moe.MOE_ERR_UNSUPPORTED
    cfg = _cfg(inter_dim=256)
    need = moe.moe_backward_workspace_size(cfg)
    assert need > 64 * 4 * 2 * 256 * 4          # at least the fp32 [g | v] of the routed rows
    lib = ctypes.CDLL(moe.LIB_PATH)
    P = ctypes.POINTER
    lib.moe_expert_ffn_backward_input.argtypes = ([P(moe.moe_config), P(moe.moe_layer), P(moe.moe_layer)] +
                                                  [ctypes.c_void_p] * 8 + [ctypes.c_size_t, ctypes.c_void_p])
    full = moe.moe_layer(16, 16, 16, 16, 16, 16, 16, 16, 16, None)
    call = lambda lt=full, dys=16, ws=16, nbytes=need: lib.moe_expert_ffn_backward_input(
        ctypes.byref(cfg), ctypes.byref(full), ctypes.byref(lt), 16, 16, 16, 16, dys, 16, 16, ws, nbytes, None)
    assert call(lt=moe.moe_layer()) == moe.MOE_ERR_INVALID_ARG           # transposed weights missing
    assert call(dys=None) == moe.MOE_ERR_INVALID_ARG                      # shared gradient missing
    assert call(nbytes=need - 1) == moe.MOE_ERR_WORKSPACE
    assert call(ws=None) == moe.MOE_ERR_WORKSPACE
    lib.moe_transpose_fp8_weights.argtypes = [ctypes.c_void_p, ctypes.c_void_p] + [ctypes.c_int32] * 3 + [ctypes.c_void_p] * 3
    assert lib.moe_transpose_fp8_weights(16, 16, 1, 192, 128, 16, 16, None) == moe.MOE_ERR_UNSUPPORTED
    assert lib.moe_transpose_fp8_weights(16, 16, -1, 128, 128, 16, 16, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_transpose_fp8_weights(None, 16, 1, 128, 128, 16, 16, None) == moe.MOE_ERR_INVALID_ARG


def test_full_backward_argument_errors():
    cfg = _cfg(inter_dim=256)
    need = moe.moe_backward_workspace_size(cfg)
    lib = ctypes.CDLL(moe.LIB_PATH)
    P = ctypes.POINTER
    lib.moe_expert_ffn_backward.argtypes = ([P(moe.moe_config), P(moe.moe_layer), P(moe.moe_layer)] +
                                            [ctypes.c_void_p] * 12 + [ctypes.c_size_t, ctypes.c_void_p])
    full = moe.moe_layer(16, 16, 16, 16, 16, 16, 16, 16, 16, None)
    def call(dx=16, dxs=16, dw13=16, dw2=16, dws13=16, dws2=16, nbytes=need):
        return lib.moe_expert_ffn_backward(ctypes.byref(cfg), ctypes.byref(full), ctypes.byref(full), 16, 16, 16, 16, 16,
                                           dx, dxs, dw13, dw2, dws13, dws2, 16, nbytes, None)
    assert call(dx=None, dw13=None) == moe.MOE_ERR_INVALID_ARG        # nothing asked for
    assert call(dw2=None) == moe.MOE_ERR_INVALID_ARG
    assert call(dws2=None) == moe.MOE_ERR_INVALID_ARG                 # shared block needs its gradients
    assert call(dx=None, dws13=None) == moe.MOE_ERR_INVALID_ARG
    assert call(dxs=None, dw13=None) == moe.MOE_ERR_INVALID_ARG       # shared dx missing
    assert call(nbytes=need - 1) == moe.MOE_ERR_WORKSPACE
    assert "dw" in moe.moe_last_error() or "workspace" in moe.moe_last_error()


def test_noalloc_forward_rejects_oversized_configs_before_any_launch():
    # the V3-shaped layer at 8192 tokens needs about 1.3 GB of scratch, far above the static array
    cfg = _cfg(T=8192, d_model=7168, n_routed=256, top_k=8, inter_dim=2048)
    assert moe.moe_workspace_size(cfg) > moe.MOE_NOALLOC_SCRATCH_BYTES
    lib = ctypes.CDLL(moe.LIB_PATH)
    lay = moe.moe_layer()
    st = lib.moe_forward_noalloc(ctypes.byref(cfg), ctypes.byref(lay), None, None, None, None, None, None)
    assert st == moe.MOE_ERR_WORKSPACE
    assert "scratch" in moe.moe_last_error()


def test_weight_layout_argument_errors():
    lib = ctypes.CDLL(moe.LIB_PATH)
    lib.moe_pack_weights.argtypes = [ctypes.POINTER(moe.moe_config), ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_void_p]
    cfg = _cfg()
    f32 = _cfg(act_dtype=moe.MOE_F32, w_dtype=moe.MOE_F32)
    assert lib.moe_pack_weights(ctypes.byref(f32), moe.MOE_PACK_W13, 16, 32, None) == moe.MOE_ERR_UNSUPPORTED
    assert lib.moe_pack_weights(ctypes.byref(cfg), 8, 16, 32, None) == moe.MOE_ERR_INVALID_ARG
    # W2^T has f rows: the tiled layout needs a multiple of 256 (inter_dim 128 here)
    assert lib.moe_pack_weights(ctypes.byref(cfg), moe.MOE_PACK_W2T, 16, 32, None) == moe.MOE_ERR_UNSUPPORTED
    assert lib.moe_pack_weights(ctypes.byref(cfg), moe.MOE_PACK_W2, 16, 16, None) == moe.MOE_ERR_INVALID_ARG  # in place
    assert lib.moe_pack_weights(ctypes.byref(cfg), moe.MOE_PACK_W2, None, 16, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_pack_weights(ctypes.byref(_cfg(n_shared=0)), moe.MOE_PACK_WS13, None, None, None) == moe.MOE_OK
    # a layer in an unknown layout, or fp32 weights in the tiled one, is refused before any launch
    lib.moe_expert_ffn.argtypes = [ctypes.POINTER(moe.moe_config), ctypes.POINTER(moe.moe_layer)] + [ctypes.c_void_p] * 6 + [ctypes.c_size_t, ctypes.c_void_p]
    bad = moe.moe_layer(16, 16, 16, 16, 16, 16, 16, 16, 16, None, 2)
    assert lib.moe_expert_ffn(ctypes.byref(cfg), ctypes.byref(bad), 16, 16, 16, 16, 16, 16, 1 << 30, None) == moe.MOE_ERR_INVALID_ARG
    tiled32 = moe.moe_layer(16, 16, None, None, 16, 16, None, None, 16, None, moe.MOE_LAYOUT_TILED)
    assert lib.moe_expert_ffn(ctypes.byref(f32), ctypes.byref(tiled32), 16, 16, 16, 16, 16, 16, 1 << 30, None) == moe.MOE_ERR_UNSUPPORTED


def test_misaligned_buffers_are_rejected():
    # the kernels move activations, weights and expert outputs in 16-byte pieces: an address off a 16-byte
    # boundary fails validation (the dummy addresses are never dereferenced)
    lib = ctypes.CDLL(moe.LIB_PATH)
    P = ctypes.POINTER
    cfg = _cfg()
    layer = moe.moe_layer()
    layer.w_gate = 16
    lib.moe_route.argtypes = [P(moe.moe_config), P(moe.moe_layer)] + [ctypes.c_void_p] * 5 + [ctypes.c_size_t, ctypes.c_void_p]
    assert lib.moe_route(ctypes.byref(cfg), ctypes.byref(layer), 24, None, 16, 16, 16, 1 << 30, None) == moe.MOE_ERR_INVALID_ARG
    assert "aligned" in moe.moe_last_error() and "u" in moe.moe_last_error()
    lib.moe_expert_ffn.argtypes = [P(moe.moe_config), P(moe.moe_layer)] + [ctypes.c_void_p] * 6 + [ctypes.c_size_t, ctypes.c_void_p]
    layer.w13, layer.w2, layer.w13_scale, layer.w2_scale = 16, 16, 16, 16
    layer.ws13, layer.ws2, layer.ws13_scale, layer.ws2_scale = 16, 16, 16, 16
    ffn = lambda u=16, yr=16, ys=16: lib.moe_expert_ffn(ctypes.byref(cfg), ctypes.byref(layer), u, 16, 16, yr, ys, 16,
                                                        1 << 30, None)
    assert ffn(yr=40) == moe.MOE_ERR_INVALID_ARG and "y_routed" in moe.moe_last_error()
    assert ffn(ys=8) == moe.MOE_ERR_INVALID_ARG and "y_shared" in moe.moe_last_error()
    layer.w2 = 48 + 4
    assert ffn() == moe.MOE_ERR_INVALID_ARG and "layer->w2" in moe.moe_last_error()
    layer.w2 = 16
    lib.moe_quantize_act.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    assert lib.moe_quantize_act(18, moe.MOE_BF16, 4, 128, 16, 16, None) == moe.MOE_ERR_INVALID_ARG
    lib.moe_pack_weights.argtypes = [P(moe.moe_config), ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    assert lib.moe_pack_weights(ctypes.byref(cfg), moe.MOE_PACK_W2, 16, 33, None) == moe.MOE_ERR_INVALID_ARG
    assert "dst" in moe.moe_last_error()
