"""An empty batch (T = 0) through the forward entry points. Each returns OK without touching its empty
arrays (passed as NULL, which T = 0 allows); moe_forward, moe_forward_noalloc and moe_dispatch write all-zero
counts (and offsets); and the bias update that follows leaves every bias unchanged, since each expert's load,
zero, equals the mean load T * K / E = 0 (DeepSeek Technical Report: MoE Architecture, 3.3, bias update)."""
import pytest
import torch

import fine_grained_mixture_gemm_amd as moe
from synth import configs
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

W = configs.WORKLOADS
CASES = {
    "fp8": W["v3_fp8"].replace(name="empty_fp8", T=64, d=512, E=20, K=4),
    "bf16": W["dsmoe2b_bf16"].replace(name="empty_bf16", T=64, d=256, E=12, K=3, f=128),
    "f32": W["tiny_f32"],
}


def _i32(n, fill=-7):
    return torch.full((n,), fill, dtype=torch.int32, device=H.DEV)


@pytest.mark.parametrize("name", list(CASES))
def test_empty_batch(name):
    print(f"[case] empty batch {name}", flush=True)
    g = H.build(CASES[name], keep_host_weights=False)
    w = g.w.replace(T=0)
    cfg = H.make_cfg(w)
    u = g.t["u"][:0]
    h = torch.empty_like(u)
    ws = torch.full((max(moe.moe_workspace_size(cfg), 256),), 0xFF, dtype=torch.uint8, device=H.DEV)
    none_i32 = torch.empty(0, dtype=torch.int32, device=H.DEV)
    none_f32 = torch.empty(0, dtype=torch.float32, device=H.DEV)

    cnt = _i32(w.E)
    moe.moe_forward(cfg, g.layer, u, g.t["bias"], h, none_i32, cnt, ws)
    cnt_na = _i32(w.E)
    moe.moe_forward_noalloc(cfg, g.layer, u, g.t["bias"], h, none_i32, cnt_na)
    moe.moe_route(cfg, g.layer, u, g.t["bias"], none_i32, none_f32, ws)
    cnt_d, off_d = _i32(w.E), _i32(w.E + 1)
    moe.moe_dispatch(cfg, none_i32, cnt_d, off_d, none_i32, none_i32, ws)
    moe.moe_expert_ffn(cfg, g.layer, u, off_d, none_i32, none_f32, none_f32, ws)
    moe.moe_combine(cfg, u, none_f32, none_f32, none_i32, none_f32, h)
    torch.cuda.synchronize()
    for label, x in (("moe_forward counts", cnt), ("moe_forward_noalloc counts", cnt_na),
                     ("moe_dispatch counts", cnt_d), ("moe_dispatch offsets", off_d)):
        assert torch.all(x == 0), f"{name}: {label} not all zero: {x.tolist()}"

    if g.t["bias"] is not None:
        b = g.t["bias"].clone()
        moe.moe_update_bias(cfg, cnt, 0.001, b)
        torch.cuda.synchronize()
        assert torch.equal(b.view(torch.int32), g.t["bias"].view(torch.int32)), f"{name}: bias moved on an empty batch"
