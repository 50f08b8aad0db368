"""moe_forward_noalloc (the entry point for callers that cannot allocate) against moe_forward with a
caller workspace: identical routing, counts and h, bit for bit, on two calls in a row, the second with a
smaller batch (the static scratch keeps the first call's contents)."""
import pytest
import torch

import fine_grained_mixture_gemm_amd as moe
from synth import configs
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

W = configs.WORKLOADS
CASES = [
    # E4M3 tiled path (T > 128), then the decode kernels (T <= 128) on the same weights
    ("fp8", W["v3_fp8"].replace(name="noalloc_fp8", T=300, d=512, E=20, K=4), 40),
    # bf16 softmax with a shared expert, then a ragged smaller batch
    ("bf16", W["dsmoe2b_bf16"].replace(name="noalloc_bf16", T=260, d=256, E=12, K=3, f=128), 33),
    ("f32", W["tiny_f32"], 17),
]


def _reference(g):
    ws = H.workspace(g, poison=True)
    h = torch.empty_like(g.t["u"])
    idx = torch.empty((g.w.T, g.w.K), dtype=torch.int32, device=H.DEV)
    cnt = torch.empty(g.w.E, dtype=torch.int32, device=H.DEV)
    moe.moe_forward(g.cfg, g.layer, g.t["u"], g.t["bias"], h, idx, cnt, ws)
    torch.cuda.synchronize()
    return h, idx, cnt


def _noalloc(g):
    h = torch.full_like(g.t["u"], float("nan"))
    idx = torch.full((g.w.T, g.w.K), -7, dtype=torch.int32, device=H.DEV)
    cnt = torch.full((g.w.E,), -7, dtype=torch.int32, device=H.DEV)
    moe.moe_forward_noalloc(g.cfg, g.layer, g.t["u"], g.t["bias"], h, idx, cnt)
    torch.cuda.synchronize()
    return h, idx, cnt


def _same(a, b):
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a.view(torch.int32), b.view(torch.int32))


@pytest.mark.parametrize("kind,w,t_small", CASES, ids=[c[0] for c in CASES])
def test_noalloc_matches_forward_twice(kind, w, t_small):
    print(f"[case] noalloc {kind} T={w.T} then T={t_small}", flush=True)
    big = H.build(w)
    small = H.build(w.replace(name=w.name + "_small", T=t_small))
    for g in (big, small):
        assert moe.moe_workspace_size(g.cfg) <= moe.MOE_NOALLOC_SCRATCH_BYTES
        got = _noalloc(g)
        ref = _reference(g)
        for x, y in zip(got, ref):
            assert _same(x, y), f"{kind} T={g.w.T}: moe_forward_noalloc differs from moe_forward"


def test_noalloc_rejects_oversized_configs():
    g = H.build(W["tiny_f32"])
    cfg = H.make_cfg(W["v3_fp8"])          # T = 8192 at the V3 shape: about 1.3 GB of scratch
    assert moe.moe_workspace_size(cfg) > moe.MOE_NOALLOC_SCRATCH_BYTES
    with pytest.raises(moe.MoeError) as e:
        moe.moe_forward_noalloc(cfg, g.layer, g.t["u"], None, torch.empty_like(g.t["u"]), None, None)
    assert e.value.status == 3   # MOE_ERR_WORKSPACE
