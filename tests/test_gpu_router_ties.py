"""Exact ties in the router at the largest d_model the library takes (8192). Two experts get the same gate
row, so their keys are equal in fp32 and in fp64: wherever the pair straddles the top-K boundary the
K-th / (K+1)-th gap is zero, the token is re-decided from fp64 logits (the recheck holds a whole 8192-wide
centroid row), and the lower expert index must win, as in the oracle's (key descending, index ascending)
order."""
import numpy as np
import pytest
import torch

import fine_grained_mixture_gemm_amd as moe
from synth import configs
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("act", ["bf16", "f32"])
def test_exact_tie_recheck_at_max_width(act):
    base = configs.WORKLOADS["dsmoe2b_bf16"] if act == "bf16" else configs.WORKLOADS["tiny_f32"]
    w = base.replace(name=f"tie_max_d_{act}", T=300, d=8192, E=8, K=2, f=512 if act == "bf16" else 64, zipf=None)
    print(f"[case] tie at d = 8192, {act} tokens", flush=True)
    g = H.build(w, keep_host_weights=False)
    g.t["wg"][1].copy_(g.t["wg"][0])
    g.wg[1] = g.wg[0]
    ws = H.workspace(g, poison=True)
    idx = torch.empty((w.T, w.K), dtype=torch.int32, device=H.DEV)
    gw = torch.empty((w.T, w.K), dtype=torch.float32, device=H.DEV)
    moe.moe_route(g.cfg, g.layer, g.t["u"], g.t["bias"], idx, gw, ws)
    torch.cuda.synchronize()
    _, r = H.oracle_route(g)
    got = idx.cpu().numpy()
    assert np.array_equal(got, r["idx"]), f"routing differs on {(got != r['idx']).any(1).sum()} tokens"
    has0, has1 = (r["idx"] == 0).any(1), (r["idx"] == 1).any(1)
    straddle = has0 ^ has1
    print(f"tokens whose top-{w.K} holds exactly one of the tied pair: {int(straddle.sum())}", flush=True)
    assert straddle.sum() > 0, "no token put the tied pair across the top-K boundary"
    assert not has1[straddle].any(), "the higher index of a tied pair was chosen"
    assert np.abs(gw.cpu().numpy() - r["w"]).max() <= 1e-5
