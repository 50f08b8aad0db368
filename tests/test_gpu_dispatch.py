"""moe_dispatch and moe_combine on caller-given expert ids, bit for bit against the semantics include/moe.h
states: a (token, slot) pair whose id lies outside [0, E) or repeats an id of an earlier slot of the same
token gets no row and row_of = -1; every other pair gets one row, the rows of an expert in ascending
token order; the combine adds the gate-weighted rows of the kept pairs only. Both dispatch paths run:
one block for T <= 256, the chunked histogram / scan / scatter above."""
import numpy as np
import pytest
import torch

import fine_grained_mixture_gemm_amd as moe
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


def host_dispatch(idx: np.ndarray, E: int):
    """The documented dispatch, by a plain loop over tokens and slots."""
    T, K = idx.shape
    kept = np.zeros((T, K), dtype=bool)
    for t in range(T):
        seen = set()
        for k in range(K):
            e = int(idx[t, k])
            if 0 <= e < E and e not in seen:
                kept[t, k] = True
                seen.add(e)
    counts = np.bincount(idx[kept], minlength=E).astype(np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    nxt = offsets[:-1].copy()
    perm = np.zeros(int(offsets[-1]), dtype=np.int32)
    row_of = np.full((T, K), -1, dtype=np.int32)
    for t in range(T):                     # tokens ascending: rows of an expert come out in token order
        for k in range(K):
            if kept[t, k]:
                e = int(idx[t, k])
                row_of[t, k] = nxt[e]
                perm[nxt[e]] = t
                nxt[e] += 1
    return counts, offsets, perm, row_of


def _ids(rng, T, E, K):
    """Distinct valid ids per token, then a share of them replaced by out-of-range ids and by repeats."""
    idx = np.stack([rng.choice(E, size=K, replace=False) for _ in range(T)]).astype(np.int32)
    r = rng.random((T, K))
    idx[r < 0.05] = -1
    idx[(r >= 0.05) & (r < 0.08)] = E
    idx[(r >= 0.08) & (r < 0.10)] = E + 1000
    dup = (r >= 0.10) & (r < 0.15)
    for t, k in zip(*np.nonzero(dup)):
        idx[t, k] = idx[t, rng.integers(0, K)]        # may repeat an earlier or a later slot, or itself
    idx[0, K - 1] = E + 5                             # at least one dropped pair
    return idx


CASES = [(1, 16, 4), (64, 256, 8), (256, 64, 6), (257, 256, 8), (1000, 32, 16), (3000, 256, 8)]


@pytest.mark.parametrize("T,E,K", CASES)
def test_dispatch_with_invalid_and_repeated_ids(T, E, K):
    print(f"[case] dispatch T={T} E={E} K={K}", flush=True)
    rng = np.random.default_rng(T * 1000 + E + K)
    cfg = moe.make_config(T, 256, E, 1, K, 128, moe.MOE_GATE_SIGMOID_BIAS, 1, moe.MOE_BF16, moe.MOE_FP8_E4M3)
    idx = _ids(rng, T, E, K)
    counts, offsets, perm, row_of = host_dispatch(idx, E)
    assert (row_of < 0).any() and (row_of >= 0).any()
    ws = torch.empty(moe.moe_workspace_size(cfg), dtype=torch.uint8, device=H.DEV)
    d_idx = torch.from_numpy(idx).to(H.DEV)
    o_counts = torch.full((E,), -7, dtype=torch.int32, device=H.DEV)
    o_offsets = torch.full((E + 1,), -7, dtype=torch.int32, device=H.DEV)
    o_perm = torch.full((T * K,), -7, dtype=torch.int32, device=H.DEV)
    o_row = torch.full((T, K), -7, dtype=torch.int32, device=H.DEV)
    moe.moe_dispatch(cfg, d_idx, o_counts, o_offsets, o_perm, o_row, ws)
    torch.cuda.synchronize()
    assert np.array_equal(o_counts.cpu().numpy(), counts)
    assert np.array_equal(o_offsets.cpu().numpy(), offsets)
    assert np.array_equal(o_perm.cpu().numpy()[:offsets[-1]], perm)
    assert np.array_equal(o_row.cpu().numpy(), row_of)


@pytest.mark.parametrize("wdt", ["fp8", "bf16"])
def test_combine_skips_dropped_pairs(wdt):
    """Small integers and gates of 1 or 2 keep every sum exact in fp32 and in the bf16 output."""
    T, E, K, d = 300, 16, 4, 256
    print(f"[case] combine {wdt}", flush=True)
    rng = np.random.default_rng(3)
    cfg = moe.make_config(T, d, E, 1, K, 128, moe.MOE_GATE_SIGMOID_BIAS, 1, moe.MOE_BF16,
                          moe.MOE_FP8_E4M3 if wdt == "fp8" else moe.MOE_BF16)
    idx = _ids(rng, T, E, K)
    counts, offsets, perm, row_of = host_dispatch(idx, E)
    ydt = torch.bfloat16 if wdt == "fp8" else torch.float32
    u = rng.integers(-4, 5, size=(T, d)).astype(np.float32)
    ys = rng.integers(-4, 5, size=(T, d)).astype(np.float32)
    yr = rng.integers(-4, 5, size=(T * K, d)).astype(np.float32)
    w = rng.choice([1.0, 2.0], size=(T, K)).astype(np.float32)
    ref = u + ys
    for t in range(T):
        for k in range(K):
            if row_of[t, k] >= 0:
                ref[t] += w[t, k] * yr[row_of[t, k]]
    h = torch.empty((T, d), dtype=torch.bfloat16, device=H.DEV)
    moe.moe_combine(cfg, torch.from_numpy(u).to(H.DEV, torch.bfloat16), torch.from_numpy(yr).to(H.DEV, ydt),
                    torch.from_numpy(ys).to(H.DEV, ydt), torch.from_numpy(row_of).to(H.DEV), torch.from_numpy(w).to(H.DEV), h)
    torch.cuda.synchronize()
    assert np.array_equal(h.float().cpu().numpy(), ref)


def test_combine_rounds_fp32_to_bf16_to_nearest_even():
    """The combine's fp32 -> bf16 output rounding on every fp32 exponent with the low 16 mantissa bits below,
    at and above the rounding midpoint (all 128 high-mantissa patterns, both signs), and on three whole
    binades (around 1, the smallest normal, the largest subnormal): h = u + y_shared + 1 * y with u and
    y_shared zero is bf16(y), compared with torch's round-to-nearest-even conversion on the CPU."""
    d = 1024
    hi = np.arange(256 * 128, dtype=np.uint32)            # exponent (8 bits) and top 7 mantissa bits
    lows = np.array([0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF], dtype=np.uint32)
    bits = ((hi[:, None] << 16) | lows[None, :]).reshape(-1)
    whole = [((np.uint32(e) << 23) | np.arange(1 << 23, dtype=np.uint32)) for e in (127, 1, 0)]
    bits = np.concatenate([bits] + whole)
    bits = np.concatenate([bits, bits | np.uint32(0x80000000)])
    vals = bits.view(np.float32)
    vals = vals[np.isfinite(vals) & (vals != 0)]
    vals = vals[np.abs(vals.astype(np.float64)) < 3.3e38]   # beyond this bf16 rounds to infinity
    T = -(-len(vals) // d)
    y = np.zeros(T * d, dtype=np.float32)
    y[:len(vals)] = vals
    y = y.reshape(T, d)
    print(f"[case] bf16 rounding, {len(vals)} values", flush=True)
    cfg = moe.make_config(T, d, 1, 1, 1, 128, moe.MOE_GATE_SOFTMAX, 0, moe.MOE_BF16, moe.MOE_BF16)
    zero_u = torch.zeros((T, d), dtype=torch.bfloat16, device=H.DEV)
    zero_s = torch.zeros((T, d), dtype=torch.float32, device=H.DEV)
    row_of = torch.arange(T, dtype=torch.int32, device=H.DEV).view(T, 1)
    w = torch.ones((T, 1), dtype=torch.float32, device=H.DEV)
    h = torch.empty((T, d), dtype=torch.bfloat16, device=H.DEV)
    moe.moe_combine(cfg, zero_u, torch.from_numpy(y).to(H.DEV), zero_s, row_of, w, h)
    torch.cuda.synchronize()
    got = h.view(torch.int16).cpu().numpy().reshape(-1)[:len(vals)]
    ref = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy()
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, f"{bad.size} values round differently, e.g. {vals[bad[:4]]}"
