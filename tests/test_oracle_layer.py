"""Pins of the oracle's experts, dispatch, combine, whole layer and bias update."""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import formats, moe, quant

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "tiny_layer_closed_form.json")))
CONST = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_constants.json")))


def _ev(x):
    env = {"L3": math.log(3.0), "S1": math.e / (1 + math.e), "__builtins__": {}}
    if isinstance(x, list):
        return [_ev(v) for v in x]
    return float(eval(x, env)) if isinstance(x, str) else float(x)


def _torch_mlp(x, w1, w3, w2):
    """Textbook SwiGLU MLP through torch's own SiLU (float64)."""
    t = lambda a: torch.as_tensor(np.asarray(a, dtype=np.float64))
    x = t(x)
    return (torch.nn.functional.silu(x @ t(w1).T) * (x @ t(w3).T) @ t(w2).T).numpy()


def _rand_layer(rng, T, d, E, f, Ks):
    experts = [(rng.normal(size=(f, d)) / math.sqrt(d), rng.normal(size=(f, d)) / math.sqrt(d),
                rng.normal(size=(d, f)) / math.sqrt(f)) for _ in range(E)]
    shared = (rng.normal(size=(Ks * f, d)) / math.sqrt(d), rng.normal(size=(Ks * f, d)) / math.sqrt(d),
              rng.normal(size=(d, Ks * f)) / math.sqrt(f))
    u = rng.normal(size=(T, d))
    wg = rng.normal(size=(E, d)) / math.sqrt(d)
    return u, wg, experts, shared


@pytest.mark.parametrize("case", GOLD["cases"], ids=lambda c: c["name"])
def test_worked_example_closed_form(case):
    inp = GOLD["inputs"]
    experts = [(np.array(_ev(e["w1"])), np.array(_ev(e["w3"])), np.array(_ev(e["w2"]))) for e in inp["experts"]]
    sh = inp["shared"]
    shared = (np.array(_ev(sh["w1"])), np.array(_ev(sh["w3"])), np.array(_ev(sh["w2"])))
    out = moe.layer_forward(np.array(_ev(inp["u"])), np.array(_ev(inp["w_gate"])), experts, shared,
                            gate=case["gate"], K=case["K"], renorm=case["renorm"],
                            bias=None if case["bias"] is None else np.array(case["bias"]))
    assert out["idx"].tolist() == case["idx"]
    assert np.allclose(out["w"], np.array(_ev(case["gates"])), rtol=0, atol=1e-15)
    assert np.allclose(out["h"], np.array(_ev(case["h"])), rtol=0, atol=1e-14)


def test_silu_closed_forms():
    assert moe.silu(np.array([0.0]))[0] == 0.0
    assert abs(moe.silu(np.array([math.log(3)]))[0] - 0.75 * math.log(3)) < 1e-15
    assert abs(moe.silu(np.array([-math.log(3)]))[0] + 0.25 * math.log(3)) < 1e-15


def test_ffn_matches_torch_mlp():
    rng = np.random.default_rng(0)
    _, _, experts, _ = _rand_layer(rng, 1, 96, 1, 40, 1)
    x = rng.normal(size=(17, 96))
    assert np.allclose(moe.swiglu_ffn(x, *experts[0]), _torch_mlp(x, *experts[0]), rtol=1e-13, atol=1e-14)


def test_single_expert_layer_is_dense_mlp_plus_shared():
    rng = np.random.default_rng(1)
    u, wg, experts, shared = _rand_layer(rng, 23, 64, 1, 32, 2)
    out = moe.layer_forward(u, wg, experts, shared, gate="softmax", K=1)
    assert np.all(out["w"] == 1.0)
    ref = u + _torch_mlp(u, *shared) + _torch_mlp(u, *experts[0])
    assert np.allclose(out["h"], ref, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("gate,renorm,K", [("softmax", False, 3), ("sigmoid_bias", True, 4)])
def test_dense_masked_equals_sparse(gate, renorm, K):
    rng = np.random.default_rng(2)
    u, wg, experts, shared = _rand_layer(rng, 50, 48, 12, 16, 1)
    b = rng.uniform(-0.1, 0.1, 12) if gate == "sigmoid_bias" else None
    sp = moe.layer_forward(u, wg, experts, shared, gate=gate, K=K, bias=b, renorm=renorm)
    de = moe.layer_forward_dense(u, wg, experts, shared, gate=gate, K=K, bias=b, renorm=renorm)
    assert np.allclose(sp["h"], de, rtol=1e-12, atol=1e-12)
    assert np.allclose(sp["h"], u + sp["y_shared"] + sp["routed"], rtol=1e-13, atol=1e-13)


def test_dense_masked_equals_sparse_fp8_bitwise():
    rng = np.random.default_rng(3)
    u, wg, experts, shared = _rand_layer(rng, 40, 256, 6, 128, 1)
    q = lambda e: (*quant.quantize_weight_128x128(np.vstack([e[0], e[1]])), *quant.quantize_weight_128x128(e[2]))
    ex8 = [q(e) for e in experts]
    sh8 = q(shared)
    b = rng.uniform(-0.1, 0.1, 6)
    sp = moe.layer_forward(u, wg, ex8, sh8, gate="sigmoid_bias", K=3, bias=b, renorm=True, fp8=True)
    de = moe.layer_forward_dense(u, wg, ex8, sh8, gate="sigmoid_bias", K=3, bias=b, renorm=True, fp8=True)
    assert np.array_equal(sp["h"], de)


def test_fp8_ffn_close_to_float_ffn():
    # E4M3 keeps 3 mantissa bits: per-element rounding is up to 2^-4 relative, so the fp8 expert
    # differs from the float expert by a few percent of the output RMS.
    rng = np.random.default_rng(4)
    _, _, experts, _ = _rand_layer(rng, 1, 256, 1, 256, 1)
    x = rng.normal(size=(30, 256))
    w1, w3, w2 = experts[0]
    w13q, w13s = quant.quantize_weight_128x128(np.vstack([w1, w3]))
    w2q, w2s = quant.quantize_weight_128x128(w2)
    y8, _ = moe.swiglu_ffn_fp8(x, w13q, w13s, w2q, w2s)
    y = moe.swiglu_ffn(x, w1, w3, w2)
    rms = np.sqrt((y ** 2).mean())
    assert np.sqrt(((y8 - y) ** 2).mean()) / rms < 0.1
    assert np.abs(y8 - y).max() / rms < 0.5


def test_fp8_gate_up_exact_for_representable_operands():
    # operands that E4M3 holds exactly, with every tile / block maximum at 448, get unit scales:
    # the block-scaled gate/up product is then the exact float product and SiLU(g) * v follows it.
    rng = np.random.default_rng(7)
    x = rng.integers(-16, 17, size=(20, 256)).astype(np.float64)
    x[:, [0, 128]] = 448.0
    w = rng.integers(-16, 17, size=(256, 256)).astype(np.float64)
    w[:, [0, 128]] = 448.0
    w13q, w13s = quant.quantize_weight_128x128(w)
    assert np.all(w13s == 1.0)
    w2q, w2s = quant.quantize_weight_128x128(np.eye(128).repeat(2, axis=0)[:128] * 448.0)
    _, a = moe.swiglu_ffn_fp8(x, w13q, w13s, w2q, w2s)
    gv = x @ w.T
    assert np.array_equal(a, moe.silu(gv[:, :128]) * gv[:, 128:])


def test_dispatch_and_unpermute_identity():
    rng = np.random.default_rng(5)
    T, E, K = 97, 11, 3
    idx = np.sort(np.array([rng.choice(E, K, replace=False) for _ in range(T)]), axis=1).astype(np.int32)
    offsets, perm_src, row_of = moe.dispatch(idx, E)
    counts = moe.expert_counts(idx, E)
    assert counts.sum() == T * K and offsets[-1] == T * K
    assert np.array_equal(np.diff(offsets), counts)
    for e in range(E):
        toks = perm_src[offsets[e]:offsets[e + 1]]
        assert np.array_equal(toks, np.sort(np.nonzero((idx == e).any(axis=1))[0]))
    # permute then unpermute is the identity, bitwise
    x = rng.normal(size=(T, 8))
    xp = x[perm_src]
    for k in range(K):
        assert np.array_equal(xp[row_of[:, k]], x)
        assert np.all(perm_src[row_of[:, k]] == np.arange(T))
    # identity experts with unit gates: combine(u = 0, no shared) returns K copies of x
    h = moe.combine(np.zeros_like(x), np.zeros_like(x), xp, row_of, np.ones((T, K)))
    assert np.array_equal(h, K * x)


def test_bias_update_rule():
    gamma = CONST["bias_update_speed_gamma"]["value"]
    T, K, E = 64, 8, 4
    b = np.array([0.05, -0.02, 0.0, 0.1], dtype=np.float32)
    counts = np.array([200, 128, 100, 84])          # mean load T*K/E = 128
    nb = moe.bias_update(b, counts, gamma, T, K)
    g = np.float32(gamma)
    assert nb[0] == np.float32(b[0] - g) and nb[1] == b[1] and nb[2] == np.float32(b[2] + g)
    assert nb[3] == np.float32(b[3] + g) and nb.dtype == np.float32
    # repeated updates drive an overloaded expert's bias down by gamma per step
    bb = b.copy()
    for _ in range(10):
        bb = moe.bias_update(bb, counts, gamma, T, K)
    assert abs(float(bb[0]) - (0.05 - 10 * gamma)) < 1e-6


def test_gap_reported_for_selection_margin():
    rng = np.random.default_rng(6)
    z = rng.normal(size=(1000, 32))
    r = moe.route(z, "softmax", 4)
    srt = -np.sort(-z, axis=1)
    assert np.allclose(r["gap"], srt[:, 3] - srt[:, 4], rtol=0, atol=0)
