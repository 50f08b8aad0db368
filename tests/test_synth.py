"""The seeded input generator: its definition, determinism and distributions."""
import numpy as np
import torch

from synth import configs, gen


def test_splitmix64_reference_outputs():
    # First outputs of SplitMix64 started from state 0, as published with the generator
    # (Vigna's reference splitmix64.c): the key-0 stream is exactly that sequence.
    ref = [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]
    assert [int(x) for x in gen.words(0, 0, 3)] == ref
    assert [gen.mix64_int(gen.GOLDEN * (i + 1)) for i in range(3)] == ref


def test_words_random_access_matches_sequence():
    key = gen.tensor_key(7, 123)
    full = gen.words(key, 0, 1000)
    assert np.array_equal(full[300:400], gen.words(key, 300, 100))
    assert int(full[5]) == gen.mix64_int(key + gen.GOLDEN * 6)


def test_normal_slices_and_determinism():
    a = gen.normal_f32(3, 44, (64, 128), 0.5)
    b = gen.normal_f32(3, 44, (16, 128), 0.5, start=32 * 128)
    assert np.array_equal(a[32:48], b)
    assert np.array_equal(a, gen.normal_f32(3, 44, (64, 128), 0.5))
    assert not np.array_equal(a, gen.normal_f32(3, 45, (64, 128), 0.5))


def test_normal_moments_and_support():
    x = gen.normal_f32(1, 2, (2_000_000,), 0.25).astype(np.float64)
    assert abs(x.mean()) < 3 * 0.25 / np.sqrt(x.size) * 3
    assert abs(x.std() / 0.25 - 1) < 3e-3
    assert np.abs(x).max() <= 0.25 * 262140 / gen.IH4_STD * (1 + 1e-6)
    # Irwin-Hall(4) excess kurtosis is -6/(5*4) = -0.3
    k = ((x - x.mean()) ** 4).mean() / x.var() ** 2 - 3
    assert abs(k + 0.3) < 0.02


def test_normal_is_integer_sum_times_fp32_scale():
    w = gen.words(gen.tensor_key(0, 0), 0, 4)
    x = gen.normal_from_words(w, 1.0)
    for i in range(4):
        wi = int(w[i])
        s = sum(2 * ((wi >> (16 * j)) & 0xFFFF) - 65535 for j in range(4))
        assert x[i] == np.float32(np.float32(s) * gen.normal_scale(1.0))


def test_bf16_rounding_matches_torch():
    x = gen.normal_f32(5, 6, (100_000,), 3.0)
    # add exact ties and near-ties of the bf16 grid
    base = x.view(np.uint32) & np.uint32(0xFFFF0000)
    ties = (base | np.uint32(0x8000)).view(np.float32)
    near = (base | np.uint32(0x7FFF)).view(np.float32)
    for v in (x, ties, near):
        ref = torch.from_numpy(v.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(gen.f32_to_bf16_bits(v), ref)
    assert np.array_equal(gen.bf16_bits_to_f32(gen.f32_to_bf16_bits(ties)),
                          torch.from_numpy(ties).to(torch.bfloat16).float().numpy())


def test_uniform_and_permutation():
    b = gen.uniform_f32(3, 2, (4096,), -0.1, 0.1)
    assert b.min() >= -0.1 and b.max() < 0.1 and abs(b.mean()) < 0.005
    p = gen.random_permutation(1, 3, 63)
    assert sorted(p.tolist()) == list(range(63))


def test_workload_router_inputs():
    w = configs.WORKLOADS["dsmoe2b_bf16"]
    wg, bias, off = configs.make_router(w)
    assert wg.shape == (63, 1024) and bias is None
    # Zipf offsets: exactly one expert has rank 1 (offset 0), ranks are a permutation of 1..E
    r = np.exp(-off.astype(np.float64) / 1.1)
    assert np.allclose(np.sort(r), np.arange(1, 64), rtol=1e-6)
    w4 = configs.WORKLOADS["v3_fp8"]
    _, b4, o4 = configs.make_router(w4)
    assert o4 is None and b4.shape == (256,) and np.abs(b4).max() < 0.1


def test_decode_workload_reuses_v3_tokens():
    w4 = configs.WORKLOADS["v3_fp8"].replace(T=80)
    w5 = configs.WORKLOADS["v3_fp8_decode"]
    assert np.array_equal(configs.make_u(w4)[:64], configs.make_u(w5))


def test_workload_shapes_follow_the_pages():
    import json, os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_constants.json")))
    v3, w4, w5 = g["v3_moe"]["value"], configs.WORKLOADS["v3_fp8"], configs.WORKLOADS["v3_fp8_decode"]
    for w in (w4, w5):
        assert (w.d, w.f, w.E, w.K, w.Ks) == (v3["hidden"], v3["moe_inter"], v3["routed"], v3["per_token"], v3["shared"])
        assert w.gate == "sigmoid_bias" and w.wdt == "fp8"
    assert w5.gamma == g["bias_update_speed_gamma"]["value"]
    b2, w2 = g["dsmoe_2b"]["value"], configs.WORKLOADS["dsmoe2b_bf16"]
    assert (w2.Ks, w2.E, w2.K) == (b2["shared"], b2["routed"], b2["active_routed"])
    assert w2.f == b2["expert_size_vs_ffn"] * 4 * w2.d
    b16, w3 = g["dsmoe_16b"]["value"], configs.WORKLOADS["dsmoe16b_bf16"]
    assert (w3.Ks, w3.E, w3.K, w3.d) == (b16["shared"], b16["routed"], b16["active_routed"], b16["hidden"])


def test_heavy_tailed_rows_are_exact_power_of_two_scalings():
    # u_tail scales whole rows by 32 or 8 and single elements by 64 (powers of two: exact in fp32), from
    # the words of their own stream; the rest of u is the plain draw
    w = configs.WORKLOADS["tiny_f32"].replace(T=400, u_tail=True)
    plain = configs.make_u(w.replace(u_tail=False))
    tail = configs.make_u(w)
    row, spikes, cols = configs.tail_factors(w)
    expect = plain * row[:, None]
    expect[spikes, cols] *= 64.0
    assert np.array_equal(tail, expect)
    assert 0.03 < (row == 32).mean() < 0.1 and 0.08 < (row == 8).mean() < 0.2 and 0.03 < len(spikes) / w.T < 0.1
    assert np.array_equal(configs.tail_factors(w)[0], row)          # a pure function of (seed, T)
