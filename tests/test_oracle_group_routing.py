"""Pins of group-limited (device/node-limited) routing in the oracle ([TR] §2.3 device-limited routing,
M = 3 devices; §3.2 / §3.8 node-limited routing, M = 4 nodes). The group-scoring rule is a reading (the
largest key of a group; see oracle.moe.group_limit): these tests pin it by hand examples, by its
reduction to ungrouped routing, and by checking the defining order properties on integer keys full of
ties."""
import numpy as np
import pytest

from oracle import moe


def test_hand_example_one_group():
    # groups {0,1} {2,3} {4,5} score 5, 4, 9: M = 1 keeps group 2 although expert 0 (key 5) beats
    # expert 4 (key 0); the group choice is decided by 9 - 5 = 4
    key = np.array([[5, 1, 4, 4, 0, 9]], dtype=np.float64)
    r = moe.route(key, "softmax", 2, n_groups=3, topk_groups=1)
    assert r["idx"].tolist() == [[4, 5]]
    masked, ggap = moe.group_limit(key, 3, 1)
    assert ggap.tolist() == [4.0]
    assert np.isneginf(masked[0, :4]).all()


def test_hand_example_two_groups():
    # M = 2 keeps groups 2 (9) and 0 (5): allowed {0, 1, 4, 5}; the top 2 of those are experts 5 and 0
    key = np.array([[5, 1, 4, 4, 0, 9]], dtype=np.float64)
    assert moe.route(key, "softmax", 2, n_groups=3, topk_groups=2)["idx"].tolist() == [[0, 5]]


def test_tied_groups_go_to_the_lower_index():
    key = np.array([[3, 0, 3, 0, 1, 1]], dtype=np.float64)
    r = moe.route(key, "softmax", 1, n_groups=3, topk_groups=1)
    assert r["idx"].tolist() == [[0]]
    assert r["gap"].tolist() == [0.0]


@pytest.mark.parametrize("gate", ["softmax", "sigmoid_bias"])
def test_reduces_to_ungrouped_routing(gate):
    rng = np.random.default_rng(0)
    z = rng.normal(0, 2, (50, 24))
    b = rng.uniform(-0.1, 0.1, 24) if gate == "sigmoid_bias" else None
    plain = moe.route(z, gate, 5, b, True)
    for G, M in ((1, 1), (4, 4), (8, 8)):
        r = moe.route(z, gate, 5, b, True, n_groups=G, topk_groups=M)
        assert np.array_equal(r["idx"], plain["idx"])
        assert np.array_equal(r["w"], plain["w"])


def test_gates_are_the_ungrouped_formula_on_the_limited_selection():
    rng = np.random.default_rng(1)
    z = rng.normal(0, 2, (20, 16))
    b = rng.uniform(-0.1, 0.1, 16)
    r = moe.route(z, "sigmoid_bias", 3, b, True, n_groups=4, topk_groups=2)
    s = moe.sigmoid(z)
    g = np.take_along_axis(s, r["idx"].astype(np.int64), axis=1)
    assert np.allclose(r["w"], g / g.sum(axis=1, keepdims=True), rtol=0, atol=1e-15)
    p = moe.softmax(z)
    r2 = moe.route(z, "softmax", 3, n_groups=4, topk_groups=2)
    assert np.allclose(r2["w"], np.take_along_axis(p, r2["idx"].astype(np.int64), axis=1), rtol=0, atol=1e-15)


def _before(a, ia, b, ib):
    """(a, ia) ranks before (b, ib) under (value descending, index ascending)."""
    return a > b or (a == b and ia < ib)


@pytest.mark.parametrize("seed", range(6))
def test_order_properties_on_integer_keys_with_ties(seed):
    rng = np.random.default_rng(seed)
    E = int(rng.choice([6, 8, 12, 16]))
    divisors = [g for g in range(1, E + 1) if E % g == 0]
    G = int(rng.choice(divisors))
    M = int(rng.integers(1, G + 1))
    gsz = E // G
    K = int(rng.integers(1, M * gsz + 1))
    key = rng.integers(0, 4, (40, E)).astype(np.float64)     # many ties
    idx = moe.route(key, "softmax", K, n_groups=G, topk_groups=M)["idx"]
    for t in range(key.shape[0]):
        sel = set(idx[t].tolist())
        assert len(sel) == K
        groups = {e // gsz for e in sel}
        assert len(groups) <= M
        score = key[t].reshape(G, gsz).max(axis=1)
        # the kept groups are exactly the M first under (score desc, group asc)
        ranked = sorted(range(G), key=lambda g: (-score[g], g))
        kept = set(ranked[:M])
        assert groups <= kept
        for g in kept:
            for h in set(range(G)) - kept:
                assert _before(score[g], g, score[h], h)
        # among the experts of the kept groups, every selected one ranks before every other
        allowed = [e for e in range(E) if e // gsz in kept]
        for e in sel:
            for f in set(allowed) - sel:
                assert _before(key[t, e], e, key[t, f], f)


def test_rejects_impossible_limits():
    key = np.zeros((2, 8))
    for G, M, K in ((3, 1, 1), (4, 0, 1), (4, 5, 1), (4, 1, 3)):
        with pytest.raises(ValueError):
            moe.route(key, "softmax", K, n_groups=G, topk_groups=M)
