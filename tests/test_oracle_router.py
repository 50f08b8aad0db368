"""Pins of the oracle's gating and top-K selection."""
import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special

from oracle import moe

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_constants.json")))


def _brute_topk(key_row, K):
    """The K-subset with the largest key sum; among equal sums the lexicographically smallest
    ascending index tuple (i.e. ties go to the lower expert index)."""
    best, best_s = None, -np.inf
    for sub in itertools.combinations(range(len(key_row)), K):
        s = sum(key_row[i] for i in sub)
        if s > best_s:
            best, best_s = sub, s
    return list(best)


@pytest.mark.parametrize("E,K", [(6, 2), (8, 3), (7, 7), (9, 1)])
def test_topk_equals_brute_force_with_ties(E, K):
    rng = np.random.default_rng(E * 10 + K)
    keys = rng.integers(0, 4, size=(200, E)).astype(np.float64)   # many exact ties
    idx, gap = moe.topk_select(keys, K)
    for t in range(200):
        assert idx[t].tolist() == _brute_topk(keys[t].tolist(), K)
    srt = -np.sort(-keys, axis=1)
    exp_gap = srt[:, K - 1] - srt[:, K] if K < E else np.full(200, np.inf)
    assert np.array_equal(gap, exp_gap)


def test_number_of_distinct_top2_of_16_sets():
    # Every top-2 set of 16 experts is reachable and distinct: C(16,2) sets.
    sets = set()
    for i, j in itertools.combinations(range(16), 2):
        key = np.zeros((1, 16))
        key[0, [i, j]] = [2.0, 1.0]
        sets.add(tuple(moe.topk_select(key, 2)[0][0]))
    assert len(sets) == GOLDEN["combinations_top2_of_16"]["value"] == math.comb(16, 2)
    assert GOLDEN["combinations_top8_of_64"]["value"] == math.comb(64, 8)


def test_zero_gate_weights_tie_break():
    u = np.random.default_rng(0).normal(size=(5, 32))
    z = moe.router_logits(u, np.zeros((16, 32)))
    r = moe.route(z, "softmax", 3)
    assert np.all(r["idx"] == [0, 1, 2]) and np.allclose(r["w"], 1 / 16, rtol=0, atol=1e-16)
    r = moe.route(z, "sigmoid_bias", 4, bias=np.zeros(16), renorm=False)
    assert np.all(r["idx"] == [0, 1, 2, 3]) and np.all(r["w"] == 0.5)
    r = moe.route(z, "sigmoid_bias", 4, bias=np.zeros(16), renorm=True)
    assert np.all(r["w"] == 0.25)


def test_zero_logits_bias_selects_top_bias():
    b = np.random.default_rng(1).uniform(-0.1, 0.1, 32).astype(np.float32)
    r = moe.route(np.zeros((3, 32)), "sigmoid_bias", 8, bias=b, renorm=True)
    assert np.all(r["idx"] == np.sort(np.argsort(-b.astype(np.float64), kind="stable")[:8]))
    assert np.allclose(r["w"], 1 / 8)


def test_bias_forces_expert_and_never_enters_gate():
    rng = np.random.default_rng(2)
    z = rng.normal(size=(50, 20))
    b = np.zeros(20)
    b[13] = 10.0
    r = moe.route(z, "sigmoid_bias", 4, bias=b, renorm=True)
    assert np.all((r["idx"] == 13).sum(axis=1) == 1)
    s = scipy.special.expit(z)
    sel = np.take_along_axis(s, r["idx"].astype(int), axis=1)
    assert np.allclose(r["w"], sel / sel.sum(axis=1, keepdims=True), rtol=1e-15)
    # a bias that leaves the selected set unchanged leaves the gates bitwise unchanged
    r0 = moe.route(z, "sigmoid_bias", 4, bias=np.zeros(20), renorm=True)
    r1 = moe.route(z, "sigmoid_bias", 4, bias=np.full(20, 0.3), renorm=True)
    assert np.array_equal(r0["idx"], r1["idx"]) and np.array_equal(r0["w"], r1["w"])


def test_softmax_gates_and_library_agreement():
    rng = np.random.default_rng(3)
    z = rng.normal(size=(40, 64)) * 3
    r = moe.route(z, "softmax", 6)
    p = scipy.special.softmax(z, axis=1)
    assert np.allclose(moe.softmax(z).sum(axis=1), 1.0, rtol=0, atol=1e-15)
    assert np.allclose(r["w"], np.take_along_axis(p, r["idx"].astype(int), axis=1), rtol=1e-14)
    # softmax selection equals selection by probability
    order = np.argsort(-p, axis=1, kind="stable")[:, :6]
    assert np.array_equal(r["idx"], np.sort(order, axis=1))
    assert np.allclose(moe.sigmoid(z), scipy.special.expit(z), rtol=1e-15)


def test_closed_form_two_expert_softmax():
    z = np.array([[math.log(3.0), 0.0]])
    r = moe.route(z, "softmax", 1)
    assert r["idx"][0, 0] == 0 and abs(r["w"][0, 0] - 0.75) < 1e-15
    assert abs(r["gap"][0] - math.log(3.0)) < 1e-15


def test_batch_invariance_and_counts():
    rng = np.random.default_rng(4)
    u = rng.normal(size=(300, 48))
    wg = rng.normal(size=(24, 48)) / 7
    b = rng.uniform(-0.1, 0.1, 24)
    full = moe.route(moe.router_logits(u, wg), "sigmoid_bias", 5, b, True)
    part = moe.route(moe.router_logits(u[100:130], wg), "sigmoid_bias", 5, b, True)
    assert np.array_equal(full["idx"][100:130], part["idx"])
    c = moe.expert_counts(full["idx"], 24)
    assert c.sum() == 300 * 5
    assert np.all(np.diff(full["idx"], axis=1) > 0)     # distinct, ascending


def test_logit_offset_shifts_logits():
    rng = np.random.default_rng(5)
    u, wg = rng.normal(size=(4, 8)), rng.normal(size=(3, 8))
    off = np.array([0.0, -1.0, 2.0], dtype=np.float32)
    assert np.allclose(moe.router_logits(u, wg, off) - moe.router_logits(u, wg), off[None, :], atol=1e-15)
