"""Pins of the load-balance statistics oracle (oracle/balance.py) against closed forms, hand-derived
values and invariants ([TR] §1.2 expert-level balance loss; [TR] §3.3 sequence-wise loss)."""
import math

import numpy as np
import pytest

from oracle import balance as ob
from oracle import moe as omoe

A1 = 0.003      # [TR] §2.3 expert-level coefficient
ASEQ = 0.0001   # [TR] §3.3 sequence-wise weight


def _random_idx(rng, T, E, K):
    return np.stack([np.sort(rng.choice(E, K, replace=False)) for _ in range(T)]).astype(np.int32)


@pytest.mark.parametrize("gate", ["softmax", "sigmoid_bias"])
def test_uniform_logits_closed_form(gate):
    # equal logits: every expert has probability 1/E whatever the selection; sum_i f_i = K, so
    # L = alpha * K / E exactly
    rng = np.random.default_rng(0)
    T, E, K = 40, 12, 3
    idx = _random_idx(rng, T, E, K)
    f, P = ob.balance_stats(np.zeros((T, E)), idx, gate, E)
    assert np.allclose(P, 1.0 / E, rtol=0, atol=1e-15)
    assert math.isclose(f.sum(), K, rel_tol=0, abs_tol=1e-12)
    assert math.isclose(ob.expert_balance_loss(f, P, A1), A1 * K / E, rel_tol=1e-13)


def test_hand_derived_two_tokens_softmax():
    # token 0: logits (0, ln 2, 0) -> probabilities (1/4, 1/2, 1/4); selects expert 1
    # token 1: logits (ln 3, 0, 0) -> probabilities (3/5, 1/5, 1/5); selects expert 0
    z = np.array([[0.0, math.log(2.0), 0.0], [math.log(3.0), 0.0, 0.0]])
    idx = np.array([[1], [0]], dtype=np.int32)
    f, P = ob.balance_stats(z, idx, "softmax", 3)
    assert np.allclose(f, [0.5, 0.5, 0.0], rtol=0, atol=1e-15)
    assert np.allclose(P, [(0.25 + 0.6) / 2, (0.5 + 0.2) / 2, (0.25 + 0.2) / 2], rtol=0, atol=1e-15)
    # sum f P = 0.5 * 0.425 + 0.5 * 0.35
    assert math.isclose(ob.expert_balance_loss(f, P, A1), A1 * 0.3875, rel_tol=1e-13)


def test_hand_derived_sigmoid_normalised_over_all_experts():
    # sigmoid(0) = 1/2, sigmoid(ln 3) = 3/4: affinities (3/4, 1/2, 1/2) normalise to (3/7, 2/7, 2/7)
    z = np.array([[math.log(3.0), 0.0, 0.0]])
    idx = np.array([[0, 2]], dtype=np.int32)
    f, P = ob.balance_stats(z, idx, "sigmoid_bias", 3)
    assert np.allclose(P, [3 / 7, 2 / 7, 2 / 7], rtol=0, atol=1e-15)
    assert np.allclose(f, [1.0, 0.0, 1.0], rtol=0, atol=0)
    assert math.isclose(ob.expert_balance_loss(f, P, 1.0), 5 / 7, rel_tol=1e-13)


@pytest.mark.parametrize("gate", ["softmax", "sigmoid_bias"])
def test_probabilities_sum_to_one_and_counts_to_k(gate):
    rng = np.random.default_rng(1)
    T, E, K = 64, 20, 4
    z = rng.normal(0, 3, (T, E))
    idx = omoe.route(z, gate, K, np.zeros(E) if gate == "sigmoid_bias" else None, True)["idx"]
    f, P = ob.balance_stats(z, idx, gate, E)
    assert math.isclose(P.sum(), 1.0, rel_tol=1e-14)
    assert math.isclose(f.sum(), K, rel_tol=1e-14)
    assert np.all(f >= 0) and np.all(f <= 1)


def test_expert_relabelling_and_token_order_invariance():
    rng = np.random.default_rng(2)
    T, E, K = 48, 10, 3
    z = rng.normal(0, 2, (T, E))
    idx = omoe.route(z, "softmax", K)["idx"]
    f, P = ob.balance_stats(z, idx, "softmax", E)
    L = ob.expert_balance_loss(f, P, A1)
    perm = rng.permutation(E)               # expert i is renamed perm[i]
    z2 = np.empty_like(z)
    z2[:, perm] = z
    f2, P2 = ob.balance_stats(z2, perm[idx], "softmax", E)
    assert np.allclose(f2[perm], f, rtol=0, atol=1e-15) and np.allclose(P2[perm], P, rtol=1e-14, atol=0)
    assert math.isclose(ob.expert_balance_loss(f2, P2, A1), L, rel_tol=1e-13)
    tp = rng.permutation(T)
    assert math.isclose(ob.expert_balance_loss(*ob.balance_stats(z[tp], idx[tp], "softmax", E), A1), L,
                        rel_tol=1e-13)


def test_sequence_loss_reduces_to_batch_loss_for_one_sequence():
    rng = np.random.default_rng(3)
    T, E, K = 32, 8, 2
    z = rng.normal(0, 1, (T, E))
    idx = omoe.route(z, "sigmoid_bias", K, np.zeros(E), True)["idx"]
    f, P = ob.balance_stats(z, idx, "sigmoid_bias", E)
    assert math.isclose(ob.sequence_balance_loss(z, idx, "sigmoid_bias", E, T, ASEQ),
                        ob.expert_balance_loss(f, P, ASEQ), rel_tol=1e-13)


def test_sequence_loss_of_repeated_sequence_and_of_mixed_sequences():
    rng = np.random.default_rng(4)
    S, E, K = 16, 6, 2
    z = rng.normal(0, 1, (S, E))
    idx = omoe.route(z, "softmax", K)["idx"]
    one = ob.sequence_balance_loss(z, idx, "softmax", E, S, ASEQ)
    three = ob.sequence_balance_loss(np.vstack([z] * 3), np.vstack([idx] * 3), "softmax", E, S, ASEQ)
    assert math.isclose(one, three, rel_tol=1e-13)
    # two different sequences: the mean of their own losses, not the loss of their union
    z2 = rng.normal(0, 1, (S, E))
    idx2 = omoe.route(z2, "softmax", K)["idx"]
    two = ob.sequence_balance_loss(np.vstack([z, z2]), np.vstack([idx, idx2]), "softmax", E, S, ASEQ)
    own = 0.5 * (one + ob.sequence_balance_loss(z2, idx2, "softmax", E, S, ASEQ))
    assert math.isclose(two, own, rel_tol=1e-13)
    union = ob.expert_balance_loss(*ob.balance_stats(np.vstack([z, z2]), np.vstack([idx, idx2]), "softmax", E), ASEQ)
    assert not math.isclose(two, union, rel_tol=1e-6)


def test_concentrated_routing_is_the_maximum():
    # every token sends its single choice to expert 0, which holds almost all probability: f_0 = 1 and
    # P_0 -> 1, the largest value sum f P can take for K = 1; balanced routing gives K / E
    T, E = 30, 5
    z = np.zeros((T, E))
    z[:, 0] = 40.0
    idx = np.zeros((T, 1), dtype=np.int32)
    f, P = ob.balance_stats(z, idx, "softmax", E)
    assert math.isclose(ob.expert_balance_loss(f, P, 1.0), 1.0, rel_tol=1e-12)


def test_sequence_length_must_divide_the_batch():
    with pytest.raises(ValueError):
        ob.sequence_balance_loss(np.zeros((10, 4)), np.zeros((10, 1), dtype=np.int32), "softmax", 4, 3, ASEQ)
