"""Load-balance statistics of one routed batch, float64 (test infrastructure: only tests/, the smoke check
and the benchmark's CPU baseline use this package).

[TR] §1.2 gives the expert-level balance loss L_ExpBal = alpha_1 * sum_i f_i * P_i, with f_i the fraction
of tokens that selected expert i and P_i the average routing probability of expert i; [TR] §2.3 gives
alpha_1 = 0.003 (V2). [TR] §3.3 and [YJ] §4.3 add, for V3, a sequence-wise balance loss with a very
small weight (alpha = 0.0001) whose formula is not printed.

Readings taken here (repeated where used):
* f_i = (tokens whose top-K contains i) / T. The pages define f_i as a share of the tokens; no normalisation by
  E/K is printed, so none is applied (sum_i f_i = K).
* P_i = (1/T) sum_t s_{i,t}, the routing probability over all routed experts: the softmax of the logits
  in softmax mode; in sigmoid mode the affinities sigmoid(z) normalised over all routed experts (the
  selection bias is not part of it, as it only steers selection).
* Sequence-wise loss: the same statistic computed over each sequence of seq_len consecutive tokens
  and averaged over the B = T / seq_len sequences: alpha * (1/B) sum_b sum_i f_i^b P_i^b.
"""
from __future__ import annotations

import numpy as np

from . import moe


def routing_probabilities(z, gate: str) -> np.ndarray:
    """s_{i,t} over all routed experts: softmax(z) ([TR] §2.3), or sigmoid(z) / sum_j sigmoid(z_j)."""
    if gate == "softmax":
        return moe.softmax(z)
    s = moe.sigmoid(z)
    return s / s.sum(axis=1, keepdims=True)


def balance_stats(z, idx, gate: str, E: int):
    """(f, P) of [TR] §1.2 for the tokens of z / idx: f_i = count_i / T, P_i = mean_t s_{i,t}."""
    T = np.asarray(z).shape[0]
    f = moe.expert_counts(idx, E).astype(np.float64) / T
    P = routing_probabilities(z, gate).mean(axis=0)
    return f, P


def expert_balance_loss(f, P, alpha: float) -> float:
    """L_ExpBal = alpha * sum_i f_i P_i ([TR] §1.2)."""
    return float(alpha * np.dot(np.asarray(f, dtype=np.float64), np.asarray(P, dtype=np.float64)))


def sequence_balance_loss(z, idx, gate: str, E: int, seq_len: int, alpha: float) -> float:
    """alpha * mean over sequences b of sum_i f_i^b P_i^b (reading of [TR] §3.3; see the header)."""
    z = np.asarray(z)
    T = z.shape[0]
    if seq_len <= 0 or T % seq_len:
        raise ValueError("T must be a positive multiple of seq_len")
    terms = []
    for b in range(T // seq_len):
        sl = slice(b * seq_len, (b + 1) * seq_len)
        f, P = balance_stats(z[sl], np.asarray(idx)[sl], gate, E)
        terms.append(float(np.dot(f, P)))
    return float(alpha * np.mean(terms))
