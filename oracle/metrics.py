"""Closed forms the pages give, fp64.  Test infrastructure.

CS349E Lecture 6, "Optimizing Autoregressive Decode":
  * section 7.2: acceptance probability of one position
        beta = sum_x min(p(x), q(x)) = 1 - TV(p, q),  TV = 1/2 sum |p - q|;
  * section 8.1, eq. (1): expected tokens per round with i.i.d. acceptance
        E = (1 - alpha^(gamma+1)) / (1 - alpha);
  * section 8.2, Theorem 3.8: wall-time speedup E / (gamma c + 1);
  * section 8.4, Theorem 3.11: compute increase (gamma c_hat + gamma + 1) / E;
  * Exercise 9: node count and tau of a greedy tree under independence.
The speculative-decoding verify-cost page (ariaki.me), section 2: speedup
(1 + p) T_decode / (T_verify + T_draft) and its break-even line.
The DeepSeek-V4 speculative performance page (akiyangdev), section on accept
metrics: strict accept rate = correct drafts / (verify count x (draft tokens
per verify - 1)), bonus excluded; accept length = completion tokens / verify
count, bonus included.
"""
from __future__ import annotations

import numpy as np


def beta(p, q) -> float:
    return float(np.minimum(np.asarray(p, np.float64), np.asarray(q, np.float64)).sum())


def total_variation(p, q) -> float:
    return float(0.5 * np.abs(np.asarray(p, np.float64) - np.asarray(q, np.float64)).sum())


def expected_tokens(alpha: float, gamma: int) -> float:
    if alpha == 1.0:
        return float(gamma + 1)
    return (1.0 - alpha ** (gamma + 1)) / (1.0 - alpha)


def walltime_speedup(alpha: float, gamma: int, c: float) -> float:
    return expected_tokens(alpha, gamma) / (gamma * c + 1.0)


def compute_increase(alpha: float, gamma: int, c_hat: float) -> float:
    return (gamma * c_hat + gamma + 1.0) / expected_tokens(alpha, gamma)


def strict_accept_rate(num_correct_drafts: int, verify_ct: int, num_draft_tokens: int) -> float:
    return num_correct_drafts / (verify_ct * (num_draft_tokens - 1))


def accept_length(completion_tokens: int, verify_ct: int) -> float:
    return completion_tokens / verify_ct


def division_speedup(p: float, t_decode: float, t_verify: float, t_draft: float) -> float:
    """Tokens per ms of a one-draft round over tokens per ms of plain decode."""
    return (1.0 + p) * t_decode / (t_verify + t_draft)


def break_even_verify(p: float, t_decode: float, t_draft: float) -> float:
    return (1.0 + p) * t_decode - t_draft


def tree_draft_nodes(branching) -> int:
    total, width = 0, 1
    for k in branching:
        width *= k
        total += width
    return total


def tree_tau_independent(branching, topk_hit) -> float:
    """Greedy tree: depth d continues when the right token is among the top k_d
    drafts; topk_hit[k] = P(right token within the top k)."""
    tau, prod = 1.0, 1.0
    for k in branching:
        prod *= topk_hit[k]
        tau += prod
    return tau
