"""Closed forms for how many tokens one verification pass yields.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Plain float64 Python.

Sources:
* "Let's start over, Misha: speculative decoding from draft to verification"
  (braintools.ru), section "How much does it give?": the constant-acceptance
  expected token count of Leviathan et al. and the speedup model with a draft
  pass costing a fraction ``c`` of a target pass.
* "Speculative decoding in production: comparing methods in the Wildberries
  shopping assistant" (kiosknews.app), section "A bit of theory", Statement 2:
  tokens per pass = 1 + E[A] = 1 + sum_k P(A >= k); and section "1. n-gram":
  tokens per step when only a share f of the steps carries a draft.
* Same Wildberries page, section "5. DFlash": with independent per-position
  acceptance probabilities the expected accepted prefix is the sum over k of
  the product of the first k probabilities.
"""
from __future__ import annotations

import numpy as np


def expected_tokens(alpha: float, K: int) -> float:
    """Expected tokens per target pass, constant acceptance ``alpha``, draft length ``K``.

    Geometric series 1 + alpha + ... + alpha**K = (1 - alpha**(K+1)) / (1 - alpha)
    ("How much does it give?", Leviathan et al.'s formula).
    """
    if alpha == 1.0:
        return float(K + 1)
    return (1.0 - alpha ** (K + 1)) / (1.0 - alpha)


def speedup(alpha: float, K: int, c: float) -> float:
    """Speedup when each of the K draft passes costs ``c`` target passes.

    Expected tokens divided by the cost of one cycle, K*c + 1 ("How much does it give?").
    """
    return expected_tokens(alpha, K) / (K * c + 1.0)


def best_draft_length(alpha: float, c: float, K_max: int = 15) -> tuple[int, float]:
    """Grid search of the draft length maximising :func:`speedup` over K = 1..K_max.

    The lowest K wins a tie.
    """
    best_k, best_s = 1, speedup(alpha, 1, c)
    for k in range(2, K_max + 1):
        s = speedup(alpha, k, c)
        if s > best_s:
            best_k, best_s = k, s
    return best_k, best_s


def tau_from_position_acceptance(a) -> float:
    """Statement 2: tau = 1 + sum_k P(A >= k), with a[k-1] = P(A >= k)."""
    return 1.0 + float(np.sum(np.asarray(a, dtype=np.float64)))


def conditional_acceptance(a) -> np.ndarray:
    """P(A >= k | A >= k-1) = a_k / a_{k-1} for k >= 2 (a_0 = 1 is not included)."""
    a = np.asarray(a, dtype=np.float64)
    return a[1:] / a[:-1]


def acceptance_rate(p, q) -> float:
    """Probability that the rejection rule accepts the drafted token: sum_v min(p_v, q_v).

    Summing min(1, p/q) * q over the draft's proposals gives sum_v min(p_v, q_v)
    (Wildberries page, "A bit of theory", proof of Statement 1).
    """
    return float(np.minimum(np.asarray(p, np.float64), np.asarray(q, np.float64)).sum())


def tau_closed_form(alphas) -> float:
    """Expected tokens per pass with independent per-position acceptance ``alphas``.

    1 + sum_{k=1..K} prod_{i<=k} alpha_i (Statement 2 with P(A >= k) = prod_{i<=k} alpha_i;
    the DFlash section's expected accepted prefix).  Positions are independent under
    the verification rule because every position draws its own draft token and coin.
    """
    al = np.asarray(alphas, dtype=np.float64)
    return 1.0 + float(np.cumprod(al).sum()) if al.size else 1.0


def tokens_per_step(f: float, tau_drafted: float) -> float:
    """Tokens per step when a draft exists on a share ``f`` of the steps.

    A step without a draft yields one token; a step with one yields ``tau_drafted``
    ("1. n-gram": the engine's tau counts only the steps that had a draft).
    """
    return 1.0 + f * (tau_drafted - 1.0)
