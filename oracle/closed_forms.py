"""Closed forms of the acceptance process, used by the statistical tests.

TEST INFRASTRUCTURE ONLY (same import rule as ``oracle.verify``).

  * acceptance rate of one position: alpha = sum_x min(p(x), q(x)) = 1 - TV(p, q)
    ("A regra de amostragem por rejeição" in "Decodificação especulativa
    explicada", gsantana.dev);
  * expected tokens per target pass with a constant alpha:
    (1 - alpha^(k+1)) / (1 - alpha), saturating at 1 / (1 - alpha), and the
    speedup (1 - alpha^(k+1)) / ((1 - alpha)(k c + 1)) with c the relative draft
    cost ("Quanto mais rápido: a matemática", same page; "La matemática que
    importa: techo y speedup" in the blog.lo0.es page gives the same ratio);
  * with position-dependent acceptance rates and independent accept tests, the
    accepted length A of one round obeys P(A >= a) = prod_{i<a} alpha_i.
"""
from __future__ import annotations

import numpy as np


def acceptance_rate(p: np.ndarray, q: np.ndarray) -> float:
    """alpha = sum_x min(p(x), q(x))."""
    return float(np.minimum(np.asarray(p, np.float64), np.asarray(q, np.float64)).sum())


def expected_tokens(alpha: float, k: int) -> float:
    """E[tokens per target pass] = (1 - alpha^(k+1)) / (1 - alpha)  (k+1 when alpha = 1)."""
    if alpha == 1.0:
        return float(k + 1)
    return (1.0 - alpha ** (k + 1)) / (1.0 - alpha)


def speedup(alpha: float, k: int, c: float) -> float:
    """Expected speedup over plain decoding with draft cost c per draft step."""
    return expected_tokens(alpha, k) / (k * c + 1.0)


def accept_length_law(alphas) -> np.ndarray:
    """P(A = a) for a = 0..k given per-position acceptance rates alpha_0..alpha_{k-1}."""
    alphas = [float(a) for a in alphas]
    k = len(alphas)
    law = np.empty(k + 1)
    survive = 1.0
    for a in range(k):
        law[a] = survive * (1.0 - alphas[a])
        survive *= alphas[a]
    law[k] = survive
    return law


def expected_tokens_from_law(alphas) -> float:
    """E[A + 1] = sum_{a=0}^{k} prod_{i<a} alpha_i."""
    law = accept_length_law(alphas)
    return float(np.dot(np.arange(1, len(law) + 1), law))
