"""CPU oracle of the "sample the target and match" verify mode.

TEST INFRASTRUCTURE ONLY (see the package header).  Plain numpy fp64.

Source: "Decodificação especulativa explicada: rascunhe barato, verifique numa passada"
(gsantana.dev), section "A regra de amostragem por rejeição", the paragraph after the biased
fallback: a simpler exact scheme draws a token from the target at each position and keeps the
draft token only while the two agree.  Every emitted token is a draw from p, so it is lossless,
but its acceptance rate is the sum of p(x) q(x), below the rejection rule's sum of
min(p(x), q(x)).

Readings where the pages leave a step open:
  M1  position i < k_b draws y_i from p_i with the uniform u[b, i]; the bonus position k_b
      draws with u[b, K] (the verify step's column layout, reading R3).  Draws use the verify
      step's inverse CDF (R5) on p_i.
  M2  drafts are kept left to right while y_i == x_i; at the first i with y_i != x_i the round
      emits y_i and ends (A = i); if all k_b agree the bonus y_{k_b} is emitted (A = k_b).
  M3  q is never read (x_i is assumed to have been drawn from the drafter's q); one-hot rows
      are treated like any other row.
  M4  greedy rows (T = 0) are the verify step's greedy rows (a point-mass p draws its argmax).
  M5  invalid rows as the verify step's R10 without the q conditions.
  M6  the decision margin is the smallest distance (normalised) of any evaluated draw to a CDF
      break; rows within 1e-6 are exempt from exact comparison.
"""
from __future__ import annotations

import math

import numpy as np

from .verify_oracle import (TEMPERATURE_MIN, OracleOut, inverse_cdf, logit_row, target_probs,
                            verify_row)


def match_row(inp, b: int, *, resample_bug: bool = False):
    """One sequence.  Returns (A, tokens[K+1], probs[K+1], margin).

    ``resample_bug`` (test-only negative control): on a mismatch, emit a fresh draw from p with
    u[b, K] instead of y_i."""
    K, V = inp.K, inp.V
    k = K if inp.num_draft is None else int(inp.num_draft[b])
    T = float(inp.temperature[b])
    invalid = (-1, [-1] * (K + 1), [0.0] * (K + 1), math.inf)
    if not (0 <= k <= K):
        return invalid
    if T == 0.0:                                      # M4
        return verify_row(inp.logits, inp.logits_dtype, None, None, inp.proposed, inp.num_draft,
                          inp.temperature, inp.uniforms, b)
    if not (math.isfinite(T) and T >= TEMPERATURE_MIN):
        return invalid
    rows = [logit_row(inp.logits, inp.logits_dtype, b, i) for i in range(k + 1)]
    for z in rows:
        if np.isnan(z).any() or np.isposinf(z).any() or not (z.max() > -math.inf):
            return invalid
    xs = [int(inp.proposed[b, i]) for i in range(k)]
    if any(not (0 <= x < V) for x in xs):
        return invalid
    us = [float(inp.uniforms[b, i]) for i in range(k)] + [float(inp.uniforms[b, K])]
    if any(not (0.0 <= u < 1.0) for u in us):
        return invalid
    tokens, probs = [-1] * (K + 1), [0.0] * (K + 1)
    margin = math.inf
    for i in range(k + 1):
        p = target_probs(rows[i], T)
        y, m = inverse_cdf(p, us[i])                  # M1
        margin = min(margin, m)
        if i < k and y == xs[i]:                      # M2: keep the draft
            tokens[i], probs[i] = y, float(p[y])
            continue
        if i < k and resample_bug:
            y, m = inverse_cdf(p, us[k])
            margin = min(margin, m)
        tokens[i], probs[i] = y, float(p[y])
        return i, tokens, probs, margin
    raise AssertionError("unreachable")


def verify_match(inp, *, rows=None, resample_bug: bool = False) -> OracleOut:
    """The match-mode oracle over a ``VerifyInputs`` batch (or the listed sequences)."""
    idx = range(inp.B) if rows is None else [int(r) for r in rows]
    n, K = len(idx), inp.K
    acc = np.empty(n, dtype=np.int32)
    tok = np.empty((n, K + 1), dtype=np.int32)
    prb = np.empty((n, K + 1), dtype=np.float64)
    mar = np.empty(n, dtype=np.float64)
    for j, b in enumerate(idx):
        acc[j], tok[j], prb[j], mar[j] = match_row(inp, b, resample_bug=resample_bug)
    return OracleOut(acc, tok, prb, mar)
