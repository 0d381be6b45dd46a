"""fp64 CPU oracle of the batched speculative-decoding verify step.

TEST INFRASTRUCTURE ONLY.  Plain, slow, obviously-correct numpy written from the
pages' definitions.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything here; the
library and its Python binding never do.  It shares no code with the HIP path.

Sources (web pages; cited by title and section):
  [P1] "Decodificação especulativa explicada: rascunhe barato, verifique numa
       passada" (gsantana.dev) -- sections "O ciclo de rascunho e verificação",
       "A regra de amostragem por rejeição", "Amostragem especulativa em numpy,
       com prova".
  [P2] "ch15 · Speculative Decoding" (snowch.github.io, LLM serving from
       scratch) -- section "Why the result is exactly the target model".
  [P3] "Speculative decoding: el secretario que adelanta lo que va a decir el
       jefe" (blog.lo0.es) -- sections "El mecanismo desnudo", "Por qué la
       calidad no se degrada (la prueba)".

What one sequence's round computes (all three pages agree on the rule):
  * the target gives k+1 next-token distributions p_0..p_k, one per drafted
    position plus one after the last draft [P1 draft-and-verify loop; P3 step 2];
  * drafts are judged left to right: draft x_i is accepted with probability
    min(1, p_i(x_i) / q_i(x_i)); the first rejection ends the round and a
    replacement is drawn from norm(max(0, p_i - q_i)) [P1 rejection rule,
    items 1-2; P2; P3 step 3];
  * if all k drafts survive, one bonus token is drawn from p_k [P1 item 3;
    P3 step 3];
  * greedy decoding is the degenerate case: p is a point mass on the target's
    argmax, so a draft survives iff it equals that argmax and the "residual"
    is the argmax itself [P1, paragraph after the proof; P2 greedy argument].

Readings where the pages leave a step open:
  R1  temperature: p_i = softmax(z_i / T) of the raw logit row; T = 0 means
      greedy.  Valid temperatures are 0 or finite T >= TEMPERATURE_MIN.
  R2  q is used exactly as supplied (never renormalised or tempered here).
  R3  the random stream is a uniforms array u[B, K+1]: u[b, i] (i < K) drives
      accept test i, u[b, K] drives the one correction-or-bonus draw.
  R4  accept iff u * q(x) < p(x): the page's strict ``u < min(1, p/q)``
      [P1 numpy listing] made total for q(x) = 0 (accept iff p(x) > 0).
  R5  sampling convention: inverse CDF over ascending token id on unnormalised
      weights, the first index whose running sum exceeds u times the total
      (the page's ``searchsorted(cumsum(w), u*sum, side="right")``), using the
      scan's own total.  Zero-mass tokens are never chosen.
  R6  if a rejection leaves a residual of zero total mass (only possible when q
      is not a distribution), the replacement is drawn from p_i itself.
  R7  greedy ties: the lowest index of the maximum.
  R8  greedy rows read neither q nor u.
  R9  one-hot (n-gram) rows: q_i = onehot(x_i), so accept iff u < p(x), and the
      residual is p_i with x_i removed.
  R10 invalid rows (reported as accept_len -1, tokens -1, probs 0): k_b outside
      [0, K]; temperature negative, NaN, infinite or in (0, TEMPERATURE_MIN);
      a used logit row (0..k_b) with a NaN or +inf entry, or with every entry
      -inf; a proposed id outside [0, V) in slots < k_b; for sampled rows a
      used uniform outside [0, 1); for sampled model-draft rows a gathered
      q_i(x_i) that is negative or not finite, or no draft tensor at all; and,
      at a model-draft rejection, any entry of the rejected slot's draft row
      q_i (the row the residual draw reads) that is negative or not finite.
      Draft rows the round never reads are never checked.
      -inf logits are zero-mass tokens.
  R11 k_b = 0 is allowed: one plain sample (or argmax) from row 0.
  R12 out_probs of a greedy row report softmax at T = 1 of the raw logits.
  R13 decision margin (used only to exempt floating-point boundary cases from
      exact comparison): the minimum over the row's evaluated accept tests of
      |u - p(x)/q(x)| (q(x) > 0), and over its sample of the distance of u to
      the nearest CDF break, in normalised CDF units.  Greedy rows: +inf.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

TEMPERATURE_MIN = 1e-6


@dataclass
class OracleOut:
    accept_len: np.ndarray   # [n] int32, A_b in [0, k_b] or -1 (invalid row)
    out_tokens: np.ndarray   # [n, K+1] int32, slots 0..A_b filled, the rest -1
    out_probs: np.ndarray    # [n, K+1] float64, target probability of each emitted token
    margin: np.ndarray       # [n] float64 decision margin (R13)


def logit_row(logits: np.ndarray, logits_dtype: str, b: int, i: int) -> np.ndarray:
    """Row (b, i) of the target logits as exact float64 (bf16 bits -> value by a 16-bit shift)."""
    row = logits[b, i]
    if logits_dtype == "bf16":
        with np.errstate(invalid="ignore"):      # signalling-NaN patterns widen to NaN
            return (row.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if logits_dtype in ("f32", "f64"):
        return row.astype(np.float64)
    raise ValueError(f"unknown logits dtype {logits_dtype!r}")


def target_probs(z: np.ndarray, T: float) -> np.ndarray:
    """p = softmax(z / T) in fp64 (reading R1); -inf logits get probability 0."""
    m = z.max()
    w = np.exp((z - m) / T)
    return w / w.sum()


def inverse_cdf(w: np.ndarray, u: float) -> tuple[int, float]:
    """Draw from unnormalised weights w with the uniform u (reading R5).

    Returns (token, margin): margin is the distance from u*total to the nearest break of the
    running sum, divided by the total."""
    c = np.cumsum(w)                     # sequential fp64 running sum, ascending token id
    total = c[-1]
    t = u * total
    y = int(np.searchsorted(c, t, side="right"))
    if y >= len(w):                      # rounding left t at the total: last positive weight
        y = int(np.flatnonzero(w > 0)[-1])
    lo = c[y - 1] if y > 0 else 0.0
    margin = min(t - lo, c[y] - t) / total
    return y, float(margin)


def _row_invalid(n_slots: int):
    return -1, [-1] * n_slots, [0.0] * n_slots, math.inf


def verify_row(logits, logits_dtype, draft_probs, draft_onehot, proposed, num_draft,
               temperature, uniforms, b: int, *, buggy: bool = False):
    """One sequence's verify round.  Returns (A, tokens[K+1], probs[K+1], margin)."""
    K = logits.shape[1] - 1
    V = logits.shape[2]
    k = K if num_draft is None else int(num_draft[b])
    T = float(temperature[b])
    if not (0 <= k <= K):
        return _row_invalid(K + 1)
    greedy = T == 0.0
    if not greedy and not (math.isfinite(T) and T >= TEMPERATURE_MIN):
        return _row_invalid(K + 1)

    # Every used target row is checked (R10), whether or not the scan reaches it.
    rows = [logit_row(logits, logits_dtype, b, i) for i in range(k + 1)]
    for z in rows:
        if np.isnan(z).any() or np.isposinf(z).any() or not (z.max() > -math.inf):
            return _row_invalid(K + 1)
    xs = [int(proposed[b, i]) for i in range(k)]
    if any(not (0 <= x < V) for x in xs):
        return _row_invalid(K + 1)

    tokens = [-1] * (K + 1)
    probs = [0.0] * (K + 1)

    if greedy:
        # Point-mass target: a draft survives iff it is the argmax; the replacement or bonus
        # is the argmax itself (R7 lowest index, R8, R12).
        for i in range(k + 1):
            z = rows[i]
            g = int(np.argmax(z))
            p1 = target_probs(z, 1.0)
            if i < k and xs[i] == g:
                tokens[i], probs[i] = xs[i], float(p1[xs[i]])
                continue
            tokens[i], probs[i] = g, float(p1[g])
            return i, tokens, probs, math.inf
        raise AssertionError("unreachable")

    us = [float(uniforms[b, i]) for i in range(k)]
    u_last = float(uniforms[b, K])
    if any(not (0.0 <= u < 1.0) for u in us + [u_last]):
        return _row_invalid(K + 1)
    onehot = draft_onehot is not None and int(draft_onehot[b]) != 0
    if not onehot and k > 0:
        if draft_probs is None:
            return _row_invalid(K + 1)
        qxs = [float(draft_probs[b, i, xs[i]]) for i in range(k)]
        if any(not (math.isfinite(q) and q >= 0.0) for q in qxs):
            return _row_invalid(K + 1)

    margin = math.inf
    for i in range(k):
        p = target_probs(rows[i], T)
        x = xs[i]
        if onehot:
            q = np.zeros(V)
            q[x] = 1.0
        else:
            q = draft_probs[b, i].astype(np.float64)
        px, qx, u = float(p[x]), float(q[x]), us[i]
        if qx > 0.0:
            margin = min(margin, abs(u - px / qx))
        # Accept with probability min(1, p/q) (R4).
        if u * qx < px:
            tokens[i], probs[i] = x, px
            continue
        # First rejection: replacement from norm(max(0, p - q)); the round ends.  The draft row
        # read here must be a vector of probabilities (R10).
        if not onehot and not bool(np.all(np.isfinite(q) & (q >= 0.0))):
            return _row_invalid(K + 1)
        r = p.copy() if buggy else np.maximum(p - q, 0.0)
        if not r.sum() > 0.0:            # R6
            r = p
        y, m_s = inverse_cdf(r, u_last)
        tokens[i], probs[i] = y, float(p[y])
        return i, tokens, probs, min(margin, m_s)

    # All k drafts survived: bonus token from the extra target row.
    p = target_probs(rows[k], T)
    y, m_s = inverse_cdf(p, u_last)
    tokens[k], probs[k] = y, float(p[y])
    return k, tokens, probs, min(margin, m_s)


def verify(inp, *, rows=None, buggy: bool = False) -> OracleOut:
    """Run the oracle over a ``VerifyInputs`` batch (or the sequences listed in ``rows``).

    ``buggy=True`` is a test-only negative control: on rejection it redraws from p instead of
    the residual (the mistake [P1] and [P2] warn about)."""
    idx = range(inp.B) if rows is None else [int(r) for r in rows]
    n = len(idx)
    K = inp.K
    acc = np.empty(n, dtype=np.int32)
    tok = np.empty((n, K + 1), dtype=np.int32)
    prb = np.empty((n, K + 1), dtype=np.float64)
    mar = np.empty(n, dtype=np.float64)
    for j, b in enumerate(idx):
        a, t, p, m = verify_row(inp.logits, inp.logits_dtype, inp.draft_probs, inp.draft_onehot,
                                inp.proposed, inp.num_draft, inp.temperature, inp.uniforms, b,
                                buggy=buggy)
        acc[j], tok[j], prb[j], mar[j] = a, t, p, m
    return OracleOut(acc, tok, prb, mar)
