"""Comparison of library outputs with the oracle's (test infrastructure only).

Rules (the tolerances the verify step is held to):
  * rows whose oracle decision margin is below BOUNDARY (a uniform within 1e-6 of an accept
    threshold or of a CDF break) are boundary rows: fp32-vs-fp64 rounding may legitimately flip
    them, so they are exempt from equality with the oracle, but they must still be a valid round
    of the rule ("Decodificação especulativa explicada", section "A regra de amostragem por
    rejeição"): a valid row stays valid (0 <= A <= k_b), the accepted slots hold the drafts, the
    emitted token is an id of the vocabulary with positive mass in the distribution it was drawn
    from (the residual max(0, p - q) at a rejection, p for the bonus), the later slots are -1, and
    every emitted probability is the target probability of the emitted token.  Greedy and
    invalid rows have an infinite margin and are never exempt;
  * every other row: accept length and every emitted token bit-exact, unused slots -1;
  * emitted-token probabilities within 1e-5 relative of the exact value, or 1e-30 absolute below
    1e-30 (fp32 underflow of very peaked rows); unused slots exactly 0.

``expected_boundary`` estimates how many boundary rows a batch should have (the measure of the
uniforms that fall within BOUNDARY of the thresholds a row evaluates), so that tests can bound
the exemption by what chance explains instead of a fixed fraction.
"""
from __future__ import annotations

import math

import numpy as np

from .verify_oracle import logit_row, target_probs

BOUNDARY = 1e-6
PROB_RTOL = 1e-5
PROB_ATOL_FLOOR = 1e-30


def _prob_ok(got: float, want: float) -> bool:
    tol = PROB_RTOL * want if want >= PROB_ATOL_FLOOR else PROB_ATOL_FLOOR
    return abs(got - want) <= tol


def _draft_row(inp, b: int, i: int, V: int) -> np.ndarray:
    """The drafter distribution q_i of sequence b as fp64 (one-hot rows: onehot(x_i))."""
    if inp.draft_onehot is not None and int(inp.draft_onehot[b]) != 0:
        q = np.zeros(V)
        q[int(inp.proposed[b, i])] = 1.0
        return q
    return inp.draft_probs[b, i].astype(np.float64)


def boundary_problems(inp, b: int, A: int, tok, prb=None, mode: str = "reject") -> list[str]:
    """Every way the device's round (A, tok, prb) of a sampled, valid sequence b breaks the rule's
    invariants (empty if it is a valid round).  Used for boundary rows, whose exact tokens may
    differ from the oracle's.  ``mode="match"``: the sample-and-match rule, whose emitted token
    is a draw from p that differs from the draft at a mismatch."""
    K, V = inp.K, inp.V
    kb = K if inp.num_draft is None else int(inp.num_draft[b])
    T = float(inp.temperature[b])
    tok = np.asarray(tok)
    out = []
    if not (0 <= A <= kb):
        return [f"accept length {A} outside [0, {kb}] for a valid row"]
    if not np.array_equal(tok[:A], inp.proposed[b, :A]):
        out.append("accepted slots are not the drafts")
    if (tok[A + 1:] != -1).any():
        out.append("slots after the emitted token are not -1")
    y = int(tok[A])
    if not (0 <= y < V):
        return out + [f"emitted token {y} outside [0, {V})"]
    p = target_probs(logit_row(inp.logits, inp.logits_dtype, b, A), T)
    if mode == "match":
        if not p[y] > 0.0:
            out.append(f"emitted token {y} has no target mass")
        if A < kb and y == int(inp.proposed[b, A]):
            out.append("mismatch slot emits the draft itself")
    elif A < kb:
        q = _draft_row(inp, b, A, V)
        r = np.maximum(p - q, 0.0)
        if r.sum() > 0.0:
            # The residual at y must be positive, up to the rounding of a near-tie p ~ q.
            if not (r[y] > 0.0 or abs(p[y] - q[y]) <= 1e-6 * max(p[y], q[y])):
                out.append(f"correction {y} has no residual mass (p={p[y]:.3g}, q={q[y]:.3g})")
        elif not p[y] > 0.0:
            out.append(f"fallback draw {y} has no target mass")
    elif not p[y] > 0.0:
        out.append(f"bonus token {y} has no target mass")
    if prb is not None:
        prb = np.asarray(prb, dtype=np.float64)
        for i in range(A + 1):
            want = float(target_probs(logit_row(inp.logits, inp.logits_dtype, b, i), T)[tok[i]])
            if not _prob_ok(float(prb[i]), want):
                out.append(f"probability of slot {i}: {prb[i]:.9g}, exact {want:.9g}")
        if (prb[A + 1:] != 0).any():
            out.append("unused slots have non-zero probabilities")
    return out


def _near(x: float) -> float:
    """Measure of the uniforms in [0, 1) within BOUNDARY of the threshold x."""
    return max(0.0, min(1.0, x + BOUNDARY) - max(0.0, x - BOUNDARY))


def _near_breaks(w: np.ndarray) -> float:
    """Measure of the uniforms in [0, 1) within BOUNDARY of a break of the running sum of w."""
    c = np.cumsum(w)
    b = c[w > 0] / c[-1]
    lo = np.maximum(b - BOUNDARY, 0.0)
    hi = np.minimum(b + BOUNDARY, 1.0)
    # Union of the intervals (sorted, since the breaks ascend).
    total, end = 0.0, 0.0
    for l, h in zip(lo, hi):
        l = max(l, end)
        if h > l:
            total += h - l
            end = h
    return total


def boundary_probability(inp, b: int, A: int, mode: str = "reject") -> float:
    """Union bound on the chance that the decisions the oracle evaluated for sequence b (its
    accept tests up to A and its one draw; in match mode its draws at slots 0..A) have a uniform
    within BOUNDARY of their thresholds."""
    K, V = inp.K, inp.V
    kb = K if inp.num_draft is None else int(inp.num_draft[b])
    T = float(inp.temperature[b])
    if A < 0 or T == 0.0:
        return 0.0
    total = 0.0
    rows = {}

    def p_of(i):
        if i not in rows:
            rows[i] = target_probs(logit_row(inp.logits, inp.logits_dtype, b, i), T)
        return rows[i]
    if mode == "match":
        return float(sum(_near_breaks(p_of(i)) for i in range(A + 1)))
    for i in range(min(A + 1, kb)):
        x = int(inp.proposed[b, i])
        qx = float(_draft_row(inp, b, i, V)[x])
        if qx > 0.0:
            total += _near(float(p_of(i)[x]) / qx)
    if A < kb:
        r = np.maximum(p_of(A) - _draft_row(inp, b, A, V), 0.0)
        w = r if r.sum() > 0.0 else p_of(A)
    else:
        w = p_of(kb)
    return total + _near_breaks(w)


def expected_boundary(inp, ref, rows=None, mode: str = "reject") -> float:
    """Expected number of boundary rows of a batch (sum of boundary_probability over its rows,
    along the oracle's own path)."""
    idx = range(inp.B) if rows is None else rows
    return float(sum(boundary_probability(inp, int(b), int(ref.accept_len[j]), mode)
                     for j, b in enumerate(idx)))


def boundary_limit(expected: float) -> int:
    """Largest boundary count the tests accept given its expectation: a Poisson tail bound
    (mean + 5 standard deviations + 3)."""
    return int(math.floor(expected + 5.0 * math.sqrt(expected) + 3.0))


def compare(inp, ref, acc, tok, prb=None, *, mode: str = "reject", max_details: int = 10) -> dict:
    """Compare device outputs (numpy) with an OracleOut for the same rows; return a report.
    ``mode``: "reject" (the rejection rule) or "match" (sample-and-match), for the invariants of
    boundary rows."""
    acc = np.asarray(acc)
    tok = np.asarray(tok)
    B = len(ref.accept_len)
    boundary = ref.margin < BOUNDARY
    rep = dict(rows=B, boundary=int(boundary.sum()), boundary_differs=0, mismatch=0, prob_mismatch=0,
               invalid=int((ref.accept_len < 0).sum()), max_prob_rel=0.0, details=[])
    for b in range(B):
        A = int(acc[b])
        if boundary[b]:
            problems = boundary_problems(inp, b, A, tok[b], None if prb is None else prb[b], mode)
            if problems:
                rep["mismatch"] += 1
                if len(rep["details"]) < max_details:
                    rep["details"].append(("boundary-invalid", b, A, problems))
            elif A != int(ref.accept_len[b]) or not np.array_equal(tok[b], ref.out_tokens[b]):
                rep["boundary_differs"] += 1
            continue
        if A != int(ref.accept_len[b]) or not np.array_equal(tok[b], ref.out_tokens[b]):
            rep["mismatch"] += 1
            if len(rep["details"]) < max_details:
                rep["details"].append(("tokens", b, A, int(ref.accept_len[b]), tok[b].tolist(),
                                       ref.out_tokens[b].tolist(), float(ref.margin[b])))
            continue
        if prb is not None:
            o = ref.out_probs[b]
            g = np.asarray(prb[b], dtype=np.float64)
            used = ref.out_tokens[b] >= 0
            tol = np.where(o >= PROB_ATOL_FLOOR, PROB_RTOL * o, PROB_ATOL_FLOOR)
            bad = (np.abs(g - o) > tol) | (~used & (g != 0))
            rel = np.abs(g - o)[used & (o > 0)] / o[used & (o > 0)]
            if rel.size:
                rep["max_prob_rel"] = max(rep["max_prob_rel"], float(rel.max()))
            if bad.any():
                rep["prob_mismatch"] += 1
                rep["mismatch"] += 1
                if len(rep["details"]) < max_details:
                    rep["details"].append(("probs", b, g.tolist(), o.tolist()))
    return rep
