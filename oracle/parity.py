"""Comparison of library outputs with the oracle's (test infrastructure only).

Rules (the tolerances the verify step is held to):
  * rows whose oracle decision margin is below BOUNDARY (a uniform within 1e-6 of an accept
    threshold or of a CDF break) are boundary rows: counted and checked only for validity,
    since fp32-vs-fp64 rounding may legitimately flip them.  Greedy rows have an infinite
    margin and are never exempt;
  * every other row: accept length and every emitted token bit-exact, unused slots -1;
  * emitted-token probabilities within 1e-5 relative of the oracle's, or 1e-30 absolute below
    1e-30 (fp32 underflow of very peaked rows); unused slots exactly 0.
"""
from __future__ import annotations

import numpy as np

BOUNDARY = 1e-6
PROB_RTOL = 1e-5
PROB_ATOL_FLOOR = 1e-30


def compare(inp, ref, acc, tok, prb=None, *, max_details: int = 10) -> dict:
    """Compare device outputs (numpy) with an OracleOut for the same rows; return a report."""
    acc = np.asarray(acc)
    tok = np.asarray(tok)
    B = len(ref.accept_len)
    kb = inp.draft_counts() if len(inp.draft_counts()) == B else None
    boundary = ref.margin < BOUNDARY
    rep = dict(rows=B, boundary=int(boundary.sum()), boundary_differs=0, mismatch=0, prob_mismatch=0,
               invalid=int((ref.accept_len < 0).sum()), max_prob_rel=0.0, details=[])
    for b in range(B):
        A = int(acc[b])
        if boundary[b]:
            ok = -1 <= A and (kb is None or A <= kb[b]) and (A < 0 or (tok[b, :A + 1] >= 0).all())
            if not ok:
                rep["mismatch"] += 1
                if len(rep["details"]) < max_details:
                    rep["details"].append(("boundary-invalid", b, A))
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
