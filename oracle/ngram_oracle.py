"""CPU oracle of the n-gram (prompt-lookup) drafter.

TEST INFRASTRUCTURE ONLY.  Plain Python written from the pages' description;
only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline leg
may import it.  It shares no code with the HIP path.

Sources (cited by title and section):
  [P1] "Decodificação especulativa explicada: rascunhe barato, verifique numa
       passada" (gsantana.dev) -- section "A família de rascunhos", paragraph on
       prompt lookup and n-gram drafting: no model; find the most recently
       generated tokens somewhere earlier in the context and propose what came
       after them there.
  [P2] "ch15 · Speculative Decoding" (snowch.github.io) -- section "What
       proposes the tokens": the n-gram drafter finds where the recent context
       appeared before and copies what followed; where nothing repeats it
       proposes nothing.
  [P3] "Speculative decoding: el secretario que adelanta lo que va a decir el
       jefe" (blog.lo0.es) -- section "Las cinco familias modernas", the
       closing paragraph on draft-free techniques: drafts proposed by
       longest-prefix match against the last generated tokens.

Readings where the pages leave a step open:
  N1  the "recent context" is the last n tokens of the sequence; n is tried
      from n_max down to n_min and the first n with an occurrence wins
      (longest match first, after P3's longest-prefix match).
  N2  an occurrence of that n-token suffix is any earlier start p with
      context[p:p+n] == suffix and p + n <= L - 1 (at least one token follows
      it; the suffix itself never matches; occurrences may overlap it).  Of
      several occurrences the earliest (smallest p) wins.
  N3  the proposal is what followed: context[p+n : p+n+K], cut at the end of
      the context, so 1 <= k_b <= K tokens.  No occurrence at any n: k_b = 0.
  N4  a length outside [0, capacity] is invalid: k_b = -1; unused proposal
      slots hold -1.
  N5  a one-hot drafter's q is onehot(x) (verify reading R9), so the verify
      step takes these rows with draft_onehot = 1.
"""
from __future__ import annotations

import numpy as np


def propose_one(ctx: np.ndarray, n_min: int, n_max: int, K: int):
    """Proposal for one sequence ``ctx`` (the valid tokens only): (tokens, n, p).

    Returns an empty list with n = p = -1 when nothing matches (N1-N3).
    """
    L = len(ctx)
    for n in range(min(n_max, L - 1), n_min - 1, -1):
        suffix = ctx[L - n:]
        for p in range(0, L - n):            # p + n <= L - 1
            if all(int(ctx[p + j]) == int(suffix[j]) for j in range(n)):
                start = p + n
                cnt = min(K, L - start)
                return [int(t) for t in ctx[start:start + cnt]], n, p
    return [], -1, -1


def ngram_propose(context: np.ndarray, lengths: np.ndarray, n_min: int, n_max: int, K: int):
    """Batched drafter: context [B, cap] int32, lengths [B] -> (proposed [B, K], num_draft [B]).

    Unused slots of ``proposed`` are -1; an invalid length gives num_draft -1 (N4).
    """
    context = np.asarray(context)
    B, cap = context.shape
    proposed = np.full((B, K), -1, dtype=np.int32)
    num_draft = np.zeros(B, dtype=np.int32)
    for b in range(B):
        L = int(lengths[b])
        if L < 0 or L > cap:
            num_draft[b] = -1
            continue
        toks, _, _ = propose_one(context[b, :L], n_min, n_max, K)
        num_draft[b] = len(toks)
        proposed[b, :len(toks)] = toks
    return proposed, num_draft
