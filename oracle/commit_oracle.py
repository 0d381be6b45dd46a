"""CPU oracle of the post-verify commit: KV-cache rollback and ragged compaction.

TEST INFRASTRUCTURE ONLY (see the package header).  Plain Python written from the pages.

Sources (cited by title and section):
  [P1] "Decodificação especulativa explicada: rascunhe barato, verifique numa
       passada" (gsantana.dev) -- section "O ciclo de rascunho e verificação": the target
       added cache entries for the k drafted positions, so the entries past the first
       rejection are dropped by truncating the cache or moving a pointer back, and the
       drafter's own cache is rolled back the same way; a round yields between 1 and k+1
       tokens.
  [P2] "ch15 · Speculative Decoding" (snowch.github.io) -- section "The build": a rejected
       proposal has to be rolled back out of the cache.
  [P3] "Speculative decoding: el secretario que adelanta lo que va a decir el jefe"
       (blog.lo0.es) -- section "Pitfalls operacionales", continuous batching: each request
       accepts a different number of tokens per iteration (nested raggedness).

Readings where the pages leave a step open:
  C1  lengths are counts.  Before the round sequence b has L = seq_len[b] tokens; the round
      emits A + 1 tokens (A = accept_len[b] accepted drafts, then the correction or bonus),
      which are appended to its history: new seq_len = L + A + 1.
  C2  a cache holds entries for a prefix of the sequence.  After the round only the entries
      of the L + A tokens before the emitted correction / bonus can be kept (the first L
      tokens and the A accepted drafts); every entry past that point is dropped by moving the
      cache length back: kv' = min(kv, L + A), for the target and the drafter alike.
  C3  the emitted tokens of all sequences are also packed, in sequence order, into one
      ragged stream with offsets = exclusive prefix sums of the per-sequence counts
      (offsets[B] = total), the shape a serving loop hands to detokenisation.
  C4  a sequence with accept_len outside [0, K] (an invalid verify row), a negative length,
      or a history that would overflow its capacity commits nothing: 0 tokens, lengths
      unchanged.
"""
from __future__ import annotations

import numpy as np


def commit(accept_len, out_tokens, tokens, seq_len, capacity, target_kv=None, draft_kv=None):
    """Returns (tokens', seq_len', target_kv', draft_kv', emitted, offsets, packed).

    ``tokens`` [B, capacity] is the history (or None); the inputs are not modified.
    """
    accept_len = np.asarray(accept_len)
    out_tokens = np.asarray(out_tokens)
    B, K1 = out_tokens.shape
    K = K1 - 1
    tok = None if tokens is None else np.array(tokens, copy=True)
    sl = np.array(seq_len, copy=True)
    tkv = None if target_kv is None else np.array(target_kv, copy=True)
    dkv = None if draft_kv is None else np.array(draft_kv, copy=True)
    emitted = np.zeros(B, dtype=np.int64)
    for b in range(B):
        A, L = int(accept_len[b]), int(seq_len[b])
        if A < 0 or A > K or L < 0 or L + A + 1 > capacity:
            continue                                   # C4
        emitted[b] = A + 1                             # C1
        if tok is not None:
            tok[b, L:L + A + 1] = out_tokens[b, :A + 1]
        sl[b] = L + A + 1
        if tkv is not None:
            tkv[b] = min(int(tkv[b]), L + A)           # C2
        if dkv is not None:
            dkv[b] = min(int(dkv[b]), L + A)
    offsets = np.zeros(B + 1, dtype=np.int64)          # C3
    packed = []
    for b in range(B):
        offsets[b + 1] = offsets[b] + emitted[b]
        packed.extend(int(t) for t in out_tokens[b, :emitted[b]])
    return tok, sl, tkv, dkv, emitted, offsets, np.array(packed, dtype=np.int64)
