"""Seeded synthetic token histories for the n-gram drafter and the post-verify commit step.

Like ``inputs.py`` this module only draws inputs; it holds none of the drafter's matching nor
the commit arithmetic.  Both the CPU oracle and the HIP path consume the arrays it returns.

A history is built the way the pages describe text that an n-gram drafter can exploit: output
that repeats its input ("What proposes the tokens" in "ch15 · Speculative Decoding",
snowch.github.io, and its measurement on a corpus that repeats; the prompt-lookup paragraph in
"Decodificação especulativa explicada", gsantana.dev).  Each history is a run of segments; a
segment is either fresh tokens drawn uniformly from the vocabulary or a copy of an earlier span
of the same history (copied token by token, so a copy may overlap itself and make runs).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

PAD_TOKEN = -7  # history slots at or past a sequence's length hold this (never a token id)


@dataclass
class Histories:
    """Token histories, host side.  tokens [B, capacity] int32, lengths [B] int32."""
    tokens: np.ndarray
    lengths: np.ndarray
    vocab: int
    name: str = "custom"
    meta: dict = field(default_factory=dict)

    @property
    def B(self) -> int:
        return self.tokens.shape[0]

    @property
    def capacity(self) -> int:
        return self.tokens.shape[1]


def _streams(seed: int, n: int = 4):
    return [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(n)]


def make_histories(B: int, capacity: int, V: int, *, seed: int,
                   len_range: tuple[int, int] | None = None, copy_frac: float = 0.5,
                   seg_range: tuple[int, int] = (8, 64), edge_cases: bool = False,
                   name: str = "custom") -> Histories:
    """B histories of lengths ~ U{len_range} (default: capacity // 2 .. capacity).

    Segments have lengths ~ U{seg_range}; each is a copy of a uniformly chosen earlier span with
    probability ``copy_frac`` (once the history is non-empty), else fresh ids ~ U{0..V-1}.  Slots
    past a history's length hold PAD_TOKEN.  With ``edge_cases`` the first sequences are replaced
    by degenerate histories: empty, one token, two equal tokens, one repeated token filling the
    capacity, and all-distinct tokens (nothing repeats).
    """
    rl, rs, rc, rt = _streams(seed)
    lo, hi = len_range if len_range is not None else (capacity // 2, capacity)
    lo, hi = max(0, min(lo, capacity)), max(0, min(hi, capacity))
    tokens = np.full((B, capacity), PAD_TOKEN, dtype=np.int32)
    lengths = rl.integers(lo, hi + 1, size=B).astype(np.int32)
    for b in range(B):
        L = int(lengths[b])
        h = np.empty(L, dtype=np.int64)
        n = 0
        while n < L:
            seg = int(rs.integers(seg_range[0], seg_range[1] + 1))
            seg = min(seg, L - n)
            if n > 0 and rc.random() < copy_frac:
                src = int(rc.integers(0, n))
                if src + seg <= n:
                    h[n:n + seg] = h[src:src + seg]
                else:
                    for j in range(seg):          # token by token: an overlapping copy repeats
                        h[n + j] = h[src + j]
            else:
                h[n:n + seg] = rt.integers(0, V, size=seg)
            n += seg
        tokens[b, :L] = h
    if edge_cases:
        cases = []
        cases.append(np.zeros(0, dtype=np.int64))
        cases.append(np.array([min(5, V - 1)]))
        cases.append(np.array([min(3, V - 1)] * 2))
        cases.append(np.full(capacity, min(1, V - 1)))
        cases.append(np.arange(min(capacity, V)) % V)
        for b, h in enumerate(cases[:B]):
            tokens[b] = PAD_TOKEN
            tokens[b, :len(h)] = h
            lengths[b] = len(h)
    return Histories(tokens, lengths, V, name=name,
                     meta=dict(seed=seed, copy_frac=copy_frac, seg_range=seg_range))


def ngram_workload(B: int = 512, capacity: int = 8192, V: int = 128256, seed: int = 6) -> Histories:
    """Drafting workload: 512 histories of 4096-8192 tokens over a 128256-token vocabulary, half
    of the segments copied from earlier in the same history (the ragged batch's n-gram rows)."""
    return make_histories(B, capacity, V, seed=seed, name="ngram_histories")


def ngram_long_workload(B: int = 256, capacity: int = 65536, V: int = 128256,
                        seed: int = 7) -> Histories:
    """Long histories: 256 histories of 32768-65536 tokens (the same copy structure), a size at
    which the drafter's pass over the history is bandwidth-bound rather than latency-bound."""
    return make_histories(B, capacity, V, seed=seed, name="ngram_long_histories")
