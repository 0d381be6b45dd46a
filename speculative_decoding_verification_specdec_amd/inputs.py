"""Seeded synthetic inputs for the batched speculative-decoding verify step.

This module only *draws* inputs: target logit rows, the drafter's proposal
distributions and proposed ids, per-sequence temperatures, draft counts and the
uniform draws that stand in for the verifier's random-number stream.  It holds
none of the verify arithmetic (no target softmax, no accept test, no residual,
no inverse-CDF sampling); both the fp64 oracle and the HIP path consume the same
arrays from here and nothing else.

The drafter side is synthesised the way the pages describe a drafter: it
proposes each token from its own distribution q and records q
("O ciclo de rascunho e verificação" in "Decodificação especulativa explicada",
gsantana.dev; "What proposes the tokens" in "ch15 · Speculative Decoding",
snowch.github.io).  q here is softmax(draft logits) computed in fp64 and
rounded to fp32, and proposals are drawn from it with numpy's categorical
sampler.  An n-gram drafter has no distribution of its own; its rows carry a
one-hot flag (q(x) = 1) and proposals that either copy the target's top token
(a "hit") or are arbitrary ids.

Recipes (sizes and value distributions) follow the five workloads the library
is measured on; every stream is a numpy ``default_rng`` sub-stream spawned from
one seed in a fixed order, so a config is a pure function of (sizes, seed).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

BF16_NAN_BITS = np.uint16(0x7FC0)
PAD_ID_OFFSET = 12345          # padded proposal slots hold V + this (out of range)
PAD_UNIFORM = np.float32(7.0)  # padded uniform slots hold a value outside [0, 1)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even); return the bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    out = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    out[np.isnan(x)] = BF16_NAN_BITS
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class VerifyInputs:
    """One batch of verify-step inputs, host side, C-contiguous.

    logits       [B, K+1, V]  uint16 bf16 bit patterns (logits_dtype "bf16") or float32 ("f32")
    draft_probs  [B, K, V]    float32, or None when no row needs a model-draft q
    draft_onehot [B]          uint8, 1 = n-gram / one-hot drafter row; or None (no such rows)
    proposed     [B, K]       int32
    num_draft    [B]          int32 per-sequence draft count k_b in [0, K]; or None (all K)
    temperature  [B]          float32; 0 = greedy row
    uniforms     [B, K+1]     float32 in [0, 1): column i < K drives accept test i,
                              column K the single correction / bonus draw
    """

    logits: np.ndarray
    logits_dtype: str
    draft_probs: np.ndarray | None
    draft_onehot: np.ndarray | None
    proposed: np.ndarray
    num_draft: np.ndarray | None
    temperature: np.ndarray
    uniforms: np.ndarray
    name: str = "custom"
    meta: dict = field(default_factory=dict)

    @property
    def B(self) -> int:
        return int(self.logits.shape[0])

    @property
    def K(self) -> int:
        return int(self.logits.shape[1]) - 1

    @property
    def V(self) -> int:
        return int(self.logits.shape[2])

    def draft_counts(self) -> np.ndarray:
        if self.num_draft is None:
            return np.full(self.B, self.K, dtype=np.int64)
        return self.num_draft.astype(np.int64)

    def subset(self, rows) -> "VerifyInputs":
        """The same inputs restricted to the given sequence indices (copies)."""
        rows = np.asarray(rows, dtype=np.int64)
        pick = lambda a: None if a is None else np.ascontiguousarray(a[rows])
        return VerifyInputs(pick(self.logits), self.logits_dtype, pick(self.draft_probs),
                            pick(self.draft_onehot), pick(self.proposed), pick(self.num_draft),
                            pick(self.temperature), pick(self.uniforms),
                            name=f"{self.name}[subset]", meta=dict(self.meta))


def _streams(seed: int, n: int = 8):
    return [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(n)]


def _drafter_probs(draft_logits: np.ndarray, temp: float) -> tuple[np.ndarray, np.ndarray]:
    """The drafter's own distribution: softmax of its logits at its temperature.

    Returns (fp32 probabilities handed to the verifier, fp64 normalised copy used to draw
    proposals)."""
    a = draft_logits.astype(np.float64) / temp
    a -= a.max(axis=-1, keepdims=True)
    e = np.exp(a)
    q64 = e / e.sum(axis=-1, keepdims=True)
    q32 = q64.astype(np.float32)
    return q32, q64


def make_batch(B: int, K: int, V: int, *, seed: int, dtype: str = "bf16", z_sigma: float = 3.0,
               boost_frac: float = 0.0, boost: float = 0.0, draft_scale: float = 0.8,
               draft_sigma: float = 1.5, draft_at_row_temp: bool = False,
               temp_range: tuple[float, float] | None = (0.5, 1.2), temp_const: float | None = None,
               greedy_frac: float = 0.0, onehot_frac: float = 0.0, onehot_hit: float = 0.5,
               ragged: bool = False, name: str = "custom") -> VerifyInputs:
    """General seeded batch.

    Target logits z ~ N(0, z_sigma^2) per entry, plus ``boost`` on a Bernoulli(``boost_frac``)
    mask, rounded to ``dtype``.  Model-draft rows: draft logits = draft_scale * z + N(0,
    draft_sigma^2); q = softmax at T=1 (or at the row's temperature when
    ``draft_at_row_temp``); proposals x ~ q.  Greedy rows (temperature 0, a seeded
    ``greedy_frac`` of sequences) propose the draft logits' argmax.  One-hot rows (a seeded
    ``onehot_frac``) propose, per slot, the target row's argmax with probability
    ``onehot_hit`` and a uniform random id otherwise; their draft rows are NaN (never read).
    With ``ragged``, k_b ~ U{1..K} and every padded slot holds garbage that must not be read.
    """
    if dtype not in ("bf16", "f32"):
        raise ValueError(dtype)
    rz, rd, rt, rk, rx, ru, rr, _ = _streams(seed)

    # Row kinds and per-sequence scalars (drawn before the big arrays, fixed order).
    n_greedy = int(round(greedy_frac * B))
    n_onehot = int(round(onehot_frac * B))
    perm = rk.permutation(B)
    greedy = np.zeros(B, dtype=bool)
    greedy[perm[:n_greedy]] = True
    onehot = np.zeros(B, dtype=bool)
    onehot[perm[n_greedy:n_greedy + n_onehot]] = True
    if temp_const is not None:
        temperature = np.full(B, temp_const, dtype=np.float32)
    else:
        lo, hi = temp_range
        temperature = rt.uniform(lo, hi, size=B).astype(np.float32)
    temperature[greedy] = 0.0
    num_draft = rr.integers(1, K + 1, size=B).astype(np.int32) if ragged else None
    kb = np.full(B, K, dtype=np.int64) if num_draft is None else num_draft.astype(np.int64)

    logits = np.empty((B, K + 1, V), dtype=np.uint16 if dtype == "bf16" else np.float32)
    need_q = bool((~onehot).any()) and K > 0
    draft_probs = np.empty((B, K, V), dtype=np.float32) if need_q else None
    proposed = np.empty((B, K), dtype=np.int32)
    uniforms = ru.random((B, K + 1), dtype=np.float32)

    for b in range(B):
        z = rz.standard_normal((K + 1, V), dtype=np.float32) * np.float32(z_sigma)
        if boost_frac > 0.0:
            z = z + np.float32(boost) * (rz.random((K + 1, V)) < boost_frac).astype(np.float32)
        if dtype == "bf16":
            bits = f32_to_bf16_bits(z)
            zv = bf16_bits_to_f32(bits)
            logits[b] = bits
        else:
            zv = z
            logits[b] = z
        k = int(kb[b])
        if onehot[b]:
            hit = rx.random(K) < onehot_hit
            rand_ids = rx.integers(0, V, size=K)
            top = np.argmax(zv[:K], axis=-1) if K > 0 else np.zeros(0, dtype=np.int64)
            proposed[b] = np.where(hit, top, rand_ids).astype(np.int32)
            if draft_probs is not None:
                draft_probs[b] = np.float32(np.nan)
        else:
            dl = np.float32(draft_scale) * zv[:K] + np.float32(draft_sigma) * rd.standard_normal(
                (K, V), dtype=np.float32)
            qt = float(temperature[b]) if (draft_at_row_temp and temperature[b] > 0) else 1.0
            if K > 0:
                q32, q64 = _drafter_probs(dl, qt)
                draft_probs[b] = q32
                if greedy[b]:
                    proposed[b] = np.argmax(dl, axis=-1).astype(np.int32)
                else:
                    for i in range(K):
                        proposed[b, i] = rx.choice(V, p=q64[i])
        if ragged and k < K:
            # Padding the verifier must never read.
            if dtype == "bf16":
                logits[b, k + 1:] = BF16_NAN_BITS
            else:
                logits[b, k + 1:] = np.float32(np.nan)
            if draft_probs is not None:
                draft_probs[b, k:] = np.float32(np.nan)
            proposed[b, k:] = V + PAD_ID_OFFSET
            uniforms[b, k:K] = PAD_UNIFORM

    return VerifyInputs(logits, dtype, draft_probs,
                        onehot.astype(np.uint8) if n_onehot > 0 else None,
                        proposed, num_draft, temperature, uniforms, name=name,
                        meta=dict(seed=seed, greedy=greedy, onehot=onehot))


# --------------------------------------------------------------------------------------------
# The five workloads (sizes overridable so parity tests can run scaled-down copies).
# --------------------------------------------------------------------------------------------

def tiny_vocab(rounds: int = 100_000, V: int = 32, K: int = 4, seed: int = 1) -> VerifyInputs:
    """Tiny vocabulary: fixed fp32 target logits ~ N(0, 2^2), draft logits = target + N(0, 1),
    q = softmax at T=1, temperature 1.0; ``rounds`` independent rounds batched as B = rounds,
    each with fresh proposals x_i ~ q_i and fresh uniforms."""
    rz, rd, _, _, rx, ru, _, _ = _streams(seed)
    z = (rz.standard_normal((K + 1, V)) * 2.0).astype(np.float32)
    dl = (z[:K].astype(np.float64) + rd.standard_normal((K, V))).astype(np.float32)
    q32, q64 = _drafter_probs(dl, 1.0)
    proposed = np.empty((rounds, K), dtype=np.int32)
    for i in range(K):
        proposed[:, i] = rx.choice(V, size=rounds, p=q64[i])
    uniforms = ru.random((rounds, K + 1), dtype=np.float32)
    logits = np.ascontiguousarray(np.broadcast_to(z, (rounds, K + 1, V)))
    draft = np.ascontiguousarray(np.broadcast_to(q32, (rounds, K, V)))
    return VerifyInputs(logits, "f32", draft, None, proposed, None,
                        np.ones(rounds, dtype=np.float32), uniforms, name="tiny_vocab",
                        meta=dict(seed=seed, z=z, q=q32))


def single_sequence(B: int = 1, V: int = 32000, K: int = 4, seed: int = 2) -> VerifyInputs:
    """Single sequence: fp32 logits ~ N(0, 3^2), draft logits 0.8 z + N(0, 1) softmaxed at T=1,
    temperature 0.7, proposals drawn from q."""
    return make_batch(B, K, V, seed=seed, dtype="f32", z_sigma=3.0, draft_scale=0.8,
                      draft_sigma=1.0, temp_range=None, temp_const=0.7, name="single_sequence")


def batch64(B: int = 64, V: int = 128256, K: int = 5, seed: int = 3,
            calibrated: bool = False) -> VerifyInputs:
    """Batch: bf16 logits ~ N(0, 3^2), draft logits 0.8 z + N(0, 1.5^2) softmaxed at T=1, per-row
    temperature U[0.5, 1.2].  ``calibrated``: draft noise 0.5 and q softmaxed at the row's
    temperature, which lands the acceptance rate in 0.6-0.8."""
    return make_batch(B, K, V, seed=seed, dtype="bf16", z_sigma=3.0, draft_scale=0.8,
                      draft_sigma=0.5 if calibrated else 1.5, draft_at_row_temp=calibrated,
                      temp_range=(0.5, 1.2), name="batch64_calibrated" if calibrated else "batch64")


def large_batch_deep(B: int = 256, V: int = 152064, K: int = 8, seed: int = 4,
                     calibrated: bool = False) -> VerifyInputs:
    """Large batch, deep draft: bf16 logits ~ N(0, 4^2) with 1% of entries boosted by +8, 25%
    greedy rows (temperature 0, proposing the draft argmax), the rest at temperature 1.0 with
    proposals from q = softmax(0.8 z + N(0, 1.5^2)).  ``calibrated``: draft noise 0.3."""
    return make_batch(B, K, V, seed=seed, dtype="bf16", z_sigma=4.0, boost_frac=0.01, boost=8.0,
                      draft_scale=0.8, draft_sigma=0.3 if calibrated else 1.5, temp_range=None,
                      temp_const=1.0, greedy_frac=0.25,
                      name="large_batch_deep_calibrated" if calibrated else "large_batch_deep")


def ragged_mixed(B: int = 512, V: int = 128256, K: int = 8, seed: int = 5) -> VerifyInputs:
    """Ragged mixed drafters: per-sequence k_b ~ U{1..K} (padded to K), bf16 logits ~ N(0, 3^2),
    temperature U[0.5, 1.2]; half the rows n-gram (one-hot q), half model-draft fp32 q."""
    return make_batch(B, K, V, seed=seed, dtype="bf16", z_sigma=3.0, draft_scale=0.8,
                      draft_sigma=1.5, temp_range=(0.5, 1.2), onehot_frac=0.5, onehot_hit=0.5,
                      ragged=True, name="ragged_mixed")


CONFIGS = {
    "tiny_vocab": tiny_vocab,
    "single_sequence": single_sequence,
    "batch64": batch64,
    "batch64_calibrated": lambda **kw: batch64(calibrated=True, **kw),
    "large_batch_deep": large_batch_deep,
    "large_batch_deep_calibrated": lambda **kw: large_batch_deep(calibrated=True, **kw),
    "ragged_mixed": ragged_mixed,
}
