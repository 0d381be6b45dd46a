"""Pins of the match-mode oracle (CPU only).

"Decodificação especulativa explicada" (gsantana.dev), section "A regra de amostragem por
rejeição": drawing a target token at every position and keeping the draft only while the two
agree is exact (every emitted token is a draw from p) and accepts with probability
sum_x p(x) q(x), less than the rejection rule's sum_x min(p(x), q(x)).  Checked here by
simulation on the tiny-vocabulary workload, with a chi-square test of the emitted tokens against
p and a negative control that the same test catches.
"""
import numpy as np
import pytest
import scipy.stats

import oracle
from oracle.match_oracle import verify_match
from speculative_decoding_verification_specdec_amd import inputs as gen

ROUNDS = 40_000


@pytest.fixture(scope="module")
def tiny():
    inp = gen.tiny_vocab(rounds=ROUNDS)
    z, q = inp.meta["z"].astype(np.float64), inp.meta["q"].astype(np.float64)
    p = np.exp(z - z.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    return inp, p, q


@pytest.fixture(scope="module")
def tiny_ref(tiny):
    return verify_match(tiny[0])


def chi2_p(tokens, p):
    obs = np.bincount(tokens, minlength=len(p)).astype(np.float64)
    exp = p * len(tokens)
    big = exp >= 5                       # pool the cells with small expectations
    o = np.append(obs[big], obs[~big].sum())
    e = np.append(exp[big], exp[~big].sum())
    if e[-1] == 0:
        o, e = o[:-1], e[:-1]
    return scipy.stats.chisquare(o, e).pvalue


def test_acceptance_rate_is_sum_p_times_q(tiny, tiny_ref):
    inp, p, q = tiny
    ref = tiny_ref
    acc0 = (ref.accept_len >= 1).mean()
    alpha_match = float((p[0] * q[0]).sum())
    alpha_rej = float(np.minimum(p[0], q[0]).sum())
    se = np.sqrt(alpha_match * (1 - alpha_match) / ROUNDS)
    assert abs(acc0 - alpha_match) < 4.5 * se
    assert alpha_match < alpha_rej
    # Position 1, given position 0 was kept: again sum p_1 q_1.
    kept = ref.accept_len >= 1
    acc1 = (ref.accept_len[kept] >= 2).mean()
    a1 = float((p[1] * q[1]).sum())
    assert abs(acc1 - a1) < 4.5 * np.sqrt(a1 * (1 - a1) / kept.sum())


def test_emitted_tokens_follow_p_and_the_resample_bug_does_not(tiny, tiny_ref):
    inp, p, _ = tiny
    ref = tiny_ref
    assert chi2_p(ref.out_tokens[:, 0], p[0]) > 1e-4
    one = ref.accept_len >= 1
    assert chi2_p(ref.out_tokens[one, 1], p[1]) > 1e-4
    bug = verify_match(inp, resample_bug=True)
    assert chi2_p(bug.out_tokens[:, 0], p[0]) < 1e-6


def test_rounds_yield_between_1_and_k_plus_1_tokens(tiny):
    inp, _, _ = tiny
    ref = verify_match(inp, rows=range(2000))
    K = inp.K
    assert ((ref.accept_len >= 0) & (ref.accept_len <= K)).all()
    emitted = (ref.out_tokens >= 0).sum(axis=1)
    assert (emitted == ref.accept_len + 1).all()
    # Kept slots hold the drafts themselves.
    for j in range(2000):
        a = ref.accept_len[j]
        assert (ref.out_tokens[j, :a] == inp.proposed[j, :a]).all()


def test_greedy_rows_equal_the_verify_greedy_rows():
    inp = gen.make_batch(24, 4, 3000, seed=31, dtype="bf16", greedy_frac=1.0)
    a, b = verify_match(inp), oracle.verify(inp)
    assert np.array_equal(a.accept_len, b.accept_len)
    assert np.array_equal(a.out_tokens, b.out_tokens)


def test_page1_toy_match_acceptance_is_below_the_rejection_rule():
    # The page-1 toy (V = 4 bigram target and draft from numpy default_rng(2)); it reproduces the
    # page's printed per-context alpha of the rejection rule, and the match scheme's
    # sum p q is lower in every context.
    g = np.random.default_rng(2)
    P = g.dirichlet(np.ones(4), size=4)
    Q = 0.55 * P + 0.45 * g.dirichlet(np.ones(4), size=4)
    pq, mn = (P * Q).sum(1), np.minimum(P, Q).sum(1)
    assert np.allclose(np.round(mn, 3), [0.672, 0.692, 0.856, 0.863])
    assert (pq < mn).all()


def test_invalid_rows():
    inp = gen.make_batch(6, 3, 500, seed=32, dtype="f32")
    inp.uniforms[1, 0] = 1.0          # a used uniform outside [0, 1)
    inp.proposed[2, 1] = 500          # an id outside [0, V)
    inp.temperature[3] = -1.0
    inp.logits[4, 2, 7] = np.inf
    ref = verify_match(inp)
    assert ref.accept_len[1:5].tolist() == [-1] * 4
    assert (ref.out_tokens[1:5] == -1).all() and (ref.out_probs[1:5] == 0).all()
    assert ref.accept_len[0] >= 0 and ref.accept_len[5] >= 0


def test_out_probs_are_the_target_probability_of_each_emitted_token():
    # Every emitted slot reports softmax(z_i / T)(token_i) of its own row i -- scipy's softmax
    # of the raw logit row, at T = 1 for greedy rows -- and unused slots report 0.  A kept draft
    # and a mismatch token are both pinned, so reporting p(x_i) instead of p(y_i) at a mismatch,
    # or another row's p, fails here.
    import scipy.special
    inp = gen.make_batch(40, 4, 400, seed=611, dtype="f32", greedy_frac=0.25, ragged=True,
                         draft_sigma=0.3, draft_at_row_temp=True)
    ref = verify_match(inp)
    kept = mismatch = 0
    for b in range(inp.B):
        A = int(ref.accept_len[b])
        assert A >= 0
        T = float(inp.temperature[b]) or 1.0
        for i in range(inp.K + 1):
            if i > A:
                assert ref.out_tokens[b, i] == -1 and ref.out_probs[b, i] == 0.0
                continue
            y = int(ref.out_tokens[b, i])
            want = scipy.special.softmax(inp.logits[b, i].astype(np.float64) / T)[y]
            assert ref.out_probs[b, i] == pytest.approx(want, rel=1e-12, abs=0.0)
            if i < A:
                kept += 1
                assert y == int(inp.proposed[b, i])
            elif A < inp.draft_counts()[b]:
                mismatch += 1
                assert y != int(inp.proposed[b, i])
    assert kept > 10 and mismatch > 10
