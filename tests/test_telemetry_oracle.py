"""Pins of the telemetry / dynamic-k oracle (CPU only): the page's printed best k per
(alpha, c), the alpha estimator on simulated rounds with a known rate, the counters against the
page's tokens-per-pass formula, and a hand-worked batch."""
import json
import math
import os

import numpy as np
import pytest

from oracle import closed_forms
from oracle.telemetry_oracle import (N_FIELDS, ROW, alpha_estimate, apply_k, choose_k, plan_k,
                                     telemetry_update)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_choose_k_reproduces_the_printed_best_k():
    g = json.load(open(os.path.join(GOLDEN, "page1_speedup_tables.json")))
    lo, hi = g["best_k_search_range"]
    for c_str, tab in g["tables"].items():
        for alpha, (k_best, s_best) in zip(g["alphas"], tab["best"]):
            k = choose_k(alpha, float(c_str), lo, hi)
            assert k == k_best, (c_str, alpha, k, k_best)
            assert round(closed_forms.speedup(alpha, k, float(c_str)), 2) == s_best


def test_choose_k_edges():
    assert choose_k(0.0, 0.05, 0, 10) == 0          # nothing survives: do not speculate
    assert choose_k(1.0, 0.0, 1, 12) == 12          # free, perfect drafts: the longest
    assert choose_k(0.9, 0.05, 3, 3) == 3


def simulate_rounds(alpha, k_of_b, rng):
    """Accepted lengths of rounds with iid per-position acceptance alpha."""
    acc = np.empty(len(k_of_b), dtype=np.int64)
    for b, k in enumerate(k_of_b):
        a = 0
        while a < k and rng.random() < alpha:
            a += 1
        acc[b] = a
    return acc


@pytest.mark.parametrize("alpha,K", [(0.3, 5), (0.75, 5), (0.9, 8)])
def test_alpha_estimate_and_tokens_per_pass(alpha, K):
    rng = np.random.default_rng(int(alpha * 100) + K)
    N = 60_000
    acc = simulate_rounds(alpha, [K] * N, rng)
    c = telemetry_update(np.zeros((1, ROW), np.int64), acc, None, None, K)
    a_hat = alpha_estimate(c[0])
    n_trials = c[0, 2] + c[0, 5]
    assert abs(a_hat - alpha) < 4.5 * math.sqrt(alpha * (1 - alpha) / n_trials)
    # Tokens per target pass (emitted / rounds) against the page's formula.
    tpp = c[0, 3] / c[0, 0]
    law = closed_forms.accept_length_law([alpha] * K)
    sd = math.sqrt(((np.arange(1, K + 2) - tpp) ** 2 * law).sum() / N)
    assert abs(tpp - closed_forms.expected_tokens(alpha, K)) < 4.5 * sd
    # The histogram is the accept-length law.
    hist = c[0, N_FIELDS:N_FIELDS + K + 1] / N
    assert np.abs(hist - law).max() < 0.01


def test_hand_worked_update_and_plan():
    K = 4
    acc = np.array([0, 4, 2, -1, 1, 3])
    nd = np.array([4, 4, 3, 4, 1, 9])           # the last k_b is out of range: invalid
    route = np.array([0, 1, 0, 0, 5, 1])        # route 5 does not exist (2 routes)
    c = telemetry_update(np.zeros((2, ROW), np.int64), acc, nd, route, K)
    # route 0: rows 0 (A=0,k=4), 2 (A=2,k=3), 3 invalid
    assert c[0, :N_FIELDS].tolist() == [2, 7, 2, 4, 0, 2, 1, 0]
    # route 1: row 1 (A=4,k=4), row 5 invalid
    assert c[1, :N_FIELDS].tolist() == [1, 4, 4, 5, 1, 0, 1, 0]
    assert c[0, N_FIELDS + 0] == 1 and c[0, N_FIELDS + 2] == 1 and c[1, N_FIELDS + 4] == 1
    assert alpha_estimate(c[0]) == 0.5 and alpha_estimate(c[1]) == 1.0
    empty = np.zeros((1, ROW), np.int64)
    assert math.isnan(alpha_estimate(empty[0]))
    table = plan_k(np.vstack([c, empty]), 0.05, 1, 20, 5)
    assert table.tolist() == [choose_k(0.5, 0.05, 1, 20), 20, 5]
    assert apply_k(np.array([6, 6, -1, 2]), np.array([0, 2, 0, 9]), table, 8).tolist() == \
        [min(6, int(table[0])), 5, -1, 2]
