"""GPU output laws: the kernels' own outputs against the distributions the pages fix.

These do not go through the oracle's sampler.  One fixed set of target rows (and draft rows) is
replicated over many independent rounds on the device, each round with its own proposals and
uniforms, and the tokens the HIP path emits are compared with closed forms:
  * slot i, given that the round reached it (A >= i), is distributed as p_i -- the accept-or-
    residual step and the bonus draw both reproduce the target ("Decodificação especulativa
    explicada", section "A regra de amostragem por rejeição"; "ch15 · Speculative Decoding",
    section "The build");
  * the accept length follows P(A >= a) = prod_{i<a} alpha_i with alpha_i = sum min(p_i, q_i)
    for a model drafter, sum r_i(x) p_i(x) for a one-hot drafter proposing x ~ r_i, and
    sum p_i q_i for the sample-and-match mode (same page, sections "A regra de amostragem por
    rejeição" and "Quanto mais rápido: a matemática").
Pearson chi-square, cells with expected count < 5 pooled; every p-value above 1e-3 divided by the
number of tests in the case (tests/laws.py).  Inputs are seeded, so each case's outcome is fixed.
"""
import pytest

from laws import Case, check_laws

pytestmark = pytest.mark.gpu


CASES = {
    # The tiny-vocabulary workload: 1e5 rounds, fp32, temperature 1.
    "tiny_vocab": dict(V=32, K=4, N=100_000, seed=101),
    "bf16_V1000_T07": dict(V=1000, K=3, N=100_000, seed=102, dtype="bf16", T=0.7, z_sigma=2.5),
    "f32_odd_V_ragged": dict(V=777, K=5, N=100_000, seed=103, T=1.2, ragged=True),
    "bf16_two_chunks": dict(V=9000, K=2, N=20_000, seed=104, dtype="bf16", z_sigma=1.0,
                            draft_sigma=0.5),
    "onehot_V64": dict(V=64, K=3, N=100_000, seed=105, T=0.8, onehot=True),
    "bf16_V50_ragged": dict(V=50, K=7, N=100_000, seed=107, dtype="bf16", T=0.9, ragged=True),
    "onehot_bf16_ragged": dict(V=512, K=4, N=100_000, seed=106, dtype="bf16", onehot=True,
                               ragged=True),
}


@pytest.mark.parametrize("name", list(CASES))
def test_verify_output_law(name):
    print(f"\n[case] law {name} {CASES[name]}", flush=True)
    case = Case(**CASES[name])
    acc, tok = case.run()
    check_laws(case, acc, tok, case.alphas())


MATCH_CASES = {
    "tiny_vocab": dict(V=32, K=4, N=100_000, seed=111),
    "bf16_V1000_ragged": dict(V=1000, K=3, N=100_000, seed=112, dtype="bf16", T=0.7,
                              draft_sigma=0.3, ragged=True),
}


@pytest.mark.parametrize("name", list(MATCH_CASES))
def test_match_mode_output_law(name):
    print(f"\n[case] match law {name} {MATCH_CASES[name]}", flush=True)
    case = Case(**MATCH_CASES[name])
    acc, tok = case.run(match=True)
    check_laws(case, acc, tok, case.alphas(match=True))


def test_rejection_rule_accepts_more_than_matching_on_the_same_rounds():
    # sum min(p, q) >= sum p q for every row; the two modes share proposals and uniforms.
    case = Case(V=200, K=4, N=50_000, seed=121, draft_sigma=0.5)
    acc_r, _ = case.run()
    acc_m, _ = case.run(match=True)
    assert all(a >= m for a, m in zip(case.alphas(), case.alphas(match=True)))
    assert acc_r.mean() > acc_m.mean()
