"""The output-law checks of tests/laws.py, run against the fp64 oracle on the CPU.

The GPU statistics tests hold the kernels to these laws; here the same checks pass on the oracle's
outputs for the same kind of rounds, and they reject the negative control that redraws from p
instead of the residual ("Decodificação especulativa explicada", section "A regra de amostragem
por rejeição": the biased fallback), so the checks have the power they are trusted with.
"""
import pytest

import oracle
from laws import Case, check_laws

CASES = {
    "tiny_vocab": dict(V=32, K=4, N=3000, seed=101),
    "onehot_ragged": dict(V=64, K=3, N=3000, seed=105, T=0.8, onehot=True, ragged=True),
}


@pytest.mark.parametrize("name", list(CASES))
def test_oracle_obeys_the_output_laws(name):
    case = Case(**CASES[name], device="cpu")
    out = oracle.verify(case.host_inputs())
    check_laws(case, out.accept_len, out.out_tokens, case.alphas())


def test_match_oracle_obeys_the_output_laws():
    case = Case(V=32, K=4, N=3000, seed=111, device="cpu")
    out = oracle.verify_match(case.host_inputs())
    check_laws(case, out.accept_len, out.out_tokens, case.alphas(match=True))


def test_the_checks_reject_redrawing_from_p():
    case = Case(V=32, K=4, N=3000, seed=107, device="cpu")
    out = oracle.verify(case.host_inputs(), buggy=True)
    with pytest.raises(AssertionError, match="slot0"):
        check_laws(case, out.accept_len, out.out_tokens, case.alphas())
