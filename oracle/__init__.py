"""fp64 CPU oracle of the speculative-decoding verify step (test infrastructure only).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import this
package; the library and its binding never do.
"""
from .verify_oracle import OracleOut, TEMPERATURE_MIN, inverse_cdf, logit_row, target_probs, verify, verify_row
from .ngram_oracle import ngram_propose, propose_one
from .commit_oracle import commit
from .match_oracle import verify_match
from . import telemetry_oracle
from . import closed_forms

__all__ = ["OracleOut", "TEMPERATURE_MIN", "inverse_cdf", "logit_row", "target_probs", "verify",
           "verify_row", "closed_forms", "ngram_propose", "propose_one", "commit", "verify_match",
           "telemetry_oracle"]
