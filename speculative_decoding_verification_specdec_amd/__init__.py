"""MI355X-native batched speculative-decoding verify step.

The compute lives in ``libspecdec.so`` (hand-written HIP for gfx950 behind a C ABI declared in
``include/specdec.h``); ``specdec_verify`` and friends below only marshal torch device tensors
into that ABI.  Importing the package does not load the library; the first call does, and it
raises if the library is missing.
"""
from .binding import (SpecdecError, specdec_verify, specdec_verify_greedy, specdec_workspace_size,
                      specdec_status_string, library_path, load_library,
                      inputs_to_device, specdec_ngram_propose, specdec_ngram_workspace_size,
                      specdec_commit, specdec_verify_match, specdec_telemetry_update,
                      specdec_apply_k, specdec_plan_k, telemetry_counters,
                      SPECDEC_PATH_AUTO, SPECDEC_PATH_STREAMING, SPECDEC_PATH_SMALL_VOCAB,
                      SPECDEC_SMALL_V_MAX, SPECDEC_PATH_ONE_LAUNCH, SPECDEC_PATH_QUAD, new_workspace,
                      specdec_verify_noalloc)

__all__ = ["SpecdecError", "specdec_verify", "specdec_verify_greedy", "specdec_workspace_size",
           "specdec_status_string", "library_path", "load_library", "inputs_to_device",
           "specdec_ngram_propose", "specdec_ngram_workspace_size", "specdec_commit",
           "specdec_verify_match", "specdec_telemetry_update", "specdec_apply_k",
           "specdec_plan_k", "telemetry_counters", "SPECDEC_PATH_AUTO", "SPECDEC_PATH_STREAMING",
           "SPECDEC_PATH_SMALL_VOCAB", "SPECDEC_SMALL_V_MAX", "SPECDEC_PATH_ONE_LAUNCH",
           "SPECDEC_PATH_QUAD",
           "new_workspace", "specdec_verify_noalloc"]
