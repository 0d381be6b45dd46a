"""specdec_verify_noalloc (the entry point that allocates nothing: its workspace is the library's
built-in device scratch) against specdec_verify with a caller workspace, through the C ABI:
calls in a row on the same device scratch, each smaller than the one before (the last one on the
small-vocabulary path), each bit-identical to specdec_verify and within the oracle parity bar."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from oracle.parity import compare
from speculative_decoding_verification_specdec_amd import (inputs_to_device, specdec_verify,
                                                           specdec_verify_noalloc)
from speculative_decoding_verification_specdec_amd import inputs as gen
from speculative_decoding_verification_specdec_amd.binding import load_library

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _bits(t):
    a = t.cpu().numpy()
    return a.view(np.uint32) if a.dtype == np.float32 else a


def test_noalloc_matches_verify_on_two_calls_the_second_smaller():
    cases = [gen.make_batch(48, 5, 60000, seed=931, greedy_frac=0.25, onehot_frac=0.25,
                            ragged=True),
             gen.make_batch(12, 3, 20003, seed=932, dtype="f32", onehot_frac=0.25),
             gen.make_batch(40, 4, 500, seed=933, onehot_frac=0.25, ragged=True)]
    for inp in cases:
        print(f"\n[case] noalloc B={inp.B} K={inp.K} V={inp.V} {inp.logits_dtype}", flush=True)
        d = inputs_to_device(inp, DEV)
        want = specdec_verify(d["logits"], d["draft_probs"], d["proposed"], d["temperature"],
                              d["uniforms"], draft_onehot=d["draft_onehot"],
                              num_draft=d["num_draft"])
        out = (torch.full((inp.B,), -7, dtype=torch.int32, device=DEV),
               torch.full((inp.B, inp.K + 1), -7, dtype=torch.int32, device=DEV),
               torch.full((inp.B, inp.K + 1), -7.0, dtype=torch.float32, device=DEV))
        torch.cuda.synchronize()
        before = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        got = specdec_verify_noalloc(d["logits"], d["draft_probs"], d["proposed"],
                                     d["temperature"], d["uniforms"],
                                     draft_onehot=d["draft_onehot"], num_draft=d["num_draft"],
                                     out=out)
        torch.cuda.synchronize()
        # Nothing allocated through torch during the call (the peak includes short-lived
        # temporaries), nor held after it.
        assert torch.cuda.max_memory_allocated() == before
        assert torch.cuda.memory_allocated() == before
        for g, w in zip(got, want):
            assert np.array_equal(_bits(g), _bits(w))
        rep = compare(inp, oracle.verify(inp), *(t.cpu().numpy() for t in got))
        assert rep["mismatch"] == 0, rep["details"]
        del d, want, out, got


def test_noalloc_refuses_sizes_beyond_its_scratch():
    # Checked on the host before any launch: B = 4096, K = 8, V = 128256 needs more than 32 MiB.
    lib = load_library()
    assert lib.specdec_noalloc_scratch_bytes() == 32 << 20
    need = lib.specdec_workspace_size(4096, 8, 128256)
    assert need > lib.specdec_noalloc_scratch_bytes()
    fake = ctypes.c_void_p(0x1000)
    st = lib.specdec_verify_noalloc(fake, 1, fake, None, fake, None, fake, fake, 4096, 8, 128256,
                                    fake, fake, fake, None)
    assert st == -7
    assert b"scratch" in lib.specdec_status_string(st)
