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


def test_noalloc_on_a_created_stream():
    # The scratch is the one of the device the call's stream belongs to: a call enqueued on a
    # created stream (not the null stream) is bit-identical to specdec_verify.
    inp = gen.make_batch(16, 4, 30000, seed=934, onehot_frac=0.25, ragged=True)
    print(f"\n[case] noalloc on a created stream B={inp.B} K={inp.K} V={inp.V}", flush=True)
    d = inputs_to_device(inp, DEV)
    want = specdec_verify(d["logits"], d["draft_probs"], d["proposed"], d["temperature"],
                          d["uniforms"], draft_onehot=d["draft_onehot"], num_draft=d["num_draft"])
    out = (torch.full((inp.B,), -7, dtype=torch.int32, device=DEV),
           torch.full((inp.B, inp.K + 1), -7, dtype=torch.int32, device=DEV),
           torch.full((inp.B, inp.K + 1), -7.0, dtype=torch.float32, device=DEV))
    s = torch.cuda.Stream()
    assert s.cuda_stream != 0
    s.wait_stream(torch.cuda.current_stream())
    got = specdec_verify_noalloc(d["logits"], d["draft_probs"], d["proposed"], d["temperature"],
                                 d["uniforms"], draft_onehot=d["draft_onehot"],
                                 num_draft=d["num_draft"], out=out, stream=s)
    s.synchronize()
    for g, w in zip(got, want):
        assert np.array_equal(_bits(g), _bits(w))


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


def test_noalloc_at_the_largest_batch_its_scratch_holds():
    # K = 3, V = 32000: the largest B whose workspace fits the scratch runs and matches
    # specdec_verify bit for bit; one sequence more is refused before any launch.  One-hot drafts
    # (no draft tensor), inputs drawn on the device: about 3 GB of bf16 logits.
    lib = load_library()
    K, V = 3, 32000
    lim = lib.specdec_noalloc_scratch_bytes()
    B = 1
    while lib.specdec_workspace_size(2 * B, K, V) <= lim:
        B *= 2
    lo, hi = B, 2 * B                       # largest B with workspace_size(B) <= lim in [lo, hi)
    while hi - lo > 1:
        mid = (lo + hi) // 2
        lo, hi = (mid, hi) if lib.specdec_workspace_size(mid, K, V) <= lim else (lo, mid)
    B = lo
    print(f"\n[case] noalloc largest batch B={B} K={K} V={V}", flush=True)
    g = torch.Generator(device=DEV).manual_seed(941)
    logits = (torch.randn((B, K + 1, V), generator=g, device=DEV) * 3.0).to(torch.bfloat16)
    proposed = torch.randint(0, V, (B, K), generator=g, device=DEV, dtype=torch.int32)
    temperature = torch.rand(B, generator=g, device=DEV) * 0.7 + 0.5
    uniforms = torch.rand((B, K + 1), generator=g, device=DEV).clamp_(max=0.999999)
    onehot = torch.ones(B, dtype=torch.uint8, device=DEV)
    want = specdec_verify(logits, None, proposed, temperature, uniforms, draft_onehot=onehot)
    out = (torch.empty(B, dtype=torch.int32, device=DEV),
           torch.empty((B, K + 1), dtype=torch.int32, device=DEV),
           torch.empty((B, K + 1), dtype=torch.float32, device=DEV))
    got = specdec_verify_noalloc(logits, None, proposed, temperature, uniforms,
                                 draft_onehot=onehot, out=out)
    torch.cuda.synchronize()
    for a, w in zip(got, want):
        assert np.array_equal(_bits(a), _bits(w))
    assert (got[0].cpu().numpy() >= 0).all()
    fake = ctypes.c_void_p(0x1000)
    st = lib.specdec_verify_noalloc(fake, 1, None, fake, fake, None, fake, fake, B + 1, K, V,
                                    fake, fake, fake, None)
    assert st == -7
    del logits, proposed, temperature, uniforms, onehot, want, out, got
    torch.cuda.empty_cache()


def test_noalloc_calls_replay_from_a_hip_graph():
    # The callers it is for: two calls captured in one HIP graph (after a first eager call on the
    # device), replayed several times with eager work in between, each replay bit-identical to
    # the eager results.
    inp = [gen.make_batch(24, 4, 30000, seed=951, onehot_frac=0.25, ragged=True),
           gen.make_batch(8, 2, 700, seed=952, dtype="f32")]
    d = [inputs_to_device(x, DEV) for x in inp]
    outs = [(torch.empty(x.B, dtype=torch.int32, device=DEV),
             torch.empty((x.B, x.K + 1), dtype=torch.int32, device=DEV),
             torch.empty((x.B, x.K + 1), dtype=torch.float32, device=DEV)) for x in inp]

    def calls():
        for dd, out in zip(d, outs):
            specdec_verify_noalloc(dd["logits"], dd["draft_probs"], dd["proposed"],
                                   dd["temperature"], dd["uniforms"],
                                   draft_onehot=dd["draft_onehot"], num_draft=dd["num_draft"],
                                   out=out)
    calls()
    torch.cuda.synchronize()
    want = [[_bits(t).copy() for t in out] for out in outs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        calls()
    torch.cuda.synchronize()
    for rep in range(4):
        for out in outs:
            for t in out:
                t.fill_(-3)
        junk = torch.randn(1 << 20, device=DEV).sum()  # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        del junk
        for out, w in zip(outs, want):
            for t, wt in zip(out, w):
                assert np.array_equal(_bits(t), wt), rep
