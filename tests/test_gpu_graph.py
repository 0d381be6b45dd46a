"""HIP-graph capture of the C-ABI entry points.

The library allocates nothing and enqueues only kernels (no memset nodes), so a caller may
capture its calls.  Each test captures calls on two input replicas into one graph (sharing one
workspace, as the benchmark does), then replays the graph several times with eager work and
synchronisations in between -- an eager call on other inputs through the same workspace, and
the outputs cleared -- and checks every replay bit-for-bit against the eager results.
"""
import numpy as np
import pytest
import torch

from speculative_decoding_verification_specdec_amd import (inputs_to_device, specdec_ngram_propose,
                                                           specdec_ngram_workspace_size,
                                                           specdec_verify, specdec_verify_match,
                                                           specdec_workspace_size)
from speculative_decoding_verification_specdec_amd import contexts as hist
from speculative_decoding_verification_specdec_amd import inputs as gen

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
REPLAYS = 4


def outputs(B, K):
    return (torch.empty(B, dtype=torch.int32, device=DEV),
            torch.empty((B, K + 1), dtype=torch.int32, device=DEV),
            torch.empty((B, K + 1), dtype=torch.float32, device=DEV))


def replay_and_check(graph, stream, outs, expected, perturb):
    for r in range(REPLAYS):
        for o in outs:
            for t in o:
                t.fill_(-7)                      # eager kernels between replays
        perturb()
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            graph.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, expected):
            for t, et in zip(o, e):
                assert torch.equal(t, et), f"replay {r} differs from the eager call"


# V = 20008: the streaming kernels; V = 32: the small-vocabulary kernel (eight sequences a wave).
@pytest.mark.parametrize("V", [20008, 32])
@pytest.mark.parametrize("match", [False, True])
def test_verify_graph_replays_match_eager(match, V):
    print(f"\n[case] graph verify match={match} V={V}", flush=True)
    inps = [gen.make_batch(16, 5, V, seed=80 + i, greedy_frac=0.25, onehot_frac=0.25,
                           ragged=True) for i in range(2)]
    other = inputs_to_device(gen.make_batch(16, 5, V, seed=90), DEV)
    B, K = 16, 5
    ws = torch.zeros(specdec_workspace_size(B, K, V), dtype=torch.uint8, device=DEV)
    ds = [inputs_to_device(i, DEV) for i in inps]

    def call(d, out):
        if match:
            return specdec_verify_match(d["logits"], d["proposed"], d["temperature"],
                                        d["uniforms"], num_draft=d["num_draft"], out=out,
                                        workspace=ws)
        return specdec_verify(d["logits"], d["draft_probs"], d["proposed"], d["temperature"],
                              d["uniforms"], draft_onehot=d["draft_onehot"],
                              num_draft=d["num_draft"], out=out, workspace=ws)

    expected = [tuple(t.clone() for t in call(d, outputs(B, K))) for d in ds]
    torch.cuda.synchronize()
    outs = [outputs(B, K) for _ in ds]
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for d, o in zip(ds, outs):               # untimed warm-up on the capture stream
            call(d, o)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for d, o in zip(ds, outs):
            call(d, o)
    scratch = outputs(B, K)
    replay_and_check(g, stream, outs, expected, lambda: call(other, scratch))


def test_ngram_graph_replays_match_eager():
    print("\n[case] graph ngram", flush=True)
    hs = [hist.make_histories(24, 20000, 5000, seed=95 + i, len_range=(100, 20000))
          for i in range(2)]
    ws = torch.empty(specdec_ngram_workspace_size(24, 20000), dtype=torch.uint8, device=DEV)
    ts = [(torch.from_numpy(h.tokens).to(DEV), torch.from_numpy(h.lengths).to(DEV)) for h in hs]
    K = 8

    def call(t, out):
        return specdec_ngram_propose(t[0], t[1], K, n_min=1, n_max=4, out=out, workspace=ws)

    def fresh():
        return (torch.empty((24, K), dtype=torch.int32, device=DEV),
                torch.empty(24, dtype=torch.int32, device=DEV))

    expected = [tuple(x.clone() for x in call(t, fresh())) for t in ts]
    torch.cuda.synchronize()
    outs = [fresh() for _ in ts]
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for t, o in zip(ts, outs):
            call(t, o)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for t, o in zip(ts, outs):
            call(t, o)
    other = (ts[1][0].flip(0).contiguous(), ts[1][1].flip(0).contiguous())
    scratch = fresh()
    replay_and_check(g, stream, outs, expected, lambda: call(other, scratch))
    assert (expected[0][1].cpu().numpy() >= 0).all()
    assert np.any(expected[0][1].cpu().numpy() > 0)
