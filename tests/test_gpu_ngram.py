"""GPU parity of the n-gram drafter (through the C ABI) against its CPU oracle.

Integer work: proposals and counts must be bit-exact.  Cases span one and several 8192-position
tiles with a ragged last tile, the 16-byte and the 4-byte load paths, every degenerate history
(empty, one token, repeated token, nothing repeats), invalid lengths, and the full 512 x 8192
drafting workload (sampled sequences, in the launch configuration the benchmark times).
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from oracle.parity import compare
from speculative_decoding_verification_specdec_amd import (inputs_to_device, specdec_ngram_propose,
                                                           specdec_verify)
from speculative_decoding_verification_specdec_amd import contexts as hist
from speculative_decoding_verification_specdec_amd import inputs as gen

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def run_gpu(tokens, lengths, K, n_min, n_max, misalign=False):
    B, cap = tokens.shape
    if misalign:   # a base address that is 4- but not 16-byte aligned: the 4-byte load path
        buf = torch.empty(B * cap + 1, dtype=torch.int32, device=DEV)
        t = buf[1:].view(B, cap)
        t.copy_(torch.from_numpy(tokens))
    else:
        t = torch.from_numpy(tokens).to(DEV)
    ln = torch.from_numpy(lengths).to(DEV)
    prop, nd = specdec_ngram_propose(t, ln, K, n_min=n_min, n_max=n_max)
    torch.cuda.synchronize()
    return prop.cpu().numpy(), nd.cpu().numpy()


def check(h, K, n_min, n_max, rows=None, misalign=False):
    print(f"\n[case] {h.name} B={h.B} cap={h.capacity} K={K} n={n_min}..{n_max} "
          f"misalign={misalign}", flush=True)
    prop, nd = run_gpu(h.tokens, h.lengths, K, n_min, n_max, misalign)
    sel = np.arange(h.B) if rows is None else np.asarray(rows)
    ref_p, ref_n = oracle.ngram_propose(h.tokens[sel], h.lengths[sel], n_min, n_max, K)
    assert np.array_equal(nd[sel], ref_n), np.nonzero(nd[sel] != ref_n)
    assert np.array_equal(prop[sel], ref_p), np.nonzero((prop[sel] != ref_p).any(axis=1))
    print(f"[report] proposing={(ref_n > 0).sum()}/{len(sel)} mean_k={ref_n[ref_n > 0].mean() if (ref_n > 0).any() else 0:.2f}",
          flush=True)
    return prop, nd


@pytest.mark.parametrize("V,cap,K,n_min,n_max", [
    (12, 300, 5, 1, 3), (12, 300, 8, 2, 32), (3, 256, 63, 1, 4), (50, 301, 1, 1, 1),
    (1000, 512, 6, 1, 5),
])
def test_small_histories(V, cap, K, n_min, n_max):
    h = hist.make_histories(96, cap, V, seed=200 + V + cap, len_range=(0, cap), seg_range=(1, 12),
                            edge_cases=True, name=f"small_V{V}")
    check(h, K, n_min, n_max)


@pytest.mark.parametrize("cap,misalign", [(20004, False), (20001, False), (20004, True),
                                          (8192, False), (8191, True), (4096, False),
                                          (4093, True)])
def test_several_tiles_and_load_paths(cap, misalign):
    # One or several 8192-position tiles with a ragged last one; a small vocabulary makes
    # matches frequent everywhere, including across tile boundaries.
    h = hist.make_histories(24, cap, 40, seed=300 + cap, len_range=(cap - 3000, cap),
                            seg_range=(2, 30), edge_cases=True, name="multi_tile")
    check(h, 8, 1, 4, misalign=misalign)


@pytest.mark.parametrize("cap,at", [(16400, 8192), (16400, 512), (16400, 1024), (16400, 8704),
                                    (16402, 8192)])
def test_matches_that_straddle_a_tile_boundary(cap, at):
    # History ending in the run 1 2 3 4 whose only earlier occurrence straddles position `at`: the
    # boundary between the first two 8192-position tiles, or between 512-position steps searched by
    # different waves of the one-workgroup-per-history kernel (capacity a multiple of 4), or, with
    # capacity 16402, the tile boundary on the 4-byte load path.
    toks = np.full((1, cap), hist.PAD_TOKEN, dtype=np.int32)
    L = 16390
    body = (np.arange(L) % 997 + 10).astype(np.int32)        # only values >= 10 elsewhere
    body[at - 2:at + 2] = [1, 2, 3, 4]
    body[at + 2] = 77
    body[L - 4:] = [1, 2, 3, 4]
    toks[0, :L] = body
    h = hist.Histories(toks, np.array([L], dtype=np.int32), 1000, name=f"straddle{at}")
    prop, nd = check(h, 5, 1, 4)
    assert nd[0] == 5 and prop[0, 0] == 77


@pytest.mark.parametrize("cap,V,n_max", [(8196, 3, 32), (16384, 40, 8), (40000, 7, 32),
                                         (65536, 2, 32)])
def test_one_workgroup_per_history_path(cap, V, n_max):
    # Capacities above one tile with 16-byte rows: one workgroup per history, its waves taking
    # 512-position steps in turn.  Lengths from 0 to the capacity (some waves get no step), tiny
    # vocabularies (candidates everywhere, runs crossing step boundaries and reaching 31 tokens
    # back into the step before), and the degenerate histories.
    h = hist.make_histories(24, cap, V, seed=500 + cap + V, len_range=(0, cap), seg_range=(1, 40),
                            edge_cases=True, name=f"history_path_V{V}")
    check(h, 12, 1, n_max)


def test_invalid_lengths_and_k0():
    h = hist.make_histories(6, 64, 5, seed=9, len_range=(10, 64))
    h.lengths[1] = -1
    h.lengths[3] = 65
    prop, nd = check(h, 4, 1, 3)
    assert nd[1] == -1 and nd[3] == -1 and (prop[[1, 3]] == -1).all()
    t = torch.from_numpy(h.tokens).to(DEV)
    ln = torch.from_numpy(h.lengths).to(DEV)
    p0, n0 = specdec_ngram_propose(t, ln, 0, n_min=1, n_max=3)
    torch.cuda.synchronize()
    n0 = n0.cpu().numpy()
    assert n0[1] == -1 and n0[3] == -1 and (np.delete(n0, [1, 3]) == 0).all()


def test_full_workload_sampled():
    h = hist.ngram_workload()
    rows = np.random.default_rng(11).choice(h.B, size=48, replace=False)
    prop, nd = check(h, 8, 1, 4, rows=rows)
    # The whole batch: every count is valid and every proposal is a copy of the history.
    assert ((nd >= 0) & (nd <= 8)).all()
    for b in range(h.B):
        k = int(nd[b])
        assert (prop[b, k:] == -1).all()


def test_long_workload_sampled():
    # 256 histories of 32768-65536 tokens, capacity 65536: eight tiles per history, so the
    # multi-tile path (per-tile keys, then the emit kernel) in the benchmark's launch shape.
    h = hist.ngram_long_workload()
    rows = np.random.default_rng(13).choice(h.B, size=32, replace=False)
    prop, nd = check(h, 8, 1, 4, rows=rows)
    assert ((nd >= 0) & (nd <= 8)).all()


def test_drafts_feed_the_verify_step():
    # The drafter's proposals, verified as one-hot rows, match the verify oracle.
    B, K, V = 16, 6, 3000
    h = hist.make_histories(B, 600, V, seed=12, len_range=(300, 600), seg_range=(4, 20))
    prop, nd = run_gpu(h.tokens, h.lengths, K, 1, 3)
    base = gen.make_batch(B, K, V, seed=13, dtype="bf16")
    inp = dataclasses.replace(base, draft_probs=None, draft_onehot=np.ones(B, dtype=np.uint8),
                              proposed=np.where(prop >= 0, prop, 0).astype(np.int32),
                              num_draft=nd.astype(np.int32), name="ngram_then_verify")
    d = inputs_to_device(inp, DEV)
    acc, tok, prb = specdec_verify(d["logits"], None, d["proposed"], d["temperature"],
                                   d["uniforms"], draft_onehot=d["draft_onehot"],
                                   num_draft=d["num_draft"])
    torch.cuda.synchronize()
    ref = oracle.verify(inp)
    rep = compare(inp, ref, acc.cpu().numpy(), tok.cpu().numpy(), prb.cpu().numpy())
    print("[report]", {k: v for k, v in rep.items() if k != "details"}, flush=True)
    assert rep["mismatch"] == 0 and rep["prob_mismatch"] == 0, rep["details"]
