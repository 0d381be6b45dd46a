"""GPU parity on seeded random shapes: batch size, draft length, vocabulary (both sides of the
small-vocabulary limit), dtype and row mix drawn per case, each compared with the oracle on the
default path and, for V <= SPECDEC_SMALL_V_MAX, on the streaming kernels too; every other case
also through the sample-and-match entry point and, the others, through the greedy entry point
(every row at temperature 0, bit-exact).  Same bar as the other parity tests (oracle/parity.py).
A second family of seeded shapes has draw grids past one resident round (the split passes),
mostly with one-hot rows.  The n-gram drafter gets its own seeded random shapes (bit-exact
against its oracle)."""
import numpy as np
import pytest
import torch

import oracle
from oracle.parity import boundary_limit, compare, expected_boundary
from speculative_decoding_verification_specdec_amd import (SPECDEC_PATH_AUTO,
                                                           SPECDEC_PATH_STREAMING,
                                                           SPECDEC_SMALL_V_MAX, inputs_to_device,
                                                           specdec_verify)
from speculative_decoding_verification_specdec_amd import inputs as gen

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
N_CASES = 64


def case(seed):
    g = np.random.default_rng(1000 + seed)
    V = int(g.choice([int(g.integers(1, 70)), int(g.integers(70, 1025)),
                      int(g.integers(1025, 30000))]))
    K = int(g.integers(0, 13))
    B = int(g.integers(1, max(2, min(200, 3_000_000 // ((K + 1) * V)))))
    return gen.make_batch(B, K, V, seed=2000 + seed, dtype=str(g.choice(["bf16", "f32"])),
                          greedy_frac=float(g.choice([0.0, 0.2, 1.0])),
                          onehot_frac=float(g.choice([0.0, 0.3])),
                          ragged=K > 0 and bool(g.integers(0, 2)),
                          draft_at_row_temp=bool(g.integers(0, 2)),
                          draft_sigma=float(g.choice([0.2, 1.5])))


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_shape_parity(seed):
    inp = case(seed)
    ref = oracle.verify(inp)
    paths = [SPECDEC_PATH_AUTO] + ([SPECDEC_PATH_STREAMING] if inp.V <= SPECDEC_SMALL_V_MAX else [])
    for path in paths:
        print(f"\n[case] seed={seed} B={inp.B} K={inp.K} V={inp.V} {inp.logits_dtype} path={path}",
              flush=True)
        d = inputs_to_device(inp, DEV)
        acc, tok, prb = specdec_verify(d["logits"], d["draft_probs"], d["proposed"],
                                       d["temperature"], d["uniforms"],
                                       draft_onehot=d["draft_onehot"], num_draft=d["num_draft"],
                                       path=path)
        torch.cuda.synchronize()
        rep = compare(inp, ref, acc.cpu().numpy(), tok.cpu().numpy(), prb.cpu().numpy())
        print("[report]", {k: v for k, v in rep.items() if k != "details"}, flush=True)
        assert rep["mismatch"] == 0, rep["details"]
        limit = boundary_limit(expected_boundary(inp, ref))
        assert rep["boundary"] <= limit, (rep, limit)


def split_case(seed):
    # Draw grids past one resident round (B x chunks > 1536): the scan pass, the draw-only pass
    # and the pick kernel; mostly one-hot rows, whose residual sums come from the partials outside
    # the rejected draft's segment.
    g = np.random.default_rng(5000 + seed)
    B = int(g.choice([128, 256, 512]))
    K = int(g.integers(1, 5))
    s_min = 1536 // B + 1
    V = int(g.integers(max(8192 * (s_min - 1) + 1, 12000), 8192 * (s_min + 3)))
    if g.integers(0, 2):
        V -= V % 8
    return gen.make_batch(B, K, V, seed=6000 + seed, dtype=str(g.choice(["bf16", "f32"])),
                          onehot_frac=float(g.choice([0.5, 0.9, 1.0])),
                          greedy_frac=float(g.choice([0.0, 0.1])), ragged=bool(g.integers(0, 2)))


@pytest.mark.parametrize("seed", range(8))
def test_random_split_grid_parity(seed):
    inp = split_case(seed)
    assert inp.B * ((inp.V + 8191) // 8192) > 1536
    print(f"\n[case] split seed={seed} B={inp.B} K={inp.K} V={inp.V} {inp.logits_dtype}",
          flush=True)
    ref = oracle.verify(inp)
    d = inputs_to_device(inp, DEV)
    acc, tok, prb = specdec_verify(d["logits"], d["draft_probs"], d["proposed"], d["temperature"],
                                   d["uniforms"], draft_onehot=d["draft_onehot"],
                                   num_draft=d["num_draft"])
    torch.cuda.synchronize()
    rep = compare(inp, ref, acc.cpu().numpy(), tok.cpu().numpy(), prb.cpu().numpy())
    print("[report]", {k: v for k, v in rep.items() if k != "details"}, flush=True)
    assert rep["mismatch"] == 0, rep["details"]
    limit = boundary_limit(expected_boundary(inp, ref))
    assert rep["boundary"] <= limit, (rep, limit)


@pytest.mark.parametrize("seed", range(0, N_CASES, 2))
def test_random_shape_match_mode_parity(seed):
    # The same shapes through the sample-and-match entry point (no draft distribution).
    from speculative_decoding_verification_specdec_amd import specdec_verify_match
    inp = case(seed)
    ref = oracle.verify_match(inp)
    print(f"\n[case] match seed={seed} B={inp.B} K={inp.K} V={inp.V} {inp.logits_dtype}",
          flush=True)
    d = inputs_to_device(inp, DEV)
    acc, tok, prb = specdec_verify_match(d["logits"], d["proposed"], d["temperature"],
                                         d["uniforms"], num_draft=d["num_draft"])
    torch.cuda.synchronize()
    rep = compare(inp, ref, acc.cpu().numpy(), tok.cpu().numpy(), prb.cpu().numpy(), mode="match")
    print("[report]", {k: v for k, v in rep.items() if k != "details"}, flush=True)
    assert rep["mismatch"] == 0, rep["details"]
    limit = boundary_limit(expected_boundary(inp, ref, mode="match"))
    assert rep["boundary"] <= limit, (rep, limit)


@pytest.mark.parametrize("seed", range(1, N_CASES, 2))
def test_random_shape_greedy_entry_point(seed):
    # The same shapes through specdec_verify_greedy: every row at temperature 0, bit-exact.
    from speculative_decoding_verification_specdec_amd import specdec_verify_greedy
    inp = case(seed)
    inp.temperature[:] = 0.0
    ref = oracle.verify(inp)
    print(f"\n[case] greedy seed={seed} B={inp.B} K={inp.K} V={inp.V} {inp.logits_dtype}",
          flush=True)
    d = inputs_to_device(inp, DEV)
    acc, tok, prb = specdec_verify_greedy(d["logits"], d["proposed"], num_draft=d["num_draft"])
    torch.cuda.synchronize()
    rep = compare(inp, ref, acc.cpu().numpy(), tok.cpu().numpy(), prb.cpu().numpy())
    assert rep["mismatch"] == 0 and rep["boundary"] == 0, rep


@pytest.mark.parametrize("seed", range(32))
def test_random_shape_ngram_drafter(seed):
    # N-gram drafter on seeded random shapes: history capacity (one tile or several, aligned for
    # 16-byte loads or not), token vocabulary, n range and draft length; bit-exact.
    from speculative_decoding_verification_specdec_amd import contexts as hist
    from speculative_decoding_verification_specdec_amd import specdec_ngram_propose
    g = np.random.default_rng(3000 + seed)
    cap = int(g.choice([int(g.integers(1, 600)), int(g.integers(600, 9000)),
                        int(g.integers(9000, 40000))]))
    B = int(g.integers(1, max(2, min(96, 1_000_000 // cap))))
    vocab = int(g.choice([3, 20, 500, 30000]))
    n_min = int(g.integers(1, 4))
    n_max = int(g.integers(n_min, 33))
    K = int(g.integers(0, 17))
    h = hist.make_histories(B, cap, vocab, seed=4000 + seed, len_range=(0, cap),
                            seg_range=(1, 16), edge_cases=True, name=f"random{seed}")
    print(f"\n[case] ngram seed={seed} B={B} cap={cap} vocab={vocab} K={K} n={n_min}..{n_max}",
          flush=True)
    t = torch.from_numpy(h.tokens).to(DEV)
    ln = torch.from_numpy(h.lengths).to(DEV)
    prop, nd = specdec_ngram_propose(t, ln, K, n_min=n_min, n_max=n_max)
    torch.cuda.synchronize()
    ref_p, ref_n = oracle.ngram_propose(h.tokens, h.lengths, n_min, n_max, K)
    assert np.array_equal(nd.cpu().numpy(), ref_n)
    assert np.array_equal(prop.cpu().numpy(), ref_p)
