"""GPU parity of the four-workgroups-per-sequence path (SPECDEC_PATH_QUAD) against the fp64 oracle.

The path streams each sequence's rows with four workgroups (a quarter of every row each) that
exchange their quarter statistics and the draw's segment sums through tagged words in the
workspace, in one launch.  It must give the oracle's results on every workload it accepts, refuse
shapes it does not take with a shape error, agree with the default path bit for bit where both
reach the same decisions, and report a sequence invalid -- never garbage -- when a bounded wait
gives up.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle.parity import compare
from speculative_decoding_verification_specdec_amd import (SPECDEC_PATH_QUAD, SPECDEC_PATH_STREAMING,
                                                           SpecdecError, inputs_to_device,
                                                           specdec_verify, specdec_workspace_size)
from speculative_decoding_verification_specdec_amd import inputs as gen

from test_gpu_parity import check  # noqa: E402  (tests/ is on sys.path under pytest)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

CASES = {
    "batch64": lambda: gen.batch64(),
    "batch64_calibrated": lambda: gen.batch64(calibrated=True),
    "large_batch_deep": lambda: gen.large_batch_deep(B=64),
    "large_batch_deep_calibrated": lambda: gen.large_batch_deep(B=48, calibrated=True),
    "ragged_mixed": lambda: gen.ragged_mixed(B=64),
    "single_sequence": lambda: gen.single_sequence(),
    "f32": lambda: gen.make_batch(16, 3, 12352, seed=40, dtype="f32"),
    "no_drafts": lambda: gen.make_batch(8, 0, 5000, seed=43),
    "all_greedy": lambda: gen.make_batch(16, 6, 9000, seed=45, greedy_frac=1.0),
    "all_onehot": lambda: gen.make_batch(16, 6, 9000, seed=46, onehot_frac=1.0),
    "bonus_everywhere": lambda: gen.make_batch(16, 5, 20008, seed=48, draft_scale=1.0,
                                               draft_sigma=0.0, draft_at_row_temp=True),
    "largest_vocab": lambda: gen.make_batch(4, 3, 262144, seed=50, draft_sigma=0.3,
                                            draft_at_row_temp=True),
    "ragged_last_quarter": lambda: gen.make_batch(12, 4, 24584, seed=52, ragged=True,
                                                  onehot_frac=0.3, greedy_frac=0.2),
    "deep_draft": lambda: gen.make_batch(6, 40, 9000, seed=54, draft_scale=1.0, draft_sigma=0.05,
                                         draft_at_row_temp=True),
}


@pytest.mark.parametrize("name", list(CASES))
def test_quad_parity(name):
    check(CASES[name](), path=SPECDEC_PATH_QUAD)


def test_quad_invalid_rows():
    inp = gen.make_batch(24, 4, 30000, seed=51, dtype="f32", onehot_frac=0.25, ragged=True)
    inp.num_draft[0] = -1
    inp.temperature[1] = np.nan
    inp.logits[2, 0, 17] = np.nan
    inp.logits[3, int(inp.num_draft[3]), 5] = np.inf
    inp.proposed[4, 0] = 30000
    check(inp, path=SPECDEC_PATH_QUAD)


@pytest.mark.parametrize("B,K,V,dtype", [(16, 3, 20003, "bf16"),   # rows not whole 8-token groups
                                         (16, 3, 12348, "f32"),
                                         (3, 3, 600000, "bf16"),   # more than 32 segments a quarter
                                         (200, 5, 8192, "bf16")])  # 800 workgroups: more than fit
def test_quad_refuses_shapes_it_does_not_take(B, K, V, dtype):
    inp = gen.make_batch(B, K, V, seed=60, dtype=dtype)
    d = inputs_to_device(inp, DEV)
    with pytest.raises(SpecdecError):
        specdec_verify(d["logits"], d["draft_probs"], d["proposed"], d["temperature"],
                       d["uniforms"], path=SPECDEC_PATH_QUAD)


def test_quad_equals_the_streaming_path_on_batch64():
    # Same decisions, same arithmetic for every emitted probability (both merge fp32 statistics
    # in a different order, so probabilities agree to the parity band, tokens and lengths exactly).
    inp = gen.batch64()
    d = inputs_to_device(inp, DEV)
    outs = []
    for path in (SPECDEC_PATH_STREAMING, SPECDEC_PATH_QUAD):
        acc, tok, prb = specdec_verify(d["logits"], d["draft_probs"], d["proposed"],
                                       d["temperature"], d["uniforms"], path=path)
        torch.cuda.synchronize()
        outs.append((acc.cpu().numpy(), tok.cpu().numpy(), prb.cpu().numpy()))
    (a0, t0, p0), (a1, t1, p1) = outs
    assert np.array_equal(a0, a1) and np.array_equal(t0, t1)
    np.testing.assert_allclose(p1, p0, rtol=1e-5, atol=0)


def test_quad_gives_up_cleanly_and_recovers():
    """With a spin limit of one poll, waits may give up: each sequence is then either reported
    invalid (accept_len -1, tokens -1, probabilities 0) or equal to the default call's result, and
    calls after it on the same workspace are exact again (their epoch differs)."""
    inp = gen.batch64(B=32, V=40000, seed=77)
    d = inputs_to_device(inp, DEV)
    ws = torch.empty(specdec_workspace_size(inp.B, inp.K, inp.V), dtype=torch.uint8, device=DEV)

    def run(limit):
        acc, tok, prb = specdec_verify(d["logits"], d["draft_probs"], d["proposed"],
                                       d["temperature"], d["uniforms"], workspace=ws,
                                       path=SPECDEC_PATH_QUAD, spin_limit=limit)
        torch.cuda.synchronize()
        return acc.cpu().numpy(), tok.cpu().numpy(), prb.cpu().numpy()

    good = run(0)
    rep = compare(inp, oracle.verify(inp), *good)
    assert rep["mismatch"] == 0, rep["details"]
    for _ in range(3):
        acc, tok, prb = run(1)
        poisoned = acc < 0
        assert (tok[poisoned] == -1).all() and (prb[poisoned] == 0).all()
        ok = ~poisoned
        assert np.array_equal(acc[ok], good[0][ok]) and np.array_equal(tok[ok], good[1][ok])
        assert np.array_equal(prb[ok].view(np.uint32), good[2][ok].view(np.uint32))
    for _ in range(2):
        again = run(0)
        for x, y in zip(again, good):
            assert np.array_equal(x.view(np.uint32) if x.dtype == np.float32 else x,
                                  y.view(np.uint32) if y.dtype == np.float32 else y)


def test_quad_workspace_left_by_the_streaming_path():
    # A workspace last used by the three-launch path (its bytes are not tagged words) and then
    # by this path: the tags reject whatever was there.
    inp = gen.batch64(B=64, seed=78)
    d = inputs_to_device(inp, DEV)
    ws = torch.empty(specdec_workspace_size(inp.B, inp.K, inp.V), dtype=torch.uint8, device=DEV)
    ref = oracle.verify(inp)
    for path in (SPECDEC_PATH_STREAMING, SPECDEC_PATH_QUAD, SPECDEC_PATH_STREAMING,
                 SPECDEC_PATH_QUAD):
        acc, tok, prb = specdec_verify(d["logits"], d["draft_probs"], d["proposed"],
                                       d["temperature"], d["uniforms"], workspace=ws, path=path)
        torch.cuda.synchronize()
        rep = compare(inp, ref, acc.cpu().numpy(), tok.cpu().numpy(), prb.cpu().numpy())
        assert rep["mismatch"] == 0, (path, rep["details"])


def quad_case(seed):
    # Seeded random shapes the path takes: V a multiple of 8 from 8 (three empty quarters) up to
    # 262144 (32 segments a quarter), K up to 63, B up to 64, both dtypes, mixed rows.
    g = np.random.default_rng(5000 + seed)
    V = 8 * int(g.choice([int(g.integers(1, 128)), int(g.integers(128, 4096)),
                          int(g.integers(4096, 32769))]))
    K = int(g.choice([int(g.integers(0, 9)), int(g.integers(9, 64))]))
    B = int(g.integers(1, max(2, min(65, 4_000_000 // ((K + 1) * V)))))
    return gen.make_batch(B, K, V, seed=6000 + seed, dtype=str(g.choice(["bf16", "f32"])),
                          greedy_frac=float(g.choice([0.0, 0.2, 1.0])),
                          onehot_frac=float(g.choice([0.0, 0.3])),
                          ragged=K > 0 and bool(g.integers(0, 2)),
                          draft_at_row_temp=bool(g.integers(0, 2)),
                          draft_sigma=float(g.choice([0.2, 1.5])))


@pytest.mark.parametrize("seed", range(24))
def test_quad_random_shapes(seed):
    check(quad_case(seed), path=SPECDEC_PATH_QUAD)
