"""The seeded input generators: determinism and the structure each workload promises."""
import numpy as np

from speculative_decoding_verification_specdec_amd.inputs import (BF16_NAN_BITS, PAD_ID_OFFSET,
                                                                   batch64, bf16_bits_to_f32,
                                                                   large_batch_deep, ragged_mixed,
                                                                   single_sequence, tiny_vocab)


def _same(a, b):
    for f in ("logits", "draft_probs", "draft_onehot", "proposed", "num_draft", "temperature",
              "uniforms"):
        x, y = getattr(a, f), getattr(b, f)
        assert (x is None) == (y is None), f
        if x is not None:
            assert np.array_equal(x, y, equal_nan=(x.dtype.kind == "f")), f


def test_generators_are_deterministic():
    _same(batch64(B=4, V=1000, seed=3), batch64(B=4, V=1000, seed=3))
    _same(ragged_mixed(B=8, V=500, seed=5), ragged_mixed(B=8, V=500, seed=5))
    a, b = batch64(B=4, V=1000, seed=3), batch64(B=4, V=1000, seed=4)
    assert not np.array_equal(a.logits, b.logits)


def test_shapes_and_dtypes():
    t = tiny_vocab(rounds=100)
    assert t.logits.shape == (100, 5, 32) and t.logits.dtype == np.float32
    assert (t.logits == t.logits[0]).all()                    # fixed rows, replicated
    s = single_sequence()
    assert s.logits.shape == (1, 5, 32000) and s.temperature[0] == np.float32(0.7)
    b = batch64(B=8, V=1000)
    assert b.logits.dtype == np.uint16 and b.draft_probs.shape == (8, 5, 1000)
    assert ((b.temperature >= 0.5) & (b.temperature <= 1.2)).all()
    np.testing.assert_allclose(b.draft_probs.astype(np.float64).sum(-1), 1.0, atol=1e-5)
    assert ((b.proposed >= 0) & (b.proposed < 1000)).all()


def test_large_batch_greedy_rows_and_boost():
    d = large_batch_deep(B=16, V=3000, K=8)
    greedy = d.temperature == 0
    assert greedy.sum() == 4 and (d.temperature[~greedy] == 1.0).all()
    z = bf16_bits_to_f32(d.logits).astype(np.float64)
    assert abs(z.mean() - 0.08) < 0.03                       # 1% of entries boosted by +8


def test_ragged_padding_is_garbage():
    r = ragged_mixed(B=32, V=777, K=8)
    kb = r.num_draft
    assert ((kb >= 1) & (kb <= 8)).all()
    assert r.draft_onehot.sum() == 16
    for b in range(r.B):
        k = kb[b]
        assert (r.logits[b, k + 1:] == BF16_NAN_BITS).all()
        assert (r.proposed[b, k:] == 777 + PAD_ID_OFFSET).all()
        assert (r.uniforms[b, k:8] > 1).all()
        assert np.isnan(r.draft_probs[b, k:]).all()
        if r.draft_onehot[b]:
            assert np.isnan(r.draft_probs[b]).all()
