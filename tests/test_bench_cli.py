"""bench.py's command line on the CPU: more than one GPU is refused with a message, before any
device work (the verify step shards by sequence with no communication; one GPU shows its
per-GPU kernel)."""
import os
import pathlib
import subprocess
import sys

ROOT = pathlib.Path(__file__).resolve().parents[1]


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"], cwd=str(ROOT),
                       capture_output=True, text=True, timeout=300,
                       env=dict(os.environ, HIP_VISIBLE_DEVICES=""))
    assert r.returncode != 0
    assert "--gpus 1" in r.stderr
    assert r.stdout.strip() == ""


def _bench_module():
    sys.path.insert(0, str(ROOT))
    import bench
    return bench


def test_median_and_spread():
    bench = _bench_module()
    m, rep = bench._median_and_spread([40.0, 37.0, 38.0, 39.0, 37.5])
    assert m == 38.0
    assert rep["repeats_us"] == [40.0, 37.0, 38.0, 39.0, 37.5]
    assert abs(rep["spread_pct"] - 3.0 / 38.0 * 100.0) < 1e-12


def test_algorithmic_bytes_bounds():
    # The algorithmic byte model on a tiny batch, worked by hand: B = 2, K = 2, V = 10, fp32 logits;
    # sequence 0 a model draft (rejected at slot 1), sequence 1 one-hot (all accepted).
    import numpy as np

    from speculative_decoding_verification_specdec_amd import inputs as gen
    bench = _bench_module()
    inp = gen.make_batch(2, 2, 10, seed=5, dtype="f32")
    inp.draft_onehot = np.array([0, 1], np.uint8)
    acc = np.array([1, 2], np.int32)
    logits, actual = bench.algorithmic_bytes(inp, acc)
    _, upper = bench.algorithmic_bytes(inp, acc, all_rejected=True)
    assert logits == 2 * 3 * 10 * 4
    per_seq = 4 * 2 + 4 * 3 + 4 + 8 * 3 + 4               # ids, u, T, outputs
    small = 2 * per_seq + 4 * 2                           # + q gathers of the model draft
    assert actual == logits + small + 4 * 10              # one draft row (sequence 0)
    assert upper == actual                                # one-hot rows read no draft row
    inp.draft_onehot = None
    _, actual2 = bench.algorithmic_bytes(inp, acc)
    _, upper2 = bench.algorithmic_bytes(inp, acc, all_rejected=True)
    assert upper2 - actual2 == 4 * 10                     # sequence 1 rejected in the bound
