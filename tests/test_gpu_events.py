"""The measurement events of specdec_verify_ex: the pair around the streaming kernel and the pair
around the kernels after it (accept scan, draw sums, pick) are both recorded, in that order, on
every draw grid: fine, one resident round (pick inside the draw kernel) and split (pick kernel
last)."""
import ctypes
import pathlib
import sys

import pytest
import torch

import oracle
from oracle.parity import compare
from speculative_decoding_verification_specdec_amd import (SPECDEC_PATH_STREAMING,
                                                           inputs_to_device, specdec_verify)
from speculative_decoding_verification_specdec_amd import inputs as gen

sys.path.insert(0, str(pathlib.Path(__file__).resolve().parents[1]))
from bench import HipEvents  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


# Draw grids (B x chunks of 8192): fine (16 x 3 <= 256), one resident round (64 x 5 <= 1536, the
# pick inside the draw kernel), split (200 x 9 > 1536, the pick kernel last).
@pytest.mark.parametrize("B,V", [(16, 20008), (64, 40000), (200, 70000)])
def test_both_event_pairs_are_recorded_in_order(B, V):
    inp = gen.make_batch(B, 4, V, seed=81, onehot_frac=0.25)
    print(f"\n[case] events B={B} V={V}", flush=True)
    d = inputs_to_device(inp, DEV)
    hot, drw = HipEvents(1), HipEvents(1)
    acc, tok, prb = specdec_verify(d["logits"], d["draft_probs"], d["proposed"], d["temperature"],
                                   d["uniforms"], draft_onehot=d["draft_onehot"],
                                   hot_events=hot.pairs[0], draw_events=drw.pairs[0],
                                   path=SPECDEC_PATH_STREAMING)
    torch.cuda.synchronize()
    ms = ctypes.c_float()
    stream_ms, draw_ms = hot.elapsed_ms(0), drw.elapsed_ms(0)
    assert stream_ms > 0.0 and draw_ms > 0.0
    # The draw chain starts after the streaming kernel has ended.
    assert hot.hip.hipEventElapsedTime(ctypes.byref(ms), hot.pairs[0][1], drw.pairs[0][0]) == 0
    assert ms.value >= 0.0
    hot.close()
    drw.close()
    rep = compare(inp, oracle.verify(inp), acc.cpu().numpy(), tok.cpu().numpy(),
                  prb.cpu().numpy())
    assert rep["mismatch"] == 0, rep["details"]
