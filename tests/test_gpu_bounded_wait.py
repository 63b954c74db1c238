"""The block-sparse attention's waits are bounded.  With the bound forced to
zero from the host (MMDIT_SPARSE_SPIN_LIMIT=0), every wait that is not
satisfied at once gives up and marks its workgroup broken.  The call must
still end (its attention values may then be wrong), the selection, which
waits on nothing, must be unchanged, and the next call with the normal bound
must reproduce the earlier bits: the library keeps no state between calls."""
import pytest
import torch

import joint_video_audio_rope_amd as J
from synth import shrink, sparse_inputs

pytestmark = pytest.mark.gpu


def test_forced_give_up_ends_and_leaves_no_state(monkeypatch):
    w = shrink("sparse2k", T=8, H=32, W=32, heads=2, seed=51)
    x = sparse_inputs(w, "cuda")
    args = (x["q"], x["k"], x["v"], w["T"], w["H"], w["W"], w["zone"], w["block"], 4, 0.8)
    ref = J.mmdit_block_sparse_attn(*args)
    torch.cuda.synchronize()
    monkeypatch.setenv("MMDIT_SPARSE_SPIN_LIMIT", "0")
    forced = J.mmdit_block_sparse_attn(*args)
    torch.cuda.synchronize()
    print("forced give-up: max |o - o_ref| = %.3g" % (forced[0] - ref[0]).abs().nan_to_num(1e30).max().item(),
          flush=True)
    assert torch.equal(forced[1], ref[1]) and torch.equal(forced[2], ref[2])
    monkeypatch.delenv("MMDIT_SPARSE_SPIN_LIMIT")
    again = J.mmdit_block_sparse_attn(*args)
    torch.cuda.synchronize()
    for a, b in zip(again, ref):
        assert torch.equal(a, b)
