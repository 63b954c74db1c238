"""The block-sparse attention's internal waits are bounded, and a wait that
gives up is loud.  With the bound lowered from the host to one sleep
(mmdit_sparse_desc.wait_limit = 1), waits that are not satisfied at once give
up, so the producer/consumer protocol of the attention kernel breaks.  Every
kernel still ends normally.  The test checks:
  * the call returns, and the selection (which waits on nothing) is unchanged;
  * every o row a broken workgroup wrote is NaN in full, with a NaN
    log-sum-exp, and at least one row is so marked;
  * every row that is not NaN equals the normal call's row bit for bit (a
    wave that finishes before any give-up computed on intact tiles);
  * the normal bound marks nothing, and the next normal call reproduces the
    earlier bits: the library keeps no state between calls."""
import pytest
import torch

import joint_video_audio_rope_amd as J
from synth import shrink, sparse_inputs

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("limit", [1, 200])
def test_forced_give_up_marks_its_rows_and_leaves_no_state(limit):
    """limit 1: practically every wait gives up; limit 200 (~6 us): some may."""
    w = shrink("sparse2k", T=8, H=32, W=32, heads=2, seed=51)
    x = sparse_inputs(w, "cuda")
    args = (x["q"], x["k"], x["v"], w["T"], w["H"], w["W"], w["zone"], w["block"], 4, 0.8)
    ref = J.mmdit_block_sparse_attn_fwd(*args)
    torch.cuda.synchronize()
    assert not torch.isnan(ref[0]).any() and not torch.isnan(ref[1]).any()
    forced = J.mmdit_block_sparse_attn_fwd(*args, wait_limit=limit)
    torch.cuda.synchronize()
    o, lse = forced[0], forced[1]
    bad = torch.isnan(o).any(dim=-1)                     # [n, heads]
    print("wait limit %d: %d of %d (token, head) rows marked" % (limit, int(bad.sum()), bad.numel()), flush=True)
    if limit == 1:
        assert bad.any()
    assert torch.isnan(o[bad]).all()
    assert torch.equal(torch.isnan(lse), bad.t())
    assert torch.equal(o[~bad], ref[0][~bad])
    assert torch.equal(lse[~bad.t()], ref[1][~bad.t()])
    assert torch.equal(forced[2], ref[2]) and torch.equal(forced[3], ref[3])
    again = J.mmdit_block_sparse_attn_fwd(*args)
    torch.cuda.synchronize()
    for a, b in zip(again, ref):
        assert torch.equal(a, b)
