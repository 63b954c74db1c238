"""The joint self-attention with its RoPE fused in (mmdit_joint_attn_rope)
against the separate calls and the fp64 oracle.

The fused call rotates K in the pass that stages V and Q in registers as the
attention kernel loads it.  Its rotated tensors must be bit for bit those of
mmdit_rope3d, and its output bit for bit that of mmdit_joint_attn on them:
the same arithmetic in the same order.  Stage by stage against the oracle
(the parity protocol of the unfused calls): the rotated Q and K within the
derived fp32 + half-ulp bound of the oracle's rotation, and O within 2e-2 of
the oracle's attention on exactly the rotated tensors the call used.  The
end-to-end distance to the oracle's fp64 rotation and attention is printed,
not gated (it includes the bf16 rounding of the rotated Q and K)."""
import numpy as np
import pytest
import torch

import joint_video_audio_rope_amd as J
from oracle import rope as R
from synth import WORKLOADS, joint_inputs, n_tokens, shrink

import oracle_pool as OP
from test_gpu_parity import rope_bf16_bound, sample_rows

pytestmark = pytest.mark.gpu
DEV = "cuda"


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


CASES = [
    ("block", None),                                  # 5850 tokens, all rows
    ("480p", 3072),                                   # 35050 tokens incl. the cond frame at t = -1
    ("small_split", None),                            # few query tiles: key range split, partials merged
    ("two_cond", None),                               # two conditioning frames at t = -2, -1
]


def workload(name):
    if name == "small_split":   # 600 tokens, 3 heads: 15 query tiles, so the keys split in two
        return shrink("block", T=2, H=16, W=16, n_audio=50, n_text=38, heads=3, audio_scale=(2, 50))
    if name == "two_cond":
        return shrink("block", T=3, H=8, W=8, n_cond_frames=2, n_audio=30, n_text=20, heads=2, input_scale=1.0,
                      audio_scale=(3, 30))
    return WORKLOADS[name]


@pytest.mark.parametrize("name,rows", CASES)
def test_fused_rope_matches_separate_calls_and_oracle(name, rows):
    w = workload(name)
    x = joint_inputs(w, DEV)
    spec = J.rope_spec_for(w)
    o, q_rot, k_rot = J.mmdit_joint_attn_rope(spec, x["q"], x["k"], x["v"])
    q2, k2 = x["q"].clone(), x["k"].clone()
    J.mmdit_rope3d(spec, q2, k2)
    o2 = J.mmdit_joint_attn(q2, k2, x["v"])
    torch.cuda.synchronize()
    assert torch.equal(q_rot, q2) and torch.equal(k_rot, k2)
    assert torch.equal(o, o2)
    # the unrotated inputs are left as they were
    x0 = joint_inputs(w, DEV)
    assert torch.equal(x["q"], x0["q"]) and torch.equal(x["k"], x0["k"])

    n = n_tokens(w)
    r = np.arange(n) if rows is None else sample_rows(n, rows, 9, must=[0, n - 1])
    pos, rot = R.token_positions(w)
    for src, got in ((x["q"], q_rot), (x["k"], k_rot)):
        s64 = f64(src[torch.from_numpy(r).to(DEV)])
        ref = R.apply_rope(s64, pos[r], rot[r], w["split"], w["theta"])
        assert np.max(np.abs(f64(got[torch.from_numpy(r).to(DEV)]) - ref) - rope_bf16_bound(s64, ref)) <= 0.0
    ref = OP.attention_rows(OP.as_f32(q_rot), OP.as_f32(k_rot), OP.as_f32(x["v"]), rows=r)
    err = np.max(np.abs(f64(o)[r] - ref))
    e2e = OP.attention_rows(R.apply_rope(f64(x["q"]), pos, rot, w["split"], w["theta"]).astype(np.float32),
                            R.apply_rope(f64(x["k"]), pos, rot, w["split"], w["theta"]).astype(np.float32),
                            OP.as_f32(x["v"]), rows=r)
    print("%s fused: %d rows, max-abs %.3e against the oracle on the rotated tensors, %.3e end to end" % (
        name, len(r), err, np.max(np.abs(f64(o)[r] - e2e))), flush=True)
    assert err <= 2e-2


def test_fused_rope_without_rotated_outputs():
    """q_rot and k_rot not wanted: the rotated K lives in the workspace."""
    w = workload("small_split")
    x = joint_inputs(w, DEV)
    spec = J.rope_spec_for(w)
    o, qr, kr = J.mmdit_joint_attn_rope(spec, x["q"], x["k"], x["v"], want_rotated=False)
    q2, k2 = x["q"].clone(), x["k"].clone()
    J.mmdit_rope3d(spec, q2, k2)
    o2 = J.mmdit_joint_attn(q2, k2, x["v"])
    torch.cuda.synchronize()
    assert qr is None and kr is None
    assert torch.equal(o, o2)
