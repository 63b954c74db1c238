"""mmdit_joint_attn_noalloc, the joint attention for callers that cannot
allocate, called through the C ABI: its output must equal mmdit_joint_attn's
(the same kernels on the same inputs, with the workspace in the library's
fixed per-GPU scratch instead of a caller buffer) bit for bit, on calls in a
row whose sizes shrink (a later call must not see an earlier call's scratch
contents), including a shape whose key range is split across workgroups
(partial results in the scratch).  Sizes beyond the scratch are rejected
before anything is enqueued, leaving the output untouched."""
import ctypes

import numpy as np
import pytest
import torch

import joint_video_audio_rope_amd as J
import joint_video_audio_rope_amd._lib as L
from oracle import attention as A
from synth import normal_tensors

pytestmark = pytest.mark.gpu
DEV = "cuda"


def noalloc(q, k, v, o):
    n_q, h, d = q.shape
    lib = J.lib()
    st = lib.mmdit_joint_attn_noalloc(
        ctypes.c_void_p(q.data_ptr()), n_q, ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(v.data_ptr()),
        k.shape[0], h, d, L.MMDIT_BF16 if q.dtype == torch.bfloat16 else L.MMDIT_FP32, 0.0,
        ctypes.c_void_p(o.data_ptr()), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st


# the 5850-token joint block (24 x 128); audio-like queries against a long key
# range (split keys, partials in the scratch); then a smaller call
CASES = [(5850, 5850, 24, 128, 71), (218, 10000, 6, 128, 72), (700, 300, 3, 64, 73)]


def test_noalloc_matches_workspace_call_on_shrinking_calls():
    for n_q, n_kv, h, d, seed in CASES:
        q, k, v = normal_tensors([(n_q, h, d), (n_kv, h, d), (n_kv, h, d)], seed=seed, device=DEV)
        ref = J.mmdit_joint_attn(q, k, v)
        o = torch.full((n_q, h, d), float("nan"), device=DEV)
        assert noalloc(q, k, v, o) == L.MMDIT_OK, J.mmdit_last_error()
        torch.cuda.synchronize()
        print("n_q %d, n_kv %d, %d x %d: equal %s" % (n_q, n_kv, h, d, torch.equal(o, ref)), flush=True)
        assert torch.equal(o, ref)
    # the last (smallest) call against the oracle as well
    err = np.max(np.abs(o.double().cpu().numpy() - A.attention(*(t.double().cpu().numpy() for t in (q, k, v)))))
    assert err <= 2e-2, err


def test_noalloc_rejects_sizes_beyond_the_scratch():
    n, h, d = 11000, 24, 128     # V^T alone needs 24 * 128 * 11008 * 2 bytes > 64 MiB
    q, k, v = normal_tensors([(8, h, d), (n, h, d), (n, h, d)], seed=74, device=DEV)
    o = torch.full((8, h, d), 3.0, device=DEV)
    assert noalloc(q, k, v, o) == L.MMDIT_ERR_WORKSPACE
    assert "scratch" in J.mmdit_last_error()
    torch.cuda.synchronize()
    assert torch.all(o == 3.0)
