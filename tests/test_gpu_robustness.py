"""Range and stream robustness of the bf16 attention calls.

V range.  The P V products run on fp16 matrix cores.  Each head's V is staged
as fp16 after a power-of-two prescale that puts its largest magnitude in
[2^14, 2^15), so no valid bf16 V overflows (|v| >= 65504 would become inf in a
plain conversion) and tiny V keeps its bits; O is scaled back exactly.  The
oracle sees the same bf16 V.  O is linear in V, so the bar is the usual 2e-2
scaled by each head's V scale.

Side streams.  A call given `stream=` while another stream is current takes
its outputs and workspace on that stream, so the caching allocator cannot
hand the workspace to other work before the call's kernels are done: a
buffer allocated and overwritten on the current stream right after the call,
while the side stream is still busy, must not change the result.
"""
import numpy as np
import pytest
import torch

import joint_video_audio_rope_amd as J
from oracle import attention as A
from oracle import block_sparse as B
from synth import normal_tensors, shrink, sparse_inputs, upstream_grad

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL_BF16 = 2e-2


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def scaled_v(shape, seed, head_scales):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    v = torch.randn(shape, generator=g, device=DEV)
    return (v * torch.tensor(head_scales, device=DEV)[None, :, None]).to(torch.bfloat16)


# head scales: beyond fp16's range, below its normal range, both in one call,
# and a head of zeros next to a huge one
SCALES = [(1e5, 3e4), (1e-6, 2e-5), (7e4, 1e-30), (0.0, 2e5)]


@pytest.mark.parametrize("scales", SCALES)
def test_joint_attn_v_range(scales):
    nq, nk, d = 300, 700, 128
    q, k = normal_tensors([(nq, 2, d), (nk, 2, d)], seed=61, device=DEV)
    v = scaled_v((nk, 2, d), 62, scales)
    o = J.mmdit_joint_attn(q, k, v)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all()
    ref = A.attention(f64(q), f64(k), f64(v))
    for hd, sc in enumerate(scales):
        err = np.max(np.abs(f64(o)[:, hd] - ref[:, hd]))
        print("head scale %.0e: max-abs %.3e" % (sc, err), flush=True)
        assert err <= TOL_BF16 * max(sc, 1e-300) or (sc == 0 and err == 0.0)


def test_audio_video_v_range():
    """Both directions; audio -> video splits the key range and merges the
    partial results, which carry the prescale already undone."""
    nv, na, d = 3000, 218, 128
    qv, kv, qa, ka = normal_tensors([(nv, 2, d), (nv, 2, d), (na, 2, d), (na, 2, d)], seed=63, device=DEV)
    vv = scaled_v((nv, 2, d), 64, (2e5, 1e-7))
    va = scaled_v((na, 2, d), 65, (1e-7, 2e5))
    o_v, o_a = J.mmdit_av_cross_attn(qv, kv, vv, qa, ka, va)
    torch.cuda.synchronize()
    ref_v = A.attention(f64(qv), f64(ka), f64(va))
    ref_a = A.attention(f64(qa), f64(kv), f64(vv))
    for hd, (sv, sa) in enumerate(((1e-7, 2e5), (2e5, 1e-7))):
        assert np.max(np.abs(f64(o_v)[:, hd] - ref_v[:, hd])) <= TOL_BF16 * sv
        assert np.max(np.abs(f64(o_a)[:, hd] - ref_a[:, hd])) <= TOL_BF16 * sa


def test_block_sparse_v_range():
    w = shrink("sparse2k", T=8, H=16, W=32, heads=2, seed=66)
    x = sparse_inputs(w, DEV)
    scales = (3e5, 1e-9)
    v = (x["v"].float() * torch.tensor(scales, device=DEV)[None, :, None]).to(torch.bfloat16)
    o, mask, _ = J.mmdit_block_sparse_attn(x["q"], x["k"], v, 8, 16, 32, top_k=3, top_p=0.7)
    torch.cuda.synchronize()
    idx = B.block_token_index(8, 16, 32)
    q64, k64, v64 = f64(x["q"]), f64(x["k"]), f64(v)
    m_ref, _, _ = B.select_blocks(B.block_probs(B.block_means(q64, idx), B.block_means(k64, idx)), 3, 0.7)
    assert np.array_equal(mask.cpu().numpy().view(np.uint32), B.pack_mask(m_ref))
    ref = B.block_sparse_attention(q64, k64, v64, idx, m_ref)
    out = f64(o)
    for (hd, i), r in ref.items():
        assert np.max(np.abs(out[idx[i], hd] - r)) <= TOL_BF16 * scales[hd]


# ---- side streams -------------------------------------------------------------------
def busy(stream, ms_hint=40):
    """Queue roughly tens of milliseconds of matrix products on `stream`."""
    with torch.cuda.stream(stream):
        a = torch.randn(4096, 4096, device=DEV)
        for _ in range(ms_hint):
            a = torch.tanh(a @ a)
    return a


def scribble(nbytes, times=60):
    """Allocate on the current stream and overwrite it again and again."""
    junk = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    for i in range(times):
        junk.fill_(0xFF if i % 2 else 0x7F)
    return junk


def side_stream_case(fn, ws_bytes):
    ref = fn(None)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    keep = busy(s)
    got = fn(s)
    junk = scribble(max(ws_bytes, 1))
    torch.cuda.synchronize()
    del keep, junk
    for a, b in zip(ref, got):
        if a is not None:
            assert torch.equal(a, b)


def test_side_stream_joint_and_cross():
    q, k, v = normal_tensors([(3000, 4, 128)] * 3, seed=67, device=DEV)
    n = q.shape[0]
    ws = J.mmdit_workspace_bytes(J.MMDIT_OP_JOINT_ATTN, n, n, 4, 128, J.MMDIT_BF16)
    side_stream_case(lambda s: (J.mmdit_joint_attn(q, k, v, stream=s),), ws)
    g = normal_tensors([(3000, 4, 128)], seed=68, device=DEV)[0]
    o, lse = J.mmdit_joint_attn_fwd(q, k, v)
    wsb = J.mmdit_workspace_bytes(J.MMDIT_OP_JOINT_ATTN_BWD, n, n, 4, 128, J.MMDIT_BF16)
    side_stream_case(lambda s: J.mmdit_joint_attn_bwd(q, k, v, o, lse, g, stream=s), wsb)
    qa, ka, va = q[:218].contiguous(), k[:218].contiguous(), v[:218].contiguous()
    wsa = J.mmdit_workspace_bytes(J.MMDIT_OP_AV_CROSS_ATTN, n, 218, 4, 128, J.MMDIT_BF16)
    side_stream_case(lambda s: J.mmdit_av_cross_attn(q, k, v, qa, ka, va, stream=s), wsa)


def test_side_stream_block_sparse():
    w = shrink("sparse2k", T=8, H=32, W=32, heads=3, seed=69)
    x = sparse_inputs(w, DEV)
    n = x["q"].shape[0]
    sd = J.sparse_desc()
    ws = J.mmdit_workspace_bytes(J.MMDIT_OP_BLOCK_SPARSE_ATTN, n, n, 3, 128, J.MMDIT_BF16, sd)
    args = (x["q"], x["k"], x["v"], 8, 32, 32)
    side_stream_case(lambda s: J.mmdit_block_sparse_attn(*args, top_k=4, top_p=0.8, stream=s), ws)
    o, lse, mask, _ = J.mmdit_block_sparse_attn_fwd(*args, top_k=4, top_p=0.8)
    g = normal_tensors([(n, 3, 128)], seed=70, device=DEV)[0]
    wsb = J.mmdit_workspace_bytes(J.MMDIT_OP_BLOCK_SPARSE_ATTN_BWD, n, n, 3, 128, J.MMDIT_BF16, sd)
    side_stream_case(lambda s: J.mmdit_block_sparse_attn_bwd(x["q"], x["k"], x["v"], o, lse, g, mask, 8, 32, 32,
                                                             stream=s), wsb)
    wsa = J.mmdit_workspace_bytes(J.MMDIT_OP_BLOCK_SPARSE_ATTN_ADAPTIVE, n, 0, 3, 128, J.MMDIT_BF16)
    side_stream_case(lambda s: tuple(J.mmdit_block_sparse_attn_adaptive(*args, top_k=4, top_p=0.8,
                                                                        stream=s).values()), wsa)
