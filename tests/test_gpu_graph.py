"""The library's calls under HIP graph capture.

Every call enqueues only kernels on the caller's stream (no memset, copy,
allocation or synchronisation inside the library), so a step of the hot path
can be captured once and replayed.  The test captures the joint attention,
both cross-attention directions, the block-sparse attention and the
content-adaptive block-sparse attention into one graph, replays it several
times with the program's own eager work and synchronisations in between, and
requires every replay to reproduce the eager results bit for bit."""
import pytest
import torch

import joint_video_audio_rope_amd as J
from synth import WORKLOADS, adaptive_inputs, joint_inputs, shrink, sparse_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def test_graph_replays_match_eager():
    w = WORKLOADS["block"]
    x = joint_inputs(w, DEV)
    q, k, v = x["q"], x["k"], x["v"]
    n, h, d = q.shape
    nv = w["T"] * w["H"] * w["W"]
    qv, kv, vv = q[:nv], k[:nv], v[:nv]
    qa, ka, va = (t[nv:nv + w["n_audio"]] for t in (q, k, v))
    ws_s = shrink("sparse2k", T=8, H=16, W=32, heads=2, seed=31)
    xs = sparse_inputs(ws_s, DEV)
    wa = shrink("adaptive2k", T=8, H=32, W=32, heads=2, fg_radius=8.0, seed=32)
    xa = adaptive_inputs(wa, DEV)

    f32 = dict(dtype=torch.float32, device=DEV)
    o = torch.empty((n, h, d), **f32)
    o_va = torch.empty((nv, h, d), **f32)
    o_av = torch.empty((w["n_audio"], h, d), **f32)
    ws_j = torch.empty(J.mmdit_workspace_bytes(J.MMDIT_OP_JOINT_ATTN, n, n, h, d, J.MMDIT_BF16),
                       dtype=torch.uint8, device=DEV)
    ws_x = torch.empty(J.mmdit_workspace_bytes(J.MMDIT_OP_AV_CROSS_ATTN, nv, w["n_audio"], h, d, J.MMDIT_BF16),
                       dtype=torch.uint8, device=DEV)
    ns = 8 * 16 * 32
    o_s = torch.empty((ns, 2, 128), **f32)
    mask = torch.empty((2, ns // 64, (ns // 64 + 31) // 32), dtype=torch.int32, device=DEV)
    cnt = torch.empty((2, ns // 64), dtype=torch.int32, device=DEV)
    sd = J.sparse_desc(ws_s["zone"], ws_s["block"], 3, 0.8)
    ws_sp = torch.empty(J.mmdit_workspace_bytes(J.MMDIT_OP_BLOCK_SPARSE_ATTN, ns, ns, 2, 128, J.MMDIT_BF16, sd),
                        dtype=torch.uint8, device=DEV)
    na = 8 * 32 * 32
    o_a = torch.empty((na, 2, 128), **f32)
    ws_ad = torch.empty(J.mmdit_workspace_bytes(J.MMDIT_OP_BLOCK_SPARSE_ATTN_ADAPTIVE, na, 0, 2, 128, J.MMDIT_BF16),
                        dtype=torch.uint8, device=DEV)
    ad = {}

    def step():
        J.mmdit_joint_attn(q, k, v, o=o, ws=ws_j)
        J.mmdit_av_cross_attn(qv, kv, vv, qa, ka, va, o_video=o_va, o_audio=o_av, ws=ws_x)
        J.mmdit_block_sparse_attn(xs["q"], xs["k"], xs["v"], 8, 16, 32, ws_s["zone"], ws_s["block"], 3, 0.8,
                                  o=o_s, sel_mask=mask, sel_count=cnt, ws=ws_sp)
        ad.update(J.mmdit_block_sparse_attn_adaptive(xa["q"], xa["k"], xa["v"], 8, 32, 32, a_norm=xa["a"],
                                                     top_k=4, top_p=0.8, o=o_a, ws=ws_ad))

    side = torch.cuda.Stream()            # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                            # eager reference (also the warm-up torch asks for)
    torch.cuda.synchronize()
    want = [t.clone() for t in (o, o_va, o_av, o_s, mask, cnt, o_a)]
    want_shape = ad["zone_shape"].clone()
    want_mask = ad["sel_mask"].clone()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        step()
    for rep in range(3):
        for t in (o, o_va, o_av, o_s, o_a):
            t.fill_(float("nan"))          # eager work between replays
        mask.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (o, o_va, o_av, o_s, mask, cnt, o_a)
        for i, (a, b) in enumerate(zip(got, want)):
            assert torch.equal(a, b), (rep, i)
        assert torch.equal(ad["zone_shape"], want_shape) and torch.equal(ad["sel_mask"], want_mask), rep


def test_two_streams_match_one():
    """Independent calls on two streams at once (separate workspaces) give the
    same bits as the same calls one after the other: the library keeps no
    state between calls."""
    w = WORKLOADS["block"]
    x = joint_inputs(w, DEV)
    q, k, v = x["q"], x["k"], x["v"]
    n, h, d = q.shape
    ws_s = shrink("sparse2k", T=8, H=32, W=32, heads=4, seed=33)
    xs = sparse_inputs(ws_s, DEV)
    seq_o = J.mmdit_joint_attn(q, k, v)
    seq_s, seq_m, seq_c = J.mmdit_block_sparse_attn(xs["q"], xs["k"], xs["v"], 8, 32, 32, top_k=4, top_p=0.8)
    torch.cuda.synchronize()
    a, b = torch.cuda.Stream(), torch.cuda.Stream()   # default priority
    a.wait_stream(torch.cuda.current_stream())
    b.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(3):
        with torch.cuda.stream(a):
            o = J.mmdit_joint_attn(q, k, v)
        with torch.cuda.stream(b):
            s, m, c = J.mmdit_block_sparse_attn(xs["q"], xs["k"], xs["v"], 8, 32, 32, top_k=4, top_p=0.8)
        outs.append((o, s, m, c))
    torch.cuda.synchronize()
    for o, s, m, c in outs:
        assert torch.equal(o, seq_o) and torch.equal(s, seq_s) and torch.equal(m, seq_m) and torch.equal(c, seq_c)
