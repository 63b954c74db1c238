"""GPU parity: every C-ABI call against the fp64 oracle, stage by stage, on the
tensors that stage consumed.  Floating point: max-abs 1e-4 on the fp32
workload, 2e-2 on bf16 workloads (fp32 outputs); RoPE bf16 outputs within the
fp32 arithmetic error plus half a bf16 ulp; block selection bit-exact."""
import math

import numpy as np
import pytest
import torch

import joint_video_audio_rope_amd as J
from oracle import attention as A
from oracle import block_sparse as B
from oracle import rope as R
from synth import WORKLOADS, joint_inputs, n_tokens, shrink, sparse_inputs

import oracle_pool as OP

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL_BF16 = 2e-2
TOL_FP32 = 1e-4


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def tol(w):
    return TOL_FP32 if w["dtype"] == "fp32" else TOL_BF16


def rope_bf16_bound(src_f64, ref_f64):
    """Largest |got - ref| a correct fp32 rotation rounded to bf16 can show.

    fp32 table entries are within 2^-25 of cos and sin; the two products and
    the sum add at most 2^-23 (|x0| + |x1|); so the fp32 result is within
    e = 2^-22 (|x0| + |x1|) of the exact rotation, and rounding it to bf16
    adds half a bf16 ulp at magnitude |ref| + e.  (One bf16 ulp of the
    result alone is not a valid gate: where x0 cos - x1 sin cancels, the fp32
    error of the terms is many ulps of the tiny result.)
    """
    pair = np.abs(src_f64[..., 0::2]) + np.abs(src_f64[..., 1::2])
    e = np.repeat(pair, 2, axis=-1) * 2.0 ** -22
    mag = np.abs(ref_f64) + e
    ulp = np.where(mag > 0, 2.0 ** (np.floor(np.log2(np.maximum(mag, 1e-300))) - 7), 0.0)
    return 0.5 * ulp + e


def bf16_ulp_diff(got_bf16, ref_f64):
    """Distance in bf16 units of the last place between got and RNE(ref)."""
    ref = torch.from_numpy(ref_f64).to(torch.float32).to(torch.bfloat16)
    def ordered(t):
        b = t.contiguous().view(torch.int16).to(torch.int32)
        mag = b & 0x7FFF
        return torch.where(b < 0, -mag, mag)
    return (ordered(got_bf16.cpu()) - ordered(ref)).abs().max().item()


def sample_rows(n, count, seed, must=()):
    rng = np.random.default_rng(seed)
    rows = set(int(r) for r in must if 0 <= r < n)
    rows.update(int(r) for r in rng.choice(n, size=min(n, count), replace=False))
    return np.array(sorted(rows))


def rotated(w):
    """Inputs of a workload with Q and K rotated on the GPU (and the originals)."""
    x = joint_inputs(w, DEV)
    q, k = x["q"].clone(), x["k"].clone()
    J.mmdit_rope3d(J.rope_spec_for(w), q, k)
    torch.cuda.synchronize()
    return x, q, k


# ---- RoPE ----------------------------------------------------------------------
@pytest.mark.parametrize("name", ["tiny", "block", "480p", "720p"])
def test_rope_parity(name):
    w = WORKLOADS[name]
    x, q, k = rotated(w)
    pos, rot = R.token_positions(w)
    n = n_tokens(w)
    rows = np.arange(n)
    for src, got in ((x["q"], q), (x["k"], k)):
        ref = R.apply_rope(f64(src[rows]), pos[rows], rot[rows], w["split"], w["theta"])
        g = got[rows]
        if w["dtype"] == "fp32":
            assert np.max(np.abs(f64(g) - ref)) <= TOL_FP32
        else:
            bound = rope_bf16_bound(f64(src[rows]), ref)
            excess = np.abs(f64(g) - ref) - bound
            assert np.max(excess) <= 0.0, (np.max(excess), bf16_ulp_diff(g, ref))
        # text tokens are neither rotated nor touched
        text = ~rot[rows]
        if text.any():
            assert torch.equal(g[torch.from_numpy(text).to(DEV)], src[rows][torch.from_numpy(text).to(DEV)])


# ---- joint self-attention ---------------------------------------------------------
def protocol_rows(w, x, n, seed):
    """Query rows to check: every row on the fp32, 5850-token and 480p-latent
    workloads; on the 720p-latent workload every outlier row plus a seeded 5 %
    of the others (the outliers carry the extreme logits)."""
    if not x["outliers"].numel():
        return None
    out = np.sort(x["outliers"].cpu().numpy())
    rest = np.setdiff1d(np.arange(n), out)
    rng = np.random.default_rng(seed)
    pick = rng.choice(rest, size=int(round(0.05 * rest.size)), replace=False)
    return np.unique(np.concatenate([out, pick, [0, n - 1]]))


@pytest.mark.parametrize("name", ["tiny", "block", "480p", "720p"])
def test_joint_attn_parity(name):
    w = WORKLOADS[name]
    x, q, k = rotated(w)
    v = x["v"]
    o = J.mmdit_joint_attn(q, k, v)
    torch.cuda.synchronize()
    n = n_tokens(w)
    r = protocol_rows(w, x, n, 2)
    ref = OP.attention_rows(OP.as_f32(q), OP.as_f32(k), OP.as_f32(v), rows=r)
    got = f64(o) if r is None else f64(o)[r]
    err = np.max(np.abs(got - ref))
    print("%s joint: %d rows x %d heads, max-abs %.3e" % (name, ref.shape[0], ref.shape[1], err), flush=True)
    assert err <= tol(w), err


def test_video_to_text_parity():
    """Every video query of the 480p-latent layer (34320, unrotated) against
    the 512 text keys."""
    w = WORKLOADS["480p"]
    x = joint_inputs(w, DEV)
    seg = A.joint_segments(w)
    v0, v1 = seg["video_stream"]
    t0, t1 = seg["text"]
    qv = x["q"][v0:v1].contiguous()
    kt, vt = x["k"][t0:t1].contiguous(), x["v"][t0:t1].contiguous()
    o = J.mmdit_joint_attn(qv, kt, vt)
    torch.cuda.synchronize()
    ref = OP.attention_rows(OP.as_f32(qv), OP.as_f32(kt), OP.as_f32(vt))
    err = np.max(np.abs(f64(o) - ref))
    print("video->text: %d rows, max-abs %.3e" % (ref.shape[0], err), flush=True)
    assert err <= TOL_BF16


# ---- audio <-> video cross-attention ---------------------------------------------------
@pytest.mark.parametrize("name", ["tiny", "block", "480p", "720p"])
def test_av_cross_attn_parity(name):
    """Every audio query; every video query, except on the 720p-latent layer:
    there every outlier video query plus a seeded 5 % of the others."""
    w = WORKLOADS[name]
    x, q, k = rotated(w)
    v = x["v"]
    seg = A.joint_segments(w)
    v0, v1 = seg["video_stream"]
    a0, a1 = seg["audio"]
    parts = [t[s0:s1].contiguous() for t in (q, k, v) for (s0, s1) in ((v0, v1), (a0, a1))]
    qv, qa, kv, ka, vv, va = parts
    o_v, o_a = J.mmdit_av_cross_attn(qv, kv, vv, qa, ka, va)
    torch.cuda.synchronize()
    nv = v1 - v0
    r = protocol_rows(w, x, n_tokens(w), 4)
    if r is not None:
        r = r[r < nv]
    ref_v = OP.attention_rows(OP.as_f32(qv), OP.as_f32(ka), OP.as_f32(va), rows=r)
    ref_a = OP.attention_rows(OP.as_f32(qa), OP.as_f32(kv), OP.as_f32(vv))
    ev = np.max(np.abs((f64(o_v) if r is None else f64(o_v)[r]) - ref_v))
    ea = np.max(np.abs(f64(o_a) - ref_a))
    print("%s video->audio: %d rows, max-abs %.3e; audio->video: %d rows, max-abs %.3e" % (
        name, ref_v.shape[0], ev, ref_a.shape[0], ea), flush=True)
    assert ev <= tol(w) and ea <= tol(w)


def test_dense_at_block_sparse_shape():
    """The dense call at the block-sparse comparison's shape (172032 video
    tokens, 24 heads, the launch the bench times against the sparse call):
    seeded query rows, the first and last of the grid and of several tiles,
    against the oracle over all keys."""
    w = WORKLOADS["sparse2k"]
    x = sparse_inputs(w, DEV)
    o = J.mmdit_joint_attn(x["q"], x["k"], x["v"])
    torch.cuda.synchronize()
    n = x["q"].shape[0]
    r = sample_rows(n, 192, 7, must=[0, 1, 63, 64, 255, 256, n // 2, n - 257, n - 256, n - 1])
    ref = OP.attention_rows(OP.as_f32(x["q"]), OP.as_f32(x["k"]), OP.as_f32(x["v"]), rows=r)
    err = np.max(np.abs(f64(o[torch.from_numpy(r).to(DEV)]) - ref))
    print("dense at 172032 tokens: %d rows x 24 heads, max-abs %.3e" % (len(r), err), flush=True)
    assert err <= TOL_BF16


# ---- edge cases of the dense kernel ---------------------------------------------------
def _rand(shape, seed, dtype=torch.bfloat16, scale=1.0):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return (torch.randn(shape, generator=g, device=DEV) * scale).to(dtype)


@pytest.mark.parametrize("nq,nkv,h,d", [(1000, 333, 3, 128), (77, 5000, 2, 128), (130, 65, 5, 64),
                                        (1, 1, 1, 128), (300, 64, 2, 64), (129, 4097, 1, 128)])
def test_ragged_and_split_shapes(nq, nkv, h, d):
    q, k, v = _rand((nq, h, d), 10), _rand((nkv, h, d), 11), _rand((nkv, h, d), 12)
    o = J.mmdit_joint_attn(q, k, v)
    torch.cuda.synchronize()
    ref = A.attention(f64(q), f64(k), f64(v))
    assert np.max(np.abs(f64(o) - ref)) <= TOL_BF16


@pytest.mark.parametrize("nq,nkv,h", [(127, 1024, 2), (129, 1025, 2), (128, 1023, 3), (385, 512, 2), (10, 1024, 2)])
def test_short_key_boundary_with_lse(nq, nkv, h):
    """Key sets of at most 1024 keys run in 128-query workgroups, longer ones in
    256-query workgroups; (10, 1024) also splits the keys across workgroups."""
    from oracle import attention_bwd as AB
    q, k, v = _rand((nq, h, 128), 20), _rand((nkv, h, 128), 21), _rand((nkv, h, 128), 22)
    o, lse = J.mmdit_joint_attn_fwd(q, k, v)
    torch.cuda.synchronize()
    o_ref, lse_ref = AB.attention_fwd_lse(f64(q), f64(k), f64(v))
    assert np.max(np.abs(f64(o) - o_ref)) <= TOL_BF16
    assert np.max(np.abs(f64(lse) - lse_ref)) <= 2e-3


def test_single_key_and_empty_queries():
    q, k, v = _rand((200, 2, 128), 13), _rand((1, 2, 128), 14), _rand((1, 2, 128), 15)
    o = J.mmdit_joint_attn(q, k, v)
    torch.cuda.synchronize()
    assert np.max(np.abs(f64(o) - f64(v)[0][None])) <= 1e-3
    e = J.mmdit_joint_attn(q[:0], k, v)
    assert e.shape == (0, 2, 128)


def test_large_logits_softmax_range():
    q, k, v = _rand((500, 2, 128), 16, scale=6.0), _rand((700, 2, 128), 17, scale=6.0), _rand((700, 2, 128), 18)
    o = J.mmdit_joint_attn(q, k, v)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all()
    assert np.max(np.abs(f64(o) - A.attention(f64(q), f64(k), f64(v)))) <= TOL_BF16


def test_repeat_is_bitwise_identical():
    w = WORKLOADS["block"]
    x = joint_inputs(w, DEV)
    a = J.mmdit_joint_attn(x["q"], x["k"], x["v"])
    b = J.mmdit_joint_attn(x["q"], x["k"], x["v"])
    c1, c2 = J.mmdit_av_cross_attn(x["q"][:5376].contiguous(), x["k"][:5376].contiguous(),
                                   x["v"][:5376].contiguous(), x["q"][5376:5594].contiguous(),
                                   x["k"][5376:5594].contiguous(), x["v"][5376:5594].contiguous())
    d1, d2 = J.mmdit_av_cross_attn(x["q"][:5376].contiguous(), x["k"][:5376].contiguous(),
                                   x["v"][:5376].contiguous(), x["q"][5376:5594].contiguous(),
                                   x["k"][5376:5594].contiguous(), x["v"][5376:5594].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(c1, d1) and torch.equal(c2, d2)


# ---- block-sparse ---------------------------------------------------------------------
def _sparse_check(w, k_sel, p_sel, n_qblocks=None, seed=5):
    x = sparse_inputs(w, DEV)
    T, H, W = w["T"], w["H"], w["W"]
    o, mask, cnt = J.mmdit_block_sparse_attn(x["q"], x["k"], x["v"], T, H, W, w["zone"], w["block"],
                                             k_sel, p_sel)
    torch.cuda.synchronize()
    idx = B.block_token_index(T, H, W, w["zone"], w["block"])
    q64, k64 = f64(x["q"]), f64(x["k"])
    P = B.block_probs(B.block_means(q64, idx), B.block_means(k64, idx))
    m_ref, c_ref, margin = B.select_blocks(P, k_sel, p_sel)
    assert margin["cumsum"] > 1e-12 and margin["rel_gap"] > 1e-12, margin
    got_mask = mask.cpu().numpy().view(np.uint32)
    assert np.array_equal(got_mask, B.pack_mask(m_ref))
    assert np.array_equal(cnt.cpu().numpy(), c_ref)
    nb = idx.shape[0]
    h = w["heads"]
    out = f64(o)
    worst = 0.0
    if n_qblocks is None:
        v64 = f64(x["v"])
        for hd in range(h):
            ref = B.block_sparse_attention(q64, k64, v64, idx, m_ref, query_blocks=range(nb), heads=[hd])
            for (hh, i), r in ref.items():
                worst = max(worst, float(np.max(np.abs(out[idx[i], hh] - r))))
    else:
        # n_qblocks seeded query blocks per head, always with the rows of the
        # largest and the smallest selection; one oracle call per head in the
        # worker pool
        del q64, k64
        q32, k32, v32 = OP.as_f32(x["q"]), OP.as_f32(x["k"]), OP.as_f32(x["v"])
        calls, picks = [], []
        for hd in range(h):
            qbs = sample_rows(nb, n_qblocks, seed + hd,
                              must=[int(np.argmax(c_ref[hd])), int(np.argmin(c_ref[hd]))])
            picks.append(qbs)
            sl = np.s_[:, hd:hd + 1]
            calls.append(((q32[sl], k32[sl], v32[sl], idx, m_ref[hd:hd + 1]),
                          dict(query_blocks=[int(i) for i in qbs], heads=[0])))
        for hd, ref in enumerate(OP.starmap("oracle.block_sparse", "block_sparse_attention", calls)):
            for (_, i), r in ref.items():
                worst = max(worst, float(np.max(np.abs(out[idx[i], hd] - r))))
        print("block-sparse O: %d query blocks x %d heads, max-abs %.3e" % (len(picks[0]), h, worst), flush=True)
    assert worst <= TOL_BF16, worst
    return c_ref


@pytest.mark.parametrize("k_sel,p_sel", [(4, 0.6), (0, 0.9), (2, 0.0), (64, 0.9), (1, 1.0)])
def test_block_sparse_small_grid(k_sel, p_sel):
    w = shrink("sparse2k", T=8, H=16, W=32, heads=4)
    _sparse_check(w, k_sel, p_sel)


def test_block_sparse_non_power_of_two_blocks():
    w = shrink("sparse2k", T=8, H=8, W=24, heads=2, seed=9)
    _sparse_check(w, 3, 0.7)


def test_block_sparse_all_blocks_equals_dense():
    w = shrink("sparse2k", T=8, H=16, W=32, heads=4, seed=6)
    x = sparse_inputs(w, DEV)
    o, _, cnt = J.mmdit_block_sparse_attn(x["q"], x["k"], x["v"], 8, 16, 32, top_k=64, top_p=0.5)
    d = J.mmdit_joint_attn(x["q"], x["k"], x["v"])
    torch.cuda.synchronize()
    assert int(cnt.min()) == 64
    assert (o - d).abs().max().item() <= TOL_BF16


def test_block_sparse_full_size():
    w = WORKLOADS["sparse2k"]
    c = _sparse_check(w, w["top_k"], w["top_p"], n_qblocks=64)
    dens = c.mean() / c.shape[1]
    assert 0.05 < dens < 0.9


def test_block_sparse_maximum_blocks():
    """4096 blocks per head, the most a selection row may hold (64 per lane)."""
    w = shrink("sparse2k", T=16, H=128, W=128, heads=1, seed=9)
    c = _sparse_check(w, 32, 0.9, n_qblocks=8)
    assert c.shape == (1, 4096)


def _sparse_tie_case(w, k_sel, p_sel, twin):
    """Key blocks copied onto other key blocks give bitwise-equal block
    probabilities; the selection must take equal values in ascending block id
    (Prism page, "Metodo" section 3: top-k and top-p are prefixes of one order)."""
    x = sparse_inputs(w, DEV)
    T, H, W = w["T"], w["H"], w["W"]
    idx = B.block_token_index(T, H, W, w["zone"], w["block"])
    it = torch.as_tensor(np.asarray(idx), device=DEV)
    k = x["k"].clone()
    for dst, src in twin:
        k[it[dst]] = k[it[src]]
    o, mask, cnt = J.mmdit_block_sparse_attn(x["q"], k, x["v"], T, H, W, w["zone"], w["block"], k_sel, p_sel)
    torch.cuda.synchronize()
    q64, k64, v64 = f64(x["q"]), f64(k), f64(x["v"])
    P = B.block_probs(B.block_means(q64, idx), B.block_means(k64, idx))
    m_ref, c_ref, _ = B.select_blocks(P, k_sel, p_sel)
    assert np.array_equal(mask.cpu().numpy().view(np.uint32), B.pack_mask(m_ref))
    assert np.array_equal(cnt.cpu().numpy(), c_ref)
    ref = B.block_sparse_attention(q64, k64, v64, idx, m_ref, query_blocks=range(idx.shape[0]),
                                   heads=range(w["heads"]))
    out = f64(o)
    worst = max(float(np.max(np.abs(out[idx[i], hh] - r))) for (hh, i), r in ref.items())
    assert worst <= TOL_BF16, worst
    return c_ref


def test_block_sparse_ties_all_equal():
    # every key block equal: uniform probabilities 1/64 (exact), so top-p 0.3
    # needs 20 blocks and the first 20 ids are taken
    w = shrink("sparse2k", T=8, H=16, W=32, heads=2, seed=11)
    c = _sparse_tie_case(w, 5, 0.3, [(j, 0) for j in range(1, 64)])
    assert (c == 20).all()


def test_block_sparse_ties_twins():
    # key blocks in equal pairs: every cut can fall between twins
    w = shrink("sparse2k", T=8, H=16, W=32, heads=2, seed=12)
    _sparse_tie_case(w, 7, 0.5, [(j + 1, j) for j in range(0, 64, 2)])


def test_block_sparse_repeat_is_bitwise_identical():
    w = shrink("sparse2k", T=16, H=32, W=48, heads=3, seed=13)
    x = sparse_inputs(w, DEV)
    a = J.mmdit_block_sparse_attn(x["q"], x["k"], x["v"], 16, 32, 48)
    b = J.mmdit_block_sparse_attn(x["q"], x["k"], x["v"], 16, 32, 48)
    torch.cuda.synchronize()
    assert all(torch.equal(u, v) for u, v in zip(a, b))


def test_rope_two_conditioning_frames():
    # conditioning frames c = 0, 1 of 2 sit at t = -2, -1 (SkyReels-V4 analysis,
    # workflow step 1: references take negative temporal indices)
    w = shrink("block", T=5, H=6, W=8, n_cond_frames=2, n_audio=40, n_text=16, heads=3)
    x, q, k = rotated(w)
    pos, rot = R.token_positions(w)
    assert pos[0][0] == -2 and pos[48][0] == -1
    for src, got in ((x["q"], q), (x["k"], k)):
        ref = R.apply_rope(f64(src), pos, rot, w["split"], w["theta"])
        excess = np.abs(f64(got) - ref) - rope_bf16_bound(f64(src), ref)
        assert np.max(excess) <= 0.0


@pytest.mark.parametrize("nq,nkv,h,d", [(500, 700, 2, 128), (257, 63, 3, 64)])
def test_fp32_path_beyond_tiny(nq, nkv, h, d):
    q, k, v = (_rand(s, seed, torch.float32) for s, seed in (((nq, h, d), 20), ((nkv, h, d), 21), ((nkv, h, d), 22)))
    o = J.mmdit_joint_attn(q, k, v)
    torch.cuda.synchronize()
    assert np.max(np.abs(f64(o) - A.attention(f64(q), f64(k), f64(v)))) <= TOL_FP32


def test_explicit_softmax_scale():
    q, k, v = _rand((400, 2, 128), 23), _rand((900, 2, 128), 24), _rand((900, 2, 128), 25)
    o = J.mmdit_joint_attn(q, k, v, softmax_scale=0.05)
    torch.cuda.synchronize()
    assert np.max(np.abs(f64(o) - A.attention(f64(q), f64(k), f64(v), scale=0.05))) <= TOL_BF16


def test_block_sparse_explicit_softmax_scale():
    w = shrink("sparse2k", T=8, H=16, W=32, heads=2, seed=14)
    x = sparse_inputs(w, DEV)
    s = 0.2
    o, mask, cnt = J.mmdit_block_sparse_attn(x["q"], x["k"], x["v"], 8, 16, 32, top_k=3, top_p=0.6,
                                             softmax_scale=s)
    torch.cuda.synchronize()
    idx = B.block_token_index(8, 16, 32, w["zone"], w["block"])
    q64, k64, v64 = f64(x["q"]), f64(x["k"]), f64(x["v"])
    P = B.block_probs(B.block_means(q64, idx), B.block_means(k64, idx), scale=s)
    m_ref, c_ref, _ = B.select_blocks(P, 3, 0.6)
    assert np.array_equal(mask.cpu().numpy().view(np.uint32), B.pack_mask(m_ref))
    ref = B.block_sparse_attention(q64, k64, v64, idx, m_ref, scale=s)
    worst = max(float(np.max(np.abs(f64(o)[idx[i], hh] - r))) for (hh, i), r in ref.items())
    assert worst <= TOL_BF16, worst


# ---- more than 4096 blocks per head: selection rows over several waves ---------------
def _sparse_large(T, H, W, heads, k_sel, p_sel, n_qblocks, seed, check_heads=None):
    """Selection bit-exact on the checked heads, O on sampled query blocks of
    those heads (with the largest and smallest selections), through the
    oracle; only the checked heads' tensors come to the host."""
    w = shrink("sparse2k", T=T, H=H, W=W, heads=heads, seed=seed)
    x = sparse_inputs(w, DEV)
    o, mask, cnt = J.mmdit_block_sparse_attn(x["q"], x["k"], x["v"], T, H, W, w["zone"], w["block"], k_sel, p_sel)
    torch.cuda.synchronize()
    hs = list(range(heads)) if check_heads is None else check_heads
    idx = B.block_token_index(T, H, W, w["zone"], w["block"])
    nb = idx.shape[0]
    sel = torch.tensor(hs, device=DEV)
    q32, k32, v32 = (x[t].index_select(1, sel).float().cpu().numpy() for t in ("q", "k", "v"))
    del x
    P = B.block_probs(B.block_means(q32, idx), B.block_means(k32, idx))
    m_ref, c_ref, margin = B.select_blocks(P, k_sel, p_sel)
    del P
    assert margin["cumsum"] > 1e-12 and margin["rel_gap"] > 1e-12, margin
    got = mask.index_select(0, sel).cpu().numpy().view(np.uint32)
    assert np.array_equal(got, B.pack_mask(m_ref))
    assert np.array_equal(cnt.index_select(0, sel).cpu().numpy(), c_ref)
    calls = []
    for hi in range(len(hs)):
        qbs = sample_rows(nb, n_qblocks, seed + hi, must=[int(np.argmax(c_ref[hi])), int(np.argmin(c_ref[hi]))])
        sl = np.s_[:, hi:hi + 1]
        calls.append(((q32[sl], k32[sl], v32[sl], idx, m_ref[hi:hi + 1]), dict(query_blocks=[int(i) for i in qbs],
                                                                              heads=[0])))
    out = o.index_select(1, sel)
    worst = 0.0
    for hi, ref in enumerate(OP.starmap("oracle.block_sparse", "block_sparse_attention", calls)):
        for (_, i), r in ref.items():
            rows = torch.from_numpy(idx[i]).to(DEV)
            worst = max(worst, float(np.max(np.abs(out[rows, hi].double().cpu().numpy() - r))))
    dens = float(c_ref.mean()) / nb
    print("%d x %d x %d (%d tokens, %d blocks/head): selection of %d heads bit-exact, density %.3f, "
          "O max-abs %.3e on %d query blocks per head" % (T, H, W, T * H * W, nb, len(hs), dens, worst,
                                                          len(calls[0][1]["query_blocks"])), flush=True)
    assert worst <= TOL_BF16, worst
    return c_ref


def test_block_sparse_8192_blocks():
    """8192 blocks per head: each selection row held by two waves."""
    _sparse_large(16, 128, 256, 2, 32, 0.9, 24, 31)


def test_block_sparse_million_tokens():
    """32 x 128 x 256 = 1048576 tokens, 16384 blocks per head, 24 heads (rows
    over four waves; the block logits computed and selected in chunks of
    query blocks): selection of two heads bit-exact, O on sampled query
    blocks of those heads."""
    _sparse_large(32, 128, 256, 24, 32, 0.9, 16, 32, check_heads=[0, 23])


def test_block_sparse_eight_wave_rows():
    """24 x 176 x 256 = 1081344 tokens, 16896 blocks per head: rows over eight waves."""
    _sparse_large(24, 176, 256, 1, 32, 0.9, 16, 33)


def test_block_sparse_ties_across_waves():
    """Every key block equal (K constant) on an 8192-block grid: the
    probabilities are exactly 2^-13, top-p 0.7 needs 5735 blocks, so the cut
    falls in the second wave of each row and the ids below it in the first
    wave must be counted (ties go to the lower id)."""
    T, H, W = 16, 128, 256
    w = shrink("sparse2k", T=T, H=H, W=W, heads=1, seed=34)
    x = sparse_inputs(w, DEV)
    k = x["k"][:1].expand_as(x["k"]).contiguous()
    o, mask, cnt = J.mmdit_block_sparse_attn(x["q"], k, x["v"], T, H, W, top_k=5, top_p=0.7)
    torch.cuda.synchronize()
    assert (cnt == 5735).all()
    m = mask.cpu().numpy().view(np.uint32)
    want = np.zeros_like(m[0, 0])
    bits = np.zeros(8192, dtype=bool)
    bits[:5735] = True
    want = np.packbits(bits.reshape(-1, 32)[:, ::-1], axis=1).view(">u4").astype(np.uint32).reshape(-1)
    assert (m == want[None, None, :]).all()
