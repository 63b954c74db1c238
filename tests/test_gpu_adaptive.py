"""GPU parity of the content-adaptive block-sparse attention and of the token
norms against the fp64 oracle (oracle/adaptive_blocks.py, oracle/block_sparse.py).

Bars: zone shape codes, block numbering, the tile-level selection bitmask and
the per-row block counts bit-exact (both sides decide in fp64); o max-abs 2e-2
(bf16 products, fp32 accumulation), lse 2e-3; token norms relative 1e-5
(fp32 sums)."""
import numpy as np
import pytest
import torch

import joint_video_audio_rope_amd as J
from oracle import adaptive_blocks as A
from oracle import attention_bwd as AB
from oracle import block_sparse as B
from synth import WORKLOADS, adaptive_inputs, normal_tensors, shrink

import grad_bounds as GB

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL_O, TOL_LSE = 2e-2, 2e-3


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def expected_tile_blocks(codes):
    """Block id of each 64-token tile: a zone of volume-B blocks holds
    512 / B blocks of B / 64 consecutive tiles."""
    out, nb = [], 0
    for c in codes:
        per = int(np.prod(A.candidate_shapes()[c])) // 64
        out += [nb + u // per for u in range(8)]
        nb += 8 // per
    return np.array(out), nb


def unpack_rows(words, nt):
    """[h, rows, ceil(nt/32)] int32 words -> [h, rows, nt] bool."""
    w = words.cpu().numpy().view(np.uint32)
    bits = (w[..., :, None] >> np.arange(32, dtype=np.uint32)) & 1
    return bits.reshape(w.shape[0], w.shape[1], -1)[:, :, :nt].astype(bool)


def run(x, T, H, W, k_sel, p_sel, use_a=True):
    return J.mmdit_block_sparse_attn_adaptive(x["q"], x["k"], x["v"], T, H, W, a_norm=x["a"] if use_a else None,
                                              top_k=k_sel, top_p=p_sel, want_lse=True)


def full_check(w, k_sel, p_sel, use_a=True, x=None):
    T, H, W = w["T"], w["H"], w["W"]
    if x is None:
        x = adaptive_inputs(w, DEV)
    r = run(x, T, H, W, k_sel, p_sel, use_a)
    torch.cuda.synchronize()
    q64, k64, v64 = f64(x["q"]), f64(x["k"]), f64(x["v"])
    a64 = f64(x["a"]) if use_a else None
    codes, ind = A.zone_shapes(v64, a64, T, H, W)
    got_codes = r["zone_shape"].cpu().numpy().astype(np.int64)
    print("volumes", np.bincount(ind["volume"], minlength=257)[[64, 128, 256]], "codes", np.bincount(codes, minlength=16),
          flush=True)
    np.testing.assert_array_equal(got_codes, codes)
    tb, nb = expected_tile_blocks(codes)
    np.testing.assert_array_equal(r["tile_block"].cpu().numpy(), tb)
    assert int(r["n_blocks"].item()) == nb
    blocks, _ = A.adaptive_block_tokens(T, H, W, codes)
    P = B.block_probs(A.ragged_means(q64, blocks), A.ragged_means(k64, blocks))
    m_ref, c_ref, margin = B.select_blocks(P, k_sel, p_sel)
    print("selection margins", margin, flush=True)
    nt = len(tb)
    want = m_ref[:, tb][:, :, tb]
    np.testing.assert_array_equal(unpack_rows(r["sel_mask"], nt), want)
    np.testing.assert_array_equal(r["sel_count"].cpu().numpy(), c_ref[:, tb])
    blk = np.empty(T * H * W, dtype=np.int64)
    for j, b in enumerate(blocks):
        blk[b] = j
    allowed = m_ref[:, blk][:, :, blk]
    o_ref, lse_ref = AB.attention_fwd_lse(q64, k64, v64, allowed=allowed)
    err_o = float(np.max(np.abs(f64(r["o"]) - o_ref)))
    err_l = float(np.max(np.abs(f64(r["lse"]) - lse_ref)))
    print("o max-abs %.3e, lse max-abs %.3e" % (err_o, err_l), flush=True)
    assert err_o <= TOL_O and err_l <= TOL_LSE
    return codes, ind, c_ref


@pytest.mark.parametrize("k_sel,p_sel", [(4, 0.8), (1, 0.3), (8, 0.95)])
def test_adaptive_small_grid(k_sel, p_sel):
    w = shrink("adaptive2k", T=8, H=32, W=32, heads=2, fg_radius=8.0, audio_radius=5.0, seed=11)
    codes, ind, _ = full_check(w, k_sel, p_sel)
    assert len(set(ind["volume"].tolist())) >= 2


def test_adaptive_without_audio_and_two_frames_of_zones():
    w = shrink("adaptive2k", T=16, H=16, W=32, heads=3, fg_radius=6.0, audio_radius=4.0, seed=12)
    full_check(w, 3, 0.7, use_a=False)


def test_adaptive_constant_values_give_256_blocks():
    w = shrink("adaptive2k", T=8, H=16, W=32, heads=2, seed=13)
    x = adaptive_inputs(w, DEV)
    x["v"] = torch.full_like(x["v"], 0.5)
    codes, ind, _ = full_check(w, 2, 0.6, x=x)
    assert np.all(ind["volume"] == 256) and np.all(codes == 13)


def test_adaptive_all_blocks_equals_dense():
    w = shrink("adaptive2k", T=8, H=16, W=32, heads=2, fg_radius=5.0, seed=14)
    x = adaptive_inputs(w, DEV)
    r = run(x, 8, 16, 32, 1000, 1.0)
    torch.cuda.synchronize()
    o_ref, lse_ref = AB.attention_fwd_lse(f64(x["q"]), f64(x["k"]), f64(x["v"]))
    assert float(np.max(np.abs(f64(r["o"]) - o_ref))) <= TOL_O
    assert float(np.max(np.abs(f64(r["lse"]) - lse_ref))) <= TOL_LSE
    assert torch.all(r["sel_count"] == r["n_blocks"])


def test_adaptive_repeat_is_bitwise_identical():
    w = shrink("adaptive2k", T=8, H=32, W=32, heads=2, fg_radius=8.0, seed=15)
    x = adaptive_inputs(w, DEV)
    a, b = run(x, 8, 32, 32, 4, 0.8), run(x, 8, 32, 32, 4, 0.8)
    for key in ("o", "lse", "zone_shape", "tile_block", "sel_mask", "sel_count"):
        assert torch.equal(a[key], b[key]), key


def test_adaptive_full_size_sampled():
    """The full 24 x 64 x 112 grid (336 zones, 24 heads): every zone's shape
    code from the oracle, the selection rows and o of sampled query blocks of
    two heads against the oracle over their selected keys."""
    w = WORKLOADS["adaptive2k"]
    T, H, W = w["T"], w["H"], w["W"]
    x = adaptive_inputs(w, DEV)
    r = run(x, T, H, W, w["top_k"], w["top_p"])
    torch.cuda.synchronize()
    codes, ind = A.zone_shapes(f64(x["v"]), f64(x["a"]), T, H, W)
    print("volumes", np.bincount(ind["volume"], minlength=257)[[64, 128, 256]], flush=True)
    np.testing.assert_array_equal(r["zone_shape"].cpu().numpy().astype(np.int64), codes)
    tb, nb = expected_tile_blocks(codes)
    np.testing.assert_array_equal(r["tile_block"].cpu().numpy(), tb)
    blocks, _ = A.adaptive_block_tokens(T, H, W, codes)
    heads = [0, 23]
    q64, k64, v64 = (f64(t[:, heads]) for t in (x["q"], x["k"], x["v"]))
    P = B.block_probs(A.ragged_means(q64, blocks), A.ragged_means(k64, blocks))
    m_ref, c_ref, _ = B.select_blocks(P, w["top_k"], w["top_p"])
    nt = len(tb)
    rows = unpack_rows(r["sel_mask"][heads], nt)
    np.testing.assert_array_equal(rows, m_ref[:, tb][:, :, tb])
    rng = np.random.default_rng(1)
    sample = np.unique(np.concatenate([[0, nb - 1], rng.choice(nb, 5, replace=False)]))
    out = A.ragged_sparse_attention(q64, k64, v64, blocks, m_ref, query_blocks=sample)
    o64 = f64(r["o"][:, heads])
    err = max(float(np.max(np.abs(o64[blocks[i], hi] - o))) for (hi, i), o in out.items())
    print("sampled o max-abs %.3e" % err, flush=True)
    assert err <= TOL_O


def test_adaptive_512_zones():
    """512 zones (4096 tiles per head, the most one selection wave holds):
    every zone's code, the whole tile bitmask, o of sampled query blocks."""
    w = shrink("adaptive2k", T=16, H=128, W=128, heads=1, fg_radius=30.0, audio_radius=15.0, seed=16)
    T, H, W = w["T"], w["H"], w["W"]
    x = adaptive_inputs(w, DEV)
    r = run(x, T, H, W, 16, 0.8)
    torch.cuda.synchronize()
    q64, k64, v64 = f64(x["q"]), f64(x["k"]), f64(x["v"])
    codes, ind = A.zone_shapes(v64, f64(x["a"]), T, H, W)
    assert len(codes) == 512 and len(set(ind["volume"].tolist())) == 3
    np.testing.assert_array_equal(r["zone_shape"].cpu().numpy().astype(np.int64), codes)
    tb, nb = expected_tile_blocks(codes)
    np.testing.assert_array_equal(r["tile_block"].cpu().numpy(), tb)
    blocks, _ = A.adaptive_block_tokens(T, H, W, codes)
    P = B.block_probs(A.ragged_means(q64, blocks), A.ragged_means(k64, blocks))
    m_ref, c_ref, _ = B.select_blocks(P, 16, 0.8)
    np.testing.assert_array_equal(unpack_rows(r["sel_mask"], len(tb)), m_ref[:, tb][:, :, tb])
    np.testing.assert_array_equal(r["sel_count"].cpu().numpy(), c_ref[:, tb])
    rng = np.random.default_rng(3)
    sample = np.unique(np.concatenate([[0, nb - 1], rng.choice(nb, 4, replace=False)]))
    out = A.ragged_sparse_attention(q64, k64, v64, blocks, m_ref, query_blocks=sample)
    o64 = f64(r["o"])
    err = max(float(np.max(np.abs(o64[blocks[i], hi] - o))) for (hi, i), o in out.items())
    assert err <= TOL_O


def test_adaptive_zones_beyond_one_per_thread():
    """1536 zones (12288 tiles per head, 786432 tokens): more zones than the
    shape pass has threads and more tiles than one selection wave holds.
    Every zone's code, the whole tile bitmask and counts, o of sampled query
    blocks."""
    w = shrink("adaptive2k", T=24, H=128, W=256, heads=1, fg_radius=40.0, audio_radius=20.0, seed=17)
    T, H, W = w["T"], w["H"], w["W"]
    x = adaptive_inputs(w, DEV)
    r = run(x, T, H, W, 16, 0.8)
    torch.cuda.synchronize()
    q64, k64, v64 = f64(x["q"]), f64(x["k"]), f64(x["v"])
    codes, ind = A.zone_shapes(v64, f64(x["a"]), T, H, W)
    assert len(codes) == 1536 and len(set(ind["volume"].tolist())) == 3
    np.testing.assert_array_equal(r["zone_shape"].cpu().numpy().astype(np.int64), codes)
    tb, nb = expected_tile_blocks(codes)
    np.testing.assert_array_equal(r["tile_block"].cpu().numpy(), tb)
    blocks, _ = A.adaptive_block_tokens(T, H, W, codes)
    P = B.block_probs(A.ragged_means(q64, blocks), A.ragged_means(k64, blocks))
    m_ref, c_ref, _ = B.select_blocks(P, 16, 0.8)
    np.testing.assert_array_equal(unpack_rows(r["sel_mask"], len(tb)), m_ref[:, tb][:, :, tb])
    np.testing.assert_array_equal(r["sel_count"].cpu().numpy(), c_ref[:, tb])
    rng = np.random.default_rng(5)
    sample = np.unique(np.concatenate([[0, nb - 1], rng.choice(nb, 4, replace=False)]))
    out = A.ragged_sparse_attention(q64, k64, v64, blocks, m_ref, query_blocks=sample)
    o64 = f64(r["o"])
    err = max(float(np.max(np.abs(o64[blocks[i], hi] - o))) for (hi, i), o in out.items())
    print("blocks %d, sampled o max-abs %.3e" % (nb, err), flush=True)
    assert err <= TOL_O


def test_token_norms_match_oracle():
    x = normal_tensors([(1000, 24, 128)], seed=3, dtype="fp32", device=DEV)[0]
    x[17] = 0.0
    got = J.mmdit_token_norms(x)
    torch.cuda.synchronize()
    ref = A.token_norms(f64(x))
    np.testing.assert_allclose(f64(got), ref, rtol=1e-5)
    assert float(got[17]) == 0.0


def check_rel(name, got, ref, rel):
    err = float(np.max(np.abs(got - ref)))
    peak = float(np.max(np.abs(ref)))
    print("%s: max-abs %.3e, max |ref| %.3e" % (name, err, peak), flush=True)
    assert err <= rel * max(peak, 1e-30), (name, err, peak)


@pytest.mark.parametrize("k_sel,p_sel,use_a", [(4, 0.8, True), (2, 0.5, False)])
def test_adaptive_bwd_small_grid(k_sel, p_sel, use_a):
    w = shrink("adaptive2k", T=8, H=32, W=32, heads=2, fg_radius=8.0, audio_radius=5.0, seed=21)
    T, H, W = w["T"], w["H"], w["W"]
    n = T * H * W
    x = adaptive_inputs(w, DEV)
    r = run(x, T, H, W, k_sel, p_sel, use_a)
    g = normal_tensors([(n, 2, 128)], seed=5, device=DEV)[0]
    dq, dk, dv = J.mmdit_block_sparse_attn_adaptive_bwd(x["q"], x["k"], x["v"], r, g, T, H, W)
    torch.cuda.synchronize()
    q64, k64, v64, g64 = f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(g)
    codes, ind = A.zone_shapes(v64, f64(x["a"]) if use_a else None, T, H, W)
    np.testing.assert_array_equal(r["zone_shape"].cpu().numpy().astype(np.int64), codes)
    assert len(set(ind["volume"].tolist())) >= 2
    blocks, _ = A.adaptive_block_tokens(T, H, W, codes)
    P = B.block_probs(A.ragged_means(q64, blocks), A.ragged_means(k64, blocks))
    m_ref, _, _ = B.select_blocks(P, k_sel, p_sel)
    blk = np.empty(n, dtype=np.int64)
    for j, b in enumerate(blocks):
        blk[b] = j
    allowed = m_ref[:, blk][:, :, blk]
    rq, rk, rv = AB.attention_bwd(q64, k64, v64, g64, allowed=allowed)
    aq, ak, av = GB.bwd_allowances(q64, k64, v64, g64, allowed=allowed)
    GB.check("dq", f64(dq), rq, aq)
    GB.check("dk", f64(dk), rk, ak)
    GB.check("dv", f64(dv), rv, av)


def test_adaptive_bwd_repeat_is_bitwise_identical():
    w = shrink("adaptive2k", T=8, H=16, W=32, heads=2, fg_radius=5.0, seed=22)
    T, H, W = w["T"], w["H"], w["W"]
    x = adaptive_inputs(w, DEV)
    g = normal_tensors([(T * H * W, 2, 128)], seed=6, device=DEV)[0]
    r = run(x, T, H, W, 3, 0.7)
    a = J.mmdit_block_sparse_attn_adaptive_bwd(x["q"], x["k"], x["v"], r, g, T, H, W)
    b = J.mmdit_block_sparse_attn_adaptive_bwd(x["q"], x["k"], x["v"], r, g, T, H, W)
    for u, v in zip(a, b):
        assert torch.equal(u, v)


def test_adaptive_bwd_full_size_sampled():
    """The full 24 x 64 x 112 grid: dq of sampled query blocks of two heads
    against the oracle over their selected keys, and sum_j dv_j = sum_i dO_i
    for every head (every query's probabilities sum to one)."""
    w = WORKLOADS["adaptive2k"]
    T, H, W = w["T"], w["H"], w["W"]
    n, h = T * H * W, w["heads"]
    x = adaptive_inputs(w, DEV)
    r = run(x, T, H, W, w["top_k"], w["top_p"])
    g = normal_tensors([(n, h, 128)], seed=17, device=DEV)[0]
    dq, dk, dv = J.mmdit_block_sparse_attn_adaptive_bwd(x["q"], x["k"], x["v"], r, g, T, H, W)
    torch.cuda.synchronize()
    codes = r["zone_shape"].cpu().numpy().astype(np.int64)
    blocks, _ = A.adaptive_block_tokens(T, H, W, codes)
    heads = [0, 23]
    q64, k64, v64, g64 = (f64(t[:, heads]) for t in (x["q"], x["k"], x["v"], g))
    P = B.block_probs(A.ragged_means(q64, blocks), A.ragged_means(k64, blocks))
    m_ref, _, _ = B.select_blocks(P, w["top_k"], w["top_p"])
    dq64 = f64(dq[:, heads])
    rng = np.random.default_rng(2)
    nb = len(blocks)
    for hi in range(2):
        for i in np.unique(np.concatenate([[0, nb - 1], rng.choice(nb, 3, replace=False)])):
            keys = np.concatenate([blocks[j] for j in np.nonzero(m_ref[hi, i])[0]])
            qt = blocks[i]
            sl = np.s_[hi:hi + 1]
            args = (q64[qt][:, sl], k64[keys][:, sl], v64[keys][:, sl], g64[qt][:, sl])
            rq, _, _ = AB.attention_bwd(*args)
            GB.check("dq h%d b%d" % (heads[hi], i), dq64[qt, hi], rq[:, 0], GB.bwd_allowances(*args)[0][:, 0])
    sums = dv.double().sum(dim=0).cpu().numpy()
    check_rel("sum dv", sums, f64(g).sum(axis=0), 1e-3)
