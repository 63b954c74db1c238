"""GPU parity of the block-sparse training calls against the fp64 oracle.

mmdit_block_sparse_attn_fwd must reproduce the oracle's selection bit for bit
(as mmdit_block_sparse_attn does) and return the log-sum-exp over each
query's selected keys; mmdit_block_sparse_attn_bwd must give the gradients of
masked softmax attention with that selection held fixed
(oracle.attention_bwd with the token-level mask of the selected block
pairs).  Tolerances as for the dense backward: bf16 gradients entry by entry
within the allowance of grad_bounds (and max-abs 2e-2 at these unit-scale
inputs), outputs max-abs 2e-2, the log-sum-exp 2e-3."""
import numpy as np
import pytest
import torch

import joint_video_audio_rope_amd as J
from oracle import attention_bwd as AB
from oracle import block_sparse as B
from synth import WORKLOADS, normal_tensors, shrink, sparse_inputs

import grad_bounds as GB

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL_BF16, TOL_LSE = 2e-2, 2e-3


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def check(name, got, ref, tol, rel=None):
    err = float(np.max(np.abs(got - ref)))
    peak = float(np.max(np.abs(ref)))
    print("%s: max-abs %.3e, max |ref| %.3e" % (name, err, peak), flush=True)
    if rel is None:
        assert err <= tol, (name, err)
    else:   # an invariant over all keys (sum of dv): relative to its largest entry
        assert err <= rel * max(peak, 1e-30), (name, err, peak)


def token_mask(idx, m_ref):
    """[h, n, n] bool: query token i may see key token j iff j's block is
    selected by i's block."""
    nb, vol = idx.shape
    blk = np.empty(nb * vol, dtype=np.int64)
    blk[idx.reshape(-1)] = np.repeat(np.arange(nb), vol)
    return m_ref[:, blk][:, :, blk]


def run(w, k_sel, p_sel, seed):
    x = sparse_inputs(w, DEV)
    T, H, W = w["T"], w["H"], w["W"]
    n, h, d = x["q"].shape
    g = normal_tensors([(n, h, d)], seed=seed, device=DEV)[0]
    o, lse, mask, cnt = J.mmdit_block_sparse_attn_fwd(x["q"], x["k"], x["v"], T, H, W, w["zone"], w["block"],
                                                      k_sel, p_sel)
    dq, dk, dv = J.mmdit_block_sparse_attn_bwd(x["q"], x["k"], x["v"], o, lse, g, mask, T, H, W, w["zone"],
                                               w["block"])
    torch.cuda.synchronize()
    return x, g, o, lse, mask, cnt, dq, dk, dv


def full_check(w, k_sel, p_sel, seed=21):
    x, g, o, lse, mask, cnt, dq, dk, dv = run(w, k_sel, p_sel, seed)
    T, H, W = w["T"], w["H"], w["W"]
    idx = B.block_token_index(T, H, W, w["zone"], w["block"])
    q64, k64, v64, g64 = f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(g)
    P = B.block_probs(B.block_means(q64, idx), B.block_means(k64, idx))
    m_ref, c_ref, _ = B.select_blocks(P, k_sel, p_sel)
    assert np.array_equal(mask.cpu().numpy().view(np.uint32), B.pack_mask(m_ref))
    assert np.array_equal(cnt.cpu().numpy(), c_ref)
    allowed = token_mask(idx, m_ref)
    o_ref, lse_ref = AB.attention_fwd_lse(q64, k64, v64, allowed=allowed)
    check("o", f64(o), o_ref, TOL_BF16)
    check("lse", f64(lse), lse_ref, TOL_LSE)
    rq, rk, rv = AB.attention_bwd(q64, k64, v64, g64, allowed=allowed)
    aq, ak, av = GB.bwd_allowances(q64, k64, v64, g64, allowed=allowed)
    GB.check("dq", f64(dq), rq, aq)
    GB.check("dk", f64(dk), rk, ak)
    GB.check("dv", f64(dv), rv, av)
    return c_ref


@pytest.mark.parametrize("k_sel,p_sel", [(3, 0.8), (1, 0.3), (6, 0.95)])
def test_sparse_bwd_small_grid(k_sel, p_sel):
    full_check(shrink("sparse2k", T=8, H=16, W=16, heads=2), k_sel, p_sel)


def test_sparse_bwd_partial_last_group():
    # zones of one block: 10 blocks, so the last workgroup of 4 blocks holds 2
    w = shrink("sparse2k", T=4, H=8, W=20, heads=3, zone=(4, 4, 4), seed=13)
    full_check(w, 2, 0.6)


def test_sparse_bwd_all_blocks_equals_dense():
    w = shrink("sparse2k", T=8, H=16, W=16, heads=2, seed=7)
    c = full_check(w, 32, 1.0)
    assert (c == 32).all()


def test_sparse_bwd_repeat_is_bitwise_identical():
    w = shrink("sparse2k", T=8, H=16, W=32, heads=2, seed=8)
    a = run(w, 4, 0.7, 3)
    b = run(w, 4, 0.7, 3)
    for i in (6, 7, 8):
        assert torch.equal(a[i], b[i])


def test_sparse_bwd_full_size_sampled():
    """The full sparse2k grid (172032 tokens, 24 heads): the selection rows of
    two heads from the oracle, dq of sampled query blocks against the oracle
    over their selected keys, and sum_j dv_j = sum_i dO_i over every head."""
    w = WORKLOADS["sparse2k"]
    x, g, o, lse, mask, cnt, dq, dk, dv = run(w, w["top_k"], w["top_p"], 17)
    T, H, W = w["T"], w["H"], w["W"]
    idx = B.block_token_index(T, H, W, w["zone"], w["block"])
    nb = idx.shape[0]
    heads = [0, 23]
    q64, k64, v64, g64 = (f64(t[:, heads]) for t in (x["q"], x["k"], x["v"], g))
    P = B.block_probs(B.block_means(q64, idx), B.block_means(k64, idx))
    m_ref, c_ref, _ = B.select_blocks(P, w["top_k"], w["top_p"])
    got = mask.cpu().numpy().view(np.uint32)[heads]
    assert np.array_equal(got, B.pack_mask(m_ref))
    rng = np.random.default_rng(0)
    dq64, lse64 = f64(dq[:, heads]), f64(lse[heads])
    for hi in range(len(heads)):
        blocks = np.unique(np.concatenate([[0, nb - 1, int(np.argmax(c_ref[hi])), int(np.argmin(c_ref[hi]))],
                                           rng.choice(nb, 4, replace=False)]))
        for i in blocks:
            keys = idx[np.nonzero(m_ref[hi, i])[0]].reshape(-1)
            qt = idx[i]
            sl = np.s_[hi:hi + 1]
            _, lse_ref = AB.attention_fwd_lse(q64[qt][:, sl], k64[keys][:, sl], v64[keys][:, sl])
            rq, _, _ = AB.attention_bwd(q64[qt][:, sl], k64[keys][:, sl], v64[keys][:, sl], g64[qt][:, sl])
            check("lse h%d b%d" % (heads[hi], i), lse64[hi, qt], lse_ref[0], TOL_LSE)
            aq = GB.bwd_allowances(q64[qt][:, sl], k64[keys][:, sl], v64[keys][:, sl], g64[qt][:, sl])[0]
            GB.check("dq h%d b%d" % (heads[hi], i), dq64[qt, hi], rq[:, 0], aq[:, 0])
    sums = dv.double().sum(dim=0).cpu().numpy()
    check("sum dv", sums, f64(g).sum(axis=0), 0.5, 1e-3)
