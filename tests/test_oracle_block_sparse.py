"""Pins of the block pooling / selection / sparse-attention oracle: brute force,
hand-built probability rows, selection invariants and reduction to dense
attention (CPU only)."""
import numpy as np
import pytest

from oracle import attention as A
from oracle import block_sparse as B
from oracle import brute
from synth import WORKLOADS, shrink, sparse_inputs


def test_block_partition_and_numbering(page_constants):
    w = WORKLOADS["sparse2k"]
    assert tuple(w["zone"]) == tuple(int(s) for s in page_constants["zone"].split())
    assert int(np.prod(w["block"])) in [int(s) for s in page_constants["block_volumes"].split()]
    T, H, W = w["T"], w["H"], w["W"]
    idx = B.block_token_index(T, H, W, w["zone"], w["block"])
    assert idx.shape == (2688, 64)
    assert np.array_equal(np.sort(idx.ravel()), np.arange(T * H * W))
    t, hh, ww = idx // (H * W), (idx // W) % H, idx % W
    # every block is a 4x4x4 cube inside one 8x8x8 zone
    for a in (t, hh, ww):
        assert np.all(a.max(1) - a.min(1) == 3)
    assert np.all(t.min(1) // 8 == t.max(1) // 8)
    # id = ((zt*(H/8) + zh)*(W/8) + zw)*8 + (bt*2 + bh)*2 + bw
    t0, h0, w0 = t.min(1), hh.min(1), ww.min(1)
    j = (((t0 // 8) * (H // 8) + h0 // 8) * (W // 8) + w0 // 8) * 8 + \
        (((t0 % 8) // 4) * 2 + (h0 % 8) // 4) * 2 + (w0 % 8) // 4
    assert np.array_equal(j, np.arange(2688))


def test_blocks_match_brute_walk():
    idx = B.block_token_index(8, 16, 8, (8, 8, 8), (4, 4, 4))
    want = brute.blocks(8, 16, 8, (8, 8, 8), (4, 4, 4))
    assert [sorted(r) for r in idx.tolist()] == [sorted(r) for r in want]


def test_block_means_match_loops():
    rng = np.random.default_rng(0)
    T, H, W = 8, 8, 16
    x = rng.standard_normal((T * H * W, 2, 8))
    idx = B.block_token_index(T, H, W)
    m = B.block_means(x, idx)
    for j, toks in enumerate(brute.blocks(T, H, W, (8, 8, 8), (4, 4, 4))):
        for hd in range(2):
            want = [sum(x[t, hd, c] for t in toks) / len(toks) for c in range(8)]
            assert np.allclose(m[hd, j], want, rtol=0, atol=1e-14)


def test_hand_built_rows():
    # dyadic probabilities: running sums 1/2, 3/4, 7/8, 15/16, ... are exact
    P = np.array([[[1 / 128, 1 / 2, 1 / 8, 1 / 4, 1 / 64, 1 / 16, 1 / 128, 1 / 32]]])
    # order: 1, 3, 2, 5, 7, 4, 0, 6 (the two 1/128 go lower id first)
    m, c, _ = B.select_blocks(P, 2, 0.9)       # running 1/2, 3/4, 7/8, 15/16 -> n_p = 4
    assert c[0, 0] == 4 and set(np.flatnonzero(m[0, 0])) == {1, 3, 2, 5}
    m, c, _ = B.select_blocks(P, 6, 0.9)       # top-k longer: 6 blocks
    assert c[0, 0] == 6 and set(np.flatnonzero(m[0, 0])) == {1, 3, 2, 5, 7, 4}
    m, c, _ = B.select_blocks(P, 7, 0.5)       # tie at the cut: id 0 before id 6
    assert set(np.flatnonzero(m[0, 0])) == {1, 3, 2, 5, 7, 4, 0}
    m, c, _ = B.select_blocks(P, 0, 0.5)       # reaching p exactly counts (>=)
    assert c[0, 0] == 1 and np.flatnonzero(m[0, 0]).tolist() == [1]
    m, c, _ = B.select_blocks(P, 0, 0.0)       # never empty
    assert c[0, 0] == 1
    flat = np.full((1, 1, 4), 0.25)
    m, c, _ = B.select_blocks(flat, 1, 0.3)
    assert np.flatnonzero(m[0, 0]).tolist() == [0, 1]


def _small_sparse(T=8, H=16, W=16, seed=11, heads=2, d=32):
    w = shrink("sparse2k", T=T, H=H, W=W, heads=heads, head_dim=d, seed=seed)
    x = sparse_inputs(w, "cpu")
    return tuple([w] + [x[t].double().numpy() for t in "qkv"])


@pytest.mark.parametrize("k,p", [(0, 0.5), (3, 0.9), (2, 0.3), (40, 0.9), (1, 1.0)])
def test_selection_matches_brute(k, p):
    w, q, kk, _ = _small_sparse()
    idx = B.block_token_index(w["T"], w["H"], w["W"])
    qb, kb = B.block_means(q, idx), B.block_means(kk, idx)
    P = B.block_probs(qb, kb)
    mask, counts, _ = B.select_blocks(P, k, p)
    sc = 1 / np.sqrt(q.shape[2])
    for hd in range(2):
        for i in range(idx.shape[0]):
            pr = brute.block_probs_row(list(qb[hd, i]), [list(r) for r in kb[hd]], sc)
            assert np.allclose(P[hd, i], pr, rtol=0, atol=1e-15)
            sel = brute.select_row(list(P[hd, i]), k, p)
            assert set(np.flatnonzero(mask[hd, i])) == sel
            assert counts[hd, i] == len(sel)


def test_selection_invariants():
    w, q, kk, _ = _small_sparse(seed=12)
    idx = B.block_token_index(w["T"], w["H"], w["W"])
    P = B.block_probs(B.block_means(q, idx), B.block_means(kk, idx))
    nb = P.shape[2]
    all_k, _, _ = B.select_blocks(P, nb, 0.2)
    all_p, _, _ = B.select_blocks(P, 0, 1.0)
    assert all_k.all() and all_p.all()
    prev = None
    for k, p in [(0, 0.3), (1, 0.5), (3, 0.5), (3, 0.8), (5, 0.95)]:
        m, c, _ = B.select_blocks(P, k, p)
        assert np.all(c >= max(1, min(k, nb)))
        assert np.all((P * m).sum(2) >= p - 1e-15)
        if prev is not None:
            assert np.all(m >= prev)            # nested as k and p grow
        prev = m
        # minimality of the nucleus: when K_i > k, dropping the last block falls below p
        for hd in range(P.shape[0]):
            for i in range(P.shape[1]):
                if c[hd, i] > k:
                    ps = np.sort(P[hd, i][m[hd, i]])
                    assert ps[1:].sum() < p + 1e-15


def test_query_pooling_equals_mean_of_query_logits():
    w, q, kk, _ = _small_sparse(seed=13)
    idx = B.block_token_index(w["T"], w["H"], w["W"])
    qb, kb = B.block_means(q, idx), B.block_means(kk, idx)
    for hd in range(2):
        per_query = np.einsum("bvd,jd->bvj", q[idx, hd, :].astype(np.float64), kb[hd]).mean(1)
        assert np.allclose(per_query, qb[hd] @ kb[hd].T, rtol=0, atol=1e-12)


def test_sparse_with_all_blocks_is_dense():
    w, q, kk, v = _small_sparse(seed=14)
    idx = B.block_token_index(w["T"], w["H"], w["W"])
    nb = idx.shape[0]
    mask = np.ones((2, nb, nb), bool)
    out = B.block_sparse_attention(q, kk, v, idx, mask)
    dense = A.attention(q, kk, v)
    for (hd, i), o in out.items():
        assert np.max(np.abs(o - dense[idx[i], hd])) < 1e-12


def test_sparse_equals_token_masked_dense_and_brute():
    w, q, kk, v = _small_sparse(seed=15)
    idx = B.block_token_index(w["T"], w["H"], w["W"])
    P = B.block_probs(B.block_means(q, idx), B.block_means(kk, idx))
    mask, _, _ = B.select_blocks(P, 2, 0.6)
    n = q.shape[0]
    owner = np.empty(n, np.int64)
    owner[idx.ravel()] = np.repeat(np.arange(idx.shape[0]), idx.shape[1])
    out = B.block_sparse_attention(q, kk, v, idx, mask)
    sc = 1 / np.sqrt(q.shape[2])
    for hd in range(2):
        allow = mask[hd][owner][:, owner]       # token-level mask
        ref = A.masked_attention(q[:, hd:hd + 1], kk[:, hd:hd + 1], v[:, hd:hd + 1], allow)
        for i in range(idx.shape[0]):
            assert np.max(np.abs(out[(hd, i)] - ref[idx[i], 0])) < 1e-12
        i = 5
        keys = [t for j in np.flatnonzero(mask[hd, i]) for t in idx[j]]
        r = 3
        want = brute.attention_row(list(q[idx[i, r], hd]), [list(kk[t, hd]) for t in keys],
                                   [list(v[t, hd]) for t in keys], sc)
        assert np.allclose(out[(hd, i)][r], want, rtol=0, atol=1e-12)


def test_pack_mask_layout():
    m = np.zeros((1, 2, 40), bool)
    m[0, 0, [0, 31, 32, 39]] = True
    m[0, 1, [5]] = True
    w = B.pack_mask(m)
    assert w.shape == (1, 2, 2) and w.dtype == np.uint32
    assert w[0, 0].tolist() == [1 | (1 << 31), 1 | (1 << 7)]
    assert w[0, 1].tolist() == [1 << 5, 0]
