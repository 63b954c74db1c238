"""Pins of the training oracle (log-sum-exp and attention gradients), CPU only.

The gradients are pinned to things other than their own formulas:
  * central finite differences of the forward oracle (oracle.attention, a
    separate module that never forms a gradient), on every input element of
    a tiny case, with and without a block mask;
  * torch autograd through scaled_dot_product_attention in float64;
  * invariants of softmax attention: a common shift of every key leaves O
    unchanged, so dK sums to zero over the keys; rows of P sum to one, so dV
    sums to the sum of dO; one key makes O constant in q and k;
  * the log-sum-exp against scipy.special.logsumexp and brute-force sums.
"""
import math

import numpy as np
import pytest
import scipy.special
import torch

from oracle import attention as A
from oracle import attention_bwd as B


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _loss(q, k, v, g, scale, allowed=None):
    if allowed is None:
        o = A.attention(q, k, v, scale=scale)
    else:
        o = A.masked_attention(q, k, v, allowed, scale=scale)
    return float(np.sum(o * g))


def _finite_diff(q, k, v, g, scale, allowed=None, eps=1e-5):
    grads = []
    for which in range(3):
        xs = [q.copy(), k.copy(), v.copy()]
        x = xs[which]
        out = np.empty_like(x)
        for idx in np.ndindex(x.shape):
            keep = x[idx]
            x[idx] = keep + eps
            lp = _loss(*xs, g, scale, allowed)
            x[idx] = keep - eps
            lm = _loss(*xs, g, scale, allowed)
            x[idx] = keep
            out[idx] = (lp - lm) / (2 * eps)
        grads.append(out)
    return grads


@pytest.mark.parametrize("scale", [None, 0.7])
def test_gradients_match_finite_differences(scale):
    q, k, v, g = _rand((5, 2, 8), 1), _rand((7, 2, 8), 2), _rand((7, 2, 8), 3), _rand((5, 2, 8), 4)
    sc = 1 / math.sqrt(8) if scale is None else scale
    fd = _finite_diff(q, k, v, g, sc)
    an = B.attention_bwd(q, k, v, g, scale=scale)
    for a, f in zip(an, fd):
        assert np.max(np.abs(a - f)) < 1e-8 * max(1.0, np.max(np.abs(f)))


def test_masked_gradients_match_finite_differences():
    rng = np.random.default_rng(5)
    q, k, v, g = _rand((6, 2, 8), 6), _rand((9, 2, 8), 7), _rand((9, 2, 8), 8), _rand((6, 2, 8), 9)
    allowed = rng.random((2, 6, 9)) < 0.5
    allowed[:, np.arange(6), np.arange(6)] = True          # every row keeps a key
    fd = _finite_diff(q, k, v, g, 0.5, allowed)
    an = B.attention_bwd(q, k, v, g, scale=0.5, allowed=allowed)
    for a, f in zip(an, fd):
        assert np.max(np.abs(a - f)) < 1e-8 * max(1.0, np.max(np.abs(f)))
    # disallowed keys of every query get no gradient from that query: a key
    # allowed by no query has dK = dV = 0
    allowed2 = allowed.copy()
    allowed2[:, :, 8] = False
    _, dk, dv = B.attention_bwd(q, k, v, g, scale=0.5, allowed=allowed2)
    assert np.all(dk[8] == 0) and np.all(dv[8] == 0)


def test_gradients_match_torch_autograd_fp64():
    q, k, v, g = _rand((50, 3, 64), 10), _rand((70, 3, 64), 11), _rand((70, 3, 64), 12), _rand((50, 3, 64), 13)
    tq, tk, tv = (torch.from_numpy(x.transpose(1, 0, 2).copy()).requires_grad_() for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv)
    o.backward(torch.from_numpy(g.transpose(1, 0, 2).copy()))
    dq, dk, dv = B.attention_bwd(q, k, v, g)
    for mine, t in ((dq, tq), (dk, tk), (dv, tv)):
        ref = t.grad.numpy().transpose(1, 0, 2)
        assert np.max(np.abs(mine - ref)) < 1e-12


def test_full_mask_equals_dense():
    q, k, v, g = _rand((11, 2, 16), 14), _rand((13, 2, 16), 15), _rand((13, 2, 16), 16), _rand((11, 2, 16), 17)
    dense = B.attention_bwd(q, k, v, g)
    masked = B.attention_bwd(q, k, v, g, allowed=np.ones((11, 13), bool))
    for a, b in zip(dense, masked):
        assert np.max(np.abs(a - b)) < 1e-14


def test_invariants():
    q, k, v, g = _rand((40, 2, 32), 18, 2.0), _rand((30, 2, 32), 19, 2.0), _rand((30, 2, 32), 20), _rand((40, 2, 32), 21)
    dq, dk, dv = B.attention_bwd(q, k, v, g)
    scale = np.max(np.abs(dk))
    assert np.max(np.abs(dk.sum(axis=0))) < 1e-12 * max(1.0, scale) * 30
    assert np.max(np.abs(dv.sum(axis=0) - g.sum(axis=0))) < 1e-11
    # one key: O = v_0 for every query, independent of q and k
    dq1, dk1, dv1 = B.attention_bwd(q, k[:1], v[:1], g)
    assert np.max(np.abs(dq1)) < 1e-15 and np.max(np.abs(dk1)) < 1e-15
    assert np.max(np.abs(dv1[0] - g.sum(axis=0))) < 1e-12
    # D written through the forward output equals sum_j P_ij dP_ij
    o, _ = B.attention_fwd_lse(q, k, v)
    P = A.attention_probs(q, k)
    dP = np.einsum("qhd,khd->hqk", g, v)
    assert np.max(np.abs(B.row_dot(o, g) - (P * dP).sum(axis=2))) < 1e-12


def test_lse_matches_scipy_and_brute_force():
    q, k, v = _rand((25, 2, 64), 22, 3.0), _rand((37, 2, 64), 23, 3.0), _rand((37, 2, 64), 24)
    o, lse = B.attention_fwd_lse(q, k, v, scale=0.3)
    logits = np.einsum("qhd,khd->hqk", q, k) * 0.3
    assert np.max(np.abs(lse - scipy.special.logsumexp(logits, axis=2))) < 1e-12
    for hd, i in ((0, 0), (1, 24)):
        tot = sum(math.exp(0.3 * float(np.dot(q[i, hd], k[j, hd])) - lse[hd, i]) for j in range(37))
        assert abs(tot - 1.0) < 1e-12
    assert np.max(np.abs(o - A.attention(q, k, v, scale=0.3))) < 1e-12


def test_key_rows_match_full_gradients():
    q, k, v, g = _rand((300, 2, 16), 25), _rand((200, 2, 16), 26), _rand((200, 2, 16), 27), _rand((300, 2, 16), 28)
    _, dk, dv = B.attention_bwd(q, k, v, g, scale=0.4)
    keys = [0, 5, 199]
    dk2, dv2 = B.key_rows_grads(q, k, v, g, keys, [1], scale=0.4, chunk=70)
    assert np.max(np.abs(dk2[:, 0] - dk[keys, 1])) < 1e-13
    assert np.max(np.abs(dv2[:, 0] - dv[keys, 1])) < 1e-13
