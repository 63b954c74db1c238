"""Pins of the dense-attention oracle: brute force, a library routine and the
invariants of softmax attention (CPU only)."""
import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import brute
from synth import WORKLOADS


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def test_matches_brute_force_tiny_joint():
    q, k, v = (_rand((88, 2, 64), s) for s in (0, 1, 2))
    o = A.attention(q, k, v)
    sc = 1 / np.sqrt(64)
    for hd in range(2):
        keys = [list(k[j, hd]) for j in range(88)]
        vals = [list(v[j, hd]) for j in range(88)]
        for i in range(0, 88, 7):
            want = brute.attention_row(list(q[i, hd]), keys, vals, sc)
            assert np.allclose(o[i, hd], want, rtol=0, atol=1e-12)


def test_matches_torch_sdpa_fp64():
    q, k, v = (_rand((300, 3, 128), s) for s in (3, 4, 5))
    kv = _rand((517, 3, 128), 6), _rand((517, 3, 128), 7)
    o = A.attention(q, kv[0], kv[1])
    tq = torch.from_numpy(q).permute(1, 0, 2)
    tk = torch.from_numpy(kv[0]).permute(1, 0, 2)
    tv = torch.from_numpy(kv[1]).permute(1, 0, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv).permute(1, 0, 2).numpy()
    assert np.max(np.abs(o - ref)) < 1e-12
    del v


def test_rows_sum_to_one_and_ones_values():
    q, k = _rand((40, 2, 64), 8, 3.0), _rand((70, 2, 64), 9, 3.0)
    P = A.attention_probs(q, k)
    assert np.max(np.abs(P.sum(axis=2) - 1)) < 1e-12
    o = A.attention(q, k, np.ones((70, 2, 64)))
    assert np.max(np.abs(o - 1)) < 1e-12


def test_single_key_returns_its_value():
    q, k, v = _rand((9, 2, 64), 10), _rand((1, 2, 64), 11), _rand((1, 2, 64), 12)
    o = A.attention(q, k, v)
    assert np.max(np.abs(o - v[0][None])) < 1e-15


def test_permutation_equivariance():
    q, k, v = _rand((33, 2, 64), 13), _rand((45, 2, 64), 14), _rand((45, 2, 64), 15)
    o = A.attention(q, k, v)
    pk = np.random.default_rng(16).permutation(45)
    pq = np.random.default_rng(17).permutation(33)
    assert np.max(np.abs(A.attention(q, k[pk], v[pk]) - o)) < 1e-12
    assert np.max(np.abs(A.attention(q[pq], k, v) - o[pq])) < 1e-12


def test_key_shift_invariance():
    # adding one vector u to every key shifts each row's logits by q.u
    q, k, v = _rand((20, 2, 64), 18), _rand((30, 2, 64), 19), _rand((30, 2, 64), 20)
    u = _rand((1, 2, 64), 21)
    assert np.max(np.abs(A.attention(q, k + u, v) - A.attention(q, k, v))) < 1e-12


def test_cross_attention_equals_masked_joint():
    w = WORKLOADS["tiny"]
    seg = A.joint_segments(w)
    n = 88
    q, k, v = (_rand((n, 2, 64), s) for s in (22, 23, 24))
    vs0, vs1 = seg["video_stream"]
    a0, a1 = seg["audio"]
    assert (vs1 - vs0, a1 - a0) == (64, 16)
    va = A.attention(q[vs0:vs1], k[a0:a1], v[a0:a1])
    av = A.attention(q[a0:a1], k[vs0:vs1], v[vs0:vs1])
    allow = np.zeros((n, n), bool)
    allow[vs0:vs1, a0:a1] = True
    allow[a0:a1, vs0:vs1] = True
    allow[a1:, :] = True                       # text rows: anything, unused
    m = A.masked_attention(q, k, v, allow)
    assert np.max(np.abs(m[vs0:vs1] - va)) < 1e-12
    assert np.max(np.abs(m[a0:a1] - av)) < 1e-12


def test_row_subset_matches_full():
    q, k, v = _rand((100, 2, 64), 25), _rand((60, 2, 64), 26), _rand((60, 2, 64), 27)
    rows = np.array([0, 7, 99, 50])
    full = A.attention(q, k, v, chunk=17)
    sub = A.attention(q, k, v, rows=rows)
    assert np.array_equal(sub, A.attention(q[rows], k, v))
    assert np.max(np.abs(sub - full[rows])) < 1e-13


@pytest.mark.parametrize("gain", [4.0, 20.0])
def test_large_logits_stay_finite(gain):
    q, k, v = _rand((16, 1, 128), 28, gain), _rand((64, 1, 128), 29, gain), _rand((64, 1, 128), 30)
    o = A.attention(q, k, v)
    assert np.isfinite(o).all()
    keys = [list(k[j, 0]) for j in range(64)]
    vals = [list(v[j, 0]) for j in range(64)]
    for i in (0, 9):
        want = brute.attention_row(list(q[i, 0]), keys, vals, 1 / np.sqrt(128))
        assert np.allclose(o[i, 0], want, rtol=0, atol=1e-11)
