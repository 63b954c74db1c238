"""Pins of the content-adaptive block-shape oracle (oracle/adaptive_blocks.py).

None of these re-types the oracle's formulas: the candidate count, volumes,
zone and thresholds come from the numbers the Prism page prints
(tests/golden/page_constants.txt); the log2 shape optimum is checked against a
numerical constrained minimisation of the page's objective; the directional
variance against closed forms of separable fields; the partition against the
uniform-block oracle; the ragged attention against masked dense attention."""
import numpy as np
import pytest
from scipy.optimize import minimize_scalar, minimize

from oracle import adaptive_blocks as A
from oracle import attention_bwd as AB
from oracle import block_sparse as B


def ints(s):
    return [int(x) for x in s.split()]


def test_candidates_match_page(page_constants):
    c = A.candidate_shapes()
    assert len(c) == int(page_constants["n_candidate_shapes"]) == 16
    assert len(set(c)) == 16
    assert sorted({a * b * d for a, b, d in c}) == ints(page_constants["block_volumes"])
    zone = ints(page_constants["zone"])
    assert tuple(zone) == A.ZONE
    for s in c:
        assert all(zone[i] % s[i] == 0 for i in range(3))
    assert [sum(1 for s in c if np.prod(s) == v) for v in A.VOLUMES] == [7, 6, 3]


def test_thresholds_match_page(page_constants):
    assert A.TAU_128 == float(page_constants["tau_128"])
    assert A.TAU_256 == float(page_constants["tau_256"])
    rho = np.array([1.0, 0.5, 0.4999, 0.25, 0.2499, 0.0])
    assert A.volume(rho).tolist() == [64, 64, 128, 128, 256, 256]


@pytest.mark.parametrize("seed", range(6))
def test_ell_star_minimises_page_objective(seed):
    """sum_d g_d (b_d^2 - 1) subject to prod b_d = B, minimised numerically
    over (log2 b_T, log2 b_H) with log2 b_W = S - the other two."""
    rng = np.random.default_rng(seed)
    g = rng.uniform(0.01, 2.0, 3)
    Bv = [64, 128, 256][seed % 3]
    S = np.log2(Bv)

    def f(x):
        l = np.array([x[0], x[1], S - x[0] - x[1]])
        return float(np.sum(g * (4.0 ** l - 1.0)))

    res = minimize(f, x0=[S / 3, S / 3], method="Nelder-Mead",
                   options=dict(xatol=1e-10, fatol=1e-14, maxiter=20000))
    ell = A.ell_star(g, Bv)
    assert abs(ell.sum() - S) < 1e-12
    np.testing.assert_allclose(ell, [res.x[0], res.x[1], S - res.x[0] - res.x[1]], atol=1e-5)
    # b_d proportional to g_d^(-1/2)
    k = 2.0 ** ell * np.sqrt(g)
    np.testing.assert_allclose(k, k[0], rtol=1e-12)


def test_ell_star_one_axis_by_line_search():
    """With g_H = g_W the optimum has b_H = b_W; a 1-D search over b_T."""
    g = np.array([0.7, 0.2, 0.2])
    S = np.log2(128.0)
    res = minimize_scalar(lambda lt: g[0] * (4 ** lt - 1) + 2 * g[1] * (4 ** ((S - lt) / 2) - 1),
                          bounds=(-5, 12), method="bounded", options=dict(xatol=1e-12))
    ell = A.ell_star(g, 128)
    assert abs(ell[0] - res.x) < 1e-6 and abs(ell[1] - ell[2]) < 1e-12


def test_nearest_shape_cases():
    c = A.candidate_shapes()
    iso = A.ell_star(np.ones(3), 64)
    assert c[A.nearest_shape(iso, 64)] == (4, 4, 4)
    # content that changes only along T: short blocks in T, long elsewhere
    g = np.array([1.0 + A.EPS, A.EPS, A.EPS])
    for Bv, want_t in ((64, 2), (128, 2), (256, 4)):
        s = c[A.nearest_shape(A.ell_star(g, Bv), Bv)]
        assert np.prod(s) == Bv and s[0] == want_t
    # content that changes along W only: short in W
    g = np.array([A.EPS, A.EPS, 1.0 + A.EPS])
    assert c[A.nearest_shape(A.ell_star(g, 256), 256)] == (8, 8, 4)
    # strong H and W variation, little along T: long in T
    g = np.array([0.02, 0.49, 0.49])
    assert c[A.nearest_shape(A.ell_star(g, 128), 128)] == (8, 4, 4)


def separable_zone(alpha, beta, gamma, f, gh, k, delta):
    """z[t, h, w, c] = alpha_c f_t + beta_c g_h + gamma_c k_w + delta_c."""
    return (alpha[None, None, None, :] * f[:, None, None, None] + beta[None, None, None, :] * gh[None, :, None, None]
            + gamma[None, None, None, :] * k[None, None, :, None] + delta[None, None, None, :])


def test_directional_variance_separable_closed_form():
    rng = np.random.default_rng(3)
    C = 11
    alpha, beta, gamma, delta = (rng.normal(size=C) for _ in range(4))
    f, gh, k = (rng.normal(size=8) for _ in range(3))
    f, gh, k = f - f.mean(), gh - gh.mean(), k - k.mean()
    z = separable_zone(alpha, beta, gamma, f, gh, k, delta)
    want = [np.mean(alpha ** 2) * np.mean(f ** 2), np.mean(beta ** 2) * np.mean(gh ** 2),
            np.mean(gamma ** 2) * np.mean(k ** 2)]
    np.testing.assert_allclose(A.directional_variance(z), want, rtol=1e-12)


def test_directional_variance_invariances():
    rng = np.random.default_rng(4)
    z = rng.normal(size=(8, 8, 8, 5))
    s = A.directional_variance(z)
    np.testing.assert_allclose(A.directional_variance(z + rng.normal(size=5)), s, rtol=1e-12)
    np.testing.assert_allclose(A.directional_variance(3.0 * z), 9.0 * s, rtol=1e-12)
    np.testing.assert_allclose(A.directional_variance(z.transpose(1, 0, 2, 3)), s[[1, 0, 2]], rtol=1e-12)
    np.testing.assert_allclose(A.directional_variance(z.transpose(2, 1, 0, 3)), s[[2, 1, 0]], rtol=1e-12)
    np.testing.assert_allclose(A.directional_variance(z[..., ::-1]), s, rtol=1e-12)


def test_zone_view_matches_uniform_enumeration():
    T, H, W = 16, 8, 24
    x = np.arange(T * H * W, dtype=np.float64)[:, None]
    zv = A.zone_view(x, T, H, W).reshape(-1, 512)
    idx = B.block_token_index(T, H, W, zone=(8, 8, 8), block=(8, 8, 8))
    np.testing.assert_array_equal(zv, idx)


def three_zone_grid(amps, a=None):
    """T=8, H=8, W=8*len(amps): zone m holds a separable pattern of amplitude amps[m]
    with different strengths per axis."""
    rng = np.random.default_rng(5)
    C = 6
    f, gh, k = (rng.normal(size=8) for _ in range(3))
    f, gh, k = f - f.mean(), gh - gh.mean(), k - k.mean()
    alpha, beta, gamma = rng.normal(size=C), 0.5 * rng.normal(size=C), 0.2 * rng.normal(size=C)
    z = separable_zone(alpha, beta, gamma, f, gh, k, np.zeros(C))
    W = 8 * len(amps)
    v = np.zeros((8, 8, W, C))
    for m, amp in enumerate(amps):
        v[:, :, 8 * m:8 * m + 8, :] = amp * z
    return v.reshape(-1, 2, C // 2), z


def test_rho_sets_volumes():
    v, z = three_zone_grid([1.0, 0.7, 0.45])
    ind = A.variation_indicator(v, None, 8, 8, 24)
    np.testing.assert_allclose(ind["rho"], [1.0, 0.49, 0.2025], rtol=1e-12)
    assert A.volume(ind["rho"]).tolist() == [64, 128, 256]
    s = A.directional_variance(z)
    for m in range(3):
        np.testing.assert_allclose(ind["r_v"][m], s / s.sum(), rtol=1e-12)
    assert np.all(ind["a_bar"] == 0.0) and np.all(ind["v_hat"] == 0.0)
    np.testing.assert_allclose(ind["g"], ind["r_v"] + A.EPS, rtol=1e-15)


def test_constant_values_give_largest_blocks():
    v = np.ones((8 * 8 * 16, 2, 4))
    codes, ind = A.zone_shapes(v, None, 8, 8, 16)
    assert np.all(ind["energy"] == 0.0) and np.all(ind["r_v"] == 0.0)
    assert ind["volume"].tolist() == [256, 256]
    # g = eps on every axis: isotropic optimum, first of the equidistant 256 shapes
    assert [A.candidate_shapes()[c] for c in codes] == [(4, 8, 8), (4, 8, 8)]


def test_audio_coupling():
    v, _ = three_zone_grid([1.0, 1.0, 1.0])
    T, H, W = 8, 8, 24
    a = np.zeros((T, H, W))
    pulse = np.array([0.0, 1.0, 3.0, 1.0, 0.0, 1.0, 3.0, 1.0])
    a[:, :, 0:8] = 2.0 + pulse[:, None, None]        # zone 0: only T varies
    a[:, :, 8:16] = 1.625                           # zone 1: constant, half of zone 0's mean 3.25
    ind = A.variation_indicator(v, a.reshape(-1), T, H, W)
    np.testing.assert_allclose(ind["a_mean"], [3.25, 1.625, 0.0], rtol=1e-15)
    np.testing.assert_allclose(ind["a_bar"], [1.0, 0.5, 0.0], rtol=1e-15)
    np.testing.assert_allclose(ind["v_hat"][0], [1.0, 0.0, 0.0], atol=1e-15)
    assert np.all(ind["v_hat"][1:] == 0.0)
    np.testing.assert_allclose(ind["sigma2_a"][0, 0], np.var(pulse), rtol=1e-12)
    np.testing.assert_allclose(ind["g"][0], ind["r_v"][0] + [1.0, 0.0, 0.0] + A.EPS, rtol=1e-14)
    # no norms behaves as all-zero norms
    i0 = A.variation_indicator(v, None, T, H, W)
    i1 = A.variation_indicator(v, np.zeros(T * H * W), T, H, W)
    np.testing.assert_array_equal(i0["g"], i1["g"])


def test_adaptive_partition_covers_zones():
    T, H, W = 16, 16, 8
    rng = np.random.default_rng(6)
    nz = 4
    codes = rng.integers(0, 16, nz)
    blocks, zone_of = A.adaptive_block_tokens(T, H, W, codes)
    allt = np.concatenate(blocks)
    assert np.array_equal(np.sort(allt), np.arange(T * H * W))
    cands = A.candidate_shapes()
    assert np.all(np.diff(zone_of) >= 0)
    for b, m in zip(blocks, zone_of):
        s = cands[codes[m]]
        assert len(b) == np.prod(s)
        t, h, w = b // (H * W), (b // W) % H, b % W
        assert (t.max() - t.min() + 1, h.max() - h.min() + 1, w.max() - w.min() + 1) == s
        assert np.all(np.diff(b) > 0)                      # raster order inside the block
        zone_t, zone_h, zone_w = t[0] // 8, h[0] // 8, w[0] // 8
        assert (zone_t * 2 + zone_h) * 1 + zone_w == m      # zones: 2 x 2 x 1 in raster order
    assert [int(np.sum(zone_of == m)) for m in range(nz)] == [512 // np.prod(cands[c]) for c in codes]


def test_uniform_codes_reduce_to_uniform_blocks():
    T, H, W = 16, 8, 16
    code = A.candidate_shapes().index((4, 4, 4))
    blocks, _ = A.adaptive_block_tokens(T, H, W, np.full(4, code))
    idx = B.block_token_index(T, H, W, (8, 8, 8), (4, 4, 4))
    np.testing.assert_array_equal(np.stack(blocks), idx)
    rng = np.random.default_rng(7)
    x = rng.normal(size=(T * H * W, 2, 3))
    np.testing.assert_array_equal(A.ragged_means(x, blocks), B.block_means(x, idx))


def test_ragged_attention_matches_masked_dense():
    T, H, W = 8, 8, 16
    rng = np.random.default_rng(8)
    codes = np.array([A.candidate_shapes().index((2, 8, 8)), A.candidate_shapes().index((8, 4, 2))])
    blocks, _ = A.adaptive_block_tokens(T, H, W, codes)
    nb = len(blocks)
    n, h, d = T * H * W, 2, 16
    q, k, v = (rng.normal(size=(n, h, d)) for _ in range(3))
    mask = rng.random((h, nb, nb)) < 0.4
    mask[:, np.arange(nb), np.arange(nb)] = True
    out = A.ragged_sparse_attention(q, k, v, blocks, mask, scale=0.3)
    blk = np.empty(n, dtype=np.int64)
    for j, b in enumerate(blocks):
        blk[b] = j
    allowed = mask[:, blk][:, :, blk]
    o_ref, _ = AB.attention_fwd_lse(q, k, v, scale=0.3, allowed=allowed)
    for (hd, i), o in out.items():
        np.testing.assert_allclose(o, o_ref[blocks[i], hd], atol=1e-12)
    full = A.ragged_sparse_attention(q, k, v, blocks, np.ones((h, nb, nb), bool), scale=0.3)
    o_dense, _ = AB.attention_fwd_lse(q, k, v, scale=0.3)
    for (hd, i), o in full.items():
        np.testing.assert_allclose(o, o_dense[blocks[i], hd], atol=1e-12)


def test_token_norms():
    rng = np.random.default_rng(9)
    x = rng.normal(size=(7, 3, 5))
    np.testing.assert_allclose(A.token_norms(x), [np.linalg.norm(x[i]) for i in range(7)], rtol=1e-14)


def test_pipeline_on_nonstationary_field():
    """A strong anisotropic pattern in one zone, a weaker one in the next and
    almost nothing in the third: three volumes and shapes that follow the
    strongest axis."""
    T, H, W = 8, 8, 24
    rng = np.random.default_rng(10)
    C = 8
    tt, hh, ww = np.meshgrid(np.arange(8), np.arange(8), np.arange(8), indexing="ij")
    ph = rng.uniform(0, 2 * np.pi, C)
    fast_t = np.sin(2.0 * tt[..., None] + ph)             # varies along T only
    fast_w = np.sin(2.0 * ww[..., None] + ph)             # along W only
    v = np.zeros((T, H, W, C))
    v[:, :, 0:8] = fast_t
    v[:, :, 8:16] = 0.6 * fast_w
    v[:, :, 16:24] = 0.01 * fast_w
    codes, ind = A.zone_shapes(v.reshape(-1, 2, C // 2), None, T, H, W)
    cands = A.candidate_shapes()
    assert ind["volume"].tolist() == [64, 128, 256]
    assert cands[codes[0]][0] == 2 and cands[codes[1]][2] == 2 and cands[codes[2]][2] == 4
    blocks, zone_of = A.adaptive_block_tokens(T, H, W, codes)
    assert len(blocks) == 8 + 4 + 2
    q = rng.normal(size=(T * H * W, 2, 16))
    kk = rng.normal(size=(T * H * W, 2, 16))
    P = B.block_probs(A.ragged_means(q, blocks), A.ragged_means(kk, blocks))
    mask, counts, _ = B.select_blocks(P, 3, 0.5)
    assert mask.shape == (2, 14, 14) and np.all(counts >= 3)
