"""Pins of the RoPE oracle against closed forms, invariants, a textbook special
case and brute force (CPU only)."""
import math

import numpy as np
import pytest

from oracle import brute
from oracle import rope as R
from synth import WORKLOADS

TH = 10000.0


def _rot(x, pos, split, theta=TH):
    x = np.asarray(x, dtype=np.float64)
    if x.ndim == 1:
        x = x[None, None, :]
    pos = np.asarray(pos, dtype=np.float64).reshape(-1, 3)
    return R.apply_rope(x, pos, np.ones(pos.shape[0], dtype=bool), split, theta)


def test_hand_worked_single_axis():
    # d = 4, all on the t axis: pair 0 turns at omega 1, pair 1 at 10000^(-1/2) = 0.01.
    y = _rot([1.0, 0.0, 0.0, 1.0], [1.0, 0.0, 0.0], (4, 0, 0))[0, 0]
    want = [math.cos(1.0), math.sin(1.0), -math.sin(0.01), math.cos(0.01)]
    assert np.allclose(y, want, rtol=0, atol=1e-15)
    y = _rot([1.0, 0.0, 0.0, 1.0], [-1.0, 0.0, 0.0], (4, 0, 0))[0, 0]
    want = [math.cos(1.0), -math.sin(1.0), math.sin(0.01), math.cos(0.01)]
    assert np.allclose(y, want, rtol=0, atol=1e-15)


def test_hand_worked_three_axes_order():
    # one pair per axis (omega 1): slice order t | h | w, adjacent pairs.
    y = _rot([1, 0, 1, 0, 0, 1], [-1.0, 2.0, 3.0], (2, 2, 2))[0, 0]
    want = [math.cos(-1), math.sin(-1), math.cos(2), math.sin(2), -math.sin(3), math.cos(3)]
    assert np.allclose(y, want, rtol=0, atol=1e-15)


def test_frequency_ladder():
    # width 8 -> omegas 1, 10^-1, 10^-2, 10^-3 for theta = 10^4
    om = R.axis_frequencies(8, TH)
    assert np.allclose(om, [1.0, 0.1, 0.01, 0.001], rtol=1e-15, atol=0)


def test_textbook_1d_rope_special_case():
    # with d_h = d_w = 0 the map is RoFormer's RoPE: pair i as a complex number
    # multiplied by exp(i * p * theta^(-2i/d)).
    rng = np.random.default_rng(5)
    d = 64
    x = rng.standard_normal((7, 3, d))
    p = rng.uniform(-50, 50, size=7)
    pos = np.stack([p, np.zeros(7), np.zeros(7)], 1)
    y = R.apply_rope(x, pos, np.ones(7, bool), (d, 0, 0), TH)
    z = x[..., 0::2] + 1j * x[..., 1::2]
    freqs = 1.0 / (TH ** (np.arange(0, d, 2) / d))
    zr = z * np.exp(1j * p[:, None, None] * freqs[None, None, :])
    assert np.allclose(y[..., 0::2], zr.real, atol=1e-12)
    assert np.allclose(y[..., 1::2], zr.imag, atol=1e-12)


@pytest.mark.parametrize("split", [(16, 24, 24), (32, 48, 48)])
def test_norm_preserved_per_slice(split):
    rng = np.random.default_rng(1)
    d = sum(split)
    x = rng.standard_normal((50, 4, d))
    pos = np.column_stack([rng.uniform(-3, 30, 50), rng.integers(0, 60, 50), rng.integers(0, 90, 50)])
    y = R.apply_rope(x, pos, np.ones(50, bool), split, TH)
    o = 0
    for w in split:
        nx = np.linalg.norm(x[..., o:o + w], axis=-1)
        ny = np.linalg.norm(y[..., o:o + w], axis=-1)
        assert np.max(np.abs(nx - ny) / nx) < 1e-12
        o += w


def test_relative_offset_invariance():
    # <R(p) q, R(p') k> depends only on p - p'; includes t = -1 and fractional audio t.
    rng = np.random.default_rng(2)
    split = (32, 48, 48)
    q = rng.standard_normal((1, 1, 128))
    k = rng.standard_normal((1, 1, 128))
    pairs = [((-1.0, 3.0, 7.0), (0.0, 3.0, 7.0)),
             ((5.0, 0.0, 0.0), (17 * 21 / 218, 0.0, 0.0)),
             ((-1.0, 12.0, 40.0), (203 * 21 / 218, 0.0, 0.0))]
    for pq, pk in pairs:
        base = np.sum(_rot(q, pq, split) * _rot(k, pk, split))
        for _ in range(5):
            delta = rng.uniform(-40, 40, 3)
            s = np.sum(_rot(q, np.add(pq, delta), split) * _rot(k, np.add(pk, delta), split))
            assert abs(s - base) <= 1e-12 * max(1.0, abs(base))


def test_composition():
    rng = np.random.default_rng(3)
    split = (16, 24, 24)
    x = rng.standard_normal((1, 2, 64))
    a = np.array([-1.0, 2.0, 5.0])
    b = np.array([0.37, 11.0, -4.0])
    ab = _rot(_rot(x, a, split), b, split)
    assert np.allclose(ab, _rot(x, a + b, split), atol=1e-12)


def test_identity_at_origin_and_text_untouched():
    w = WORKLOADS["tiny"]
    pos, rot = R.token_positions(w)
    rng = np.random.default_rng(4)
    x = rng.standard_normal((len(rot), 2, 64))
    y = R.apply_rope(x, pos, rot, w["split"], w["theta"])
    assert np.array_equal(y[~rot], x[~rot])
    zero = np.flatnonzero(rot & np.all(pos == 0, axis=1))
    assert zero.size >= 2                      # video (0,0,0) and audio j=0
    assert np.array_equal(y[zero], x[zero])


def test_positions_of_tiny_layout(page_constants):
    w = WORKLOADS["tiny"]
    pos, rot = R.token_positions(w)
    assert pos.shape == (88, 3)
    # 16 conditioning tokens at t = -1 in raster (h, w)
    assert np.all(pos[:16, 0] == float(page_constants["cond_time_sign"]))
    assert np.array_equal(pos[5, 1:], [1.0, 1.0])
    # video frame t, row h, column w sits at 16 + (t*4 + h)*4 + w
    assert np.array_equal(pos[16 + (2 * 4 + 3) * 4 + 1], [2.0, 3.0, 1.0])
    # audio j at j * 3/16, text not rotated
    assert np.allclose(pos[64:80, 0], np.arange(16) * 3 / 16, rtol=0, atol=0)
    assert np.all(pos[64:80, 1:] == 0)
    assert not rot[80:].any() and rot[:80].all()


def test_page_constants_in_workloads(page_constants):
    num, den = (int(s) for s in page_constants["audio_rope_scale"].split("/"))
    for name in ("block", "480p", "720p"):
        w = WORKLOADS[name]
        assert w["audio_scale"] == (num, den)
        assert w["T"] == int(page_constants["audio_video_frames"])
        assert w["n_audio"] == int(page_constants["audio_tokens"])
    # the tiny case scales by T_generated / N_audio as well (cond frames excluded)
    t = WORKLOADS["tiny"]
    assert t["audio_scale"] == (t["T"], t["n_audio"])


def test_video_audio_logit_depends_on_time_offset_only():
    # video token at (t, h, w) against audio j: equal to a video token at
    # (t - j*s, h, w) against an audio token at position 0.
    rng = np.random.default_rng(6)
    split = (32, 48, 48)
    s = 21 / 218
    for _ in range(6):
        q = rng.standard_normal((1, 1, 128))
        k = rng.standard_normal((1, 1, 128))
        t, h, w, j = rng.integers(-1, 21), rng.integers(0, 30), rng.integers(0, 52), rng.integers(0, 218)
        a = np.sum(_rot(q, (t, h, w), split) * _rot(k, (j * s, 0, 0), split))
        b = np.sum(_rot(q, (t - j * s, h, w), split) * _rot(k, (0, 0, 0), split))
        assert abs(a - b) <= 1e-12 * max(1, abs(a))


def test_matches_brute_force_on_tiny():
    w = WORKLOADS["tiny"]
    pos, rot = R.token_positions(w)
    rng = np.random.default_rng(7)
    x = rng.standard_normal((88, 2, 64))
    y = R.apply_rope(x, pos, rot, w["split"], w["theta"])
    bpos = brute.sequence_positions(w["T"], w["H"], w["W"], w["n_cond_frames"], w["n_audio"],
                                    w["n_text"], *w["audio_scale"])
    for n, p in enumerate(bpos):
        for hd in range(2):
            want = list(x[n, hd]) if p is None else brute.rope_token(list(x[n, hd]), *p, w["split"], w["theta"])
            assert np.allclose(y[n, hd], want, rtol=0, atol=1e-12)


def test_table_matches_rotation():
    # table entries reproduce the rotation of a unit pair
    w = WORKLOADS["tiny"]
    tab = R.rope_table(w)
    assert tab["cond_t"].shape == (1, 8, 2)
    assert tab["video_t"].shape == (3, 8, 2) and tab["h"].shape == (4, 12, 2)
    assert tab["audio_t"].shape == (16, 8, 2)
    assert np.allclose(tab["cond_t"][0, 0], [math.cos(-1.0), math.sin(-1.0)], atol=1e-16)
    assert np.allclose(tab["audio_t"][5, 1], [math.cos(5 * 3 / 16 * TH ** (-2 / 16)),
                                              math.sin(5 * 3 / 16 * TH ** (-2 / 16))], atol=1e-15)
