"""Elementwise error allowances of the bf16 attention backward.

Test infrastructure: what a correct bf16 backward may differ from the fp64
gradients by, entry by entry, derived from where the kernels round.  Per head,
with s the softmax scale, P the attention probabilities (rebuilt in fp32 from
the bf16 Q K^T products and the forward's log-sum-exp), dP = dO V^T, D_i =
<dO_i, O_i> and dS = P o (dP - D):

  * dV_j = sum_i P_ij dO_i takes P rounded to bf16 (relative 2^-9), so an
    entry moves by at most 2^-9 sum_i P_ij |dO_id|;
  * dS_ij is rounded to bf16 (2^-9 of |dS_ij|), and dP and D carry the fp32
    accumulation errors of their 128-term dot products, at most gamma_128
    (about 2^-17) times sum_c |dO_ic| |v_jc| and sum_c |dO_ic| |O_ic|; all of
    it is bounded by 2^-9 M_ij with
        M_ij = P_ij (sum_c |dO_ic| |v_jc| + sum_c |dO_ic| |O_ic|) >= |dS_ij|;
    dQ_i = s sum_j dS_ij k_j then moves by at most s 2^-9 sum_j M_ij |k_jd|,
    and dK_j = s sum_i dS_ij q_i by at most s 2^-9 sum_i M_ij |q_id|;
  * the rebuilt P itself is off by the fp32 error of the logit (gamma_128 s
    sum_c |q_c k_c|) and of the forward's log-sum-exp (the fp16-rounded
    probabilities it sums, relative 2^-11), each a fraction of 2^-9 at these
    scales, and the fp32 sums over tokens add their own rounding.

The allowance is C = 4 times the 2^-9 terms (covering the terms of the last
point with room), plus an absolute 1e-6 for entries whose terms all vanish.
Unlike a bar relative to a tensor's largest entry, it holds every entry to
its own scale: a small gradient next to a large one gets a small allowance.
"""
import numpy as np

U = 2.0 ** -9
C = 4.0
FLOOR = 1e-6
TOL_UNIT = 2e-2     # the absolute bar, also kept at unit-scale inputs


def _scale(d, scale):
    return np.float64(1.0 / np.sqrt(d)) if scale is None else np.float64(scale)


def _probs(qh, kh, s, allow_h):
    logits = (qh @ kh.T) * s
    if allow_h is not None:
        logits = np.where(allow_h, logits, -np.inf)
    m = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - m)
    return e / e.sum(axis=1, keepdims=True)


def _terms(qh, kh, vh, gh, s, allow_h):
    p = _probs(qh, kh, s, allow_h)
    o = p @ vh
    ag = np.abs(gh)
    m = p * (ag @ np.abs(vh).T + np.sum(ag * np.abs(o), axis=1, keepdims=True))
    return p, m, ag


def bwd_allowances(q, k, v, d_o, scale=None, allowed=None):
    """Allowances (aq [Nq, h, d], ak [Nk, h, d], av [Nk, h, d]) for the
    gradients of softmax attention of q against k, v (allowed: None,
    [Nq, Nk] or [h, Nq, Nk] boolean mask)."""
    q64, k64, v64, g64 = (np.asarray(x, dtype=np.float64) for x in (q, k, v, d_o))
    nq, h, d = q64.shape
    s = _scale(d, scale)
    if allowed is not None:
        allowed = np.asarray(allowed, dtype=bool)
        if allowed.ndim == 2:
            allowed = np.broadcast_to(allowed, (h,) + allowed.shape)
    aq, ak, av = np.empty_like(q64), np.empty_like(k64), np.empty_like(v64)
    for hd in range(h):
        p, m, ag = _terms(q64[:, hd], k64[:, hd], v64[:, hd], g64[:, hd], s,
                          None if allowed is None else allowed[hd])
        aq[:, hd] = s * (m @ np.abs(k64[:, hd]))
        ak[:, hd] = s * (m.T @ np.abs(q64[:, hd]))
        av[:, hd] = p.T @ ag
    return tuple(C * U * a + FLOOR for a in (aq, ak, av))


def key_rows_allowances(q, k, v, d_o, keys, heads, scale=None, chunk=2048):
    """Allowances (ak, av) [len(keys), len(heads), d] of the listed keys'
    gradients, each query's probabilities formed over all keys in chunks."""
    q64, k64, v64, g64 = (np.asarray(x, dtype=np.float64) for x in (q, k, v, d_o))
    nq, _, d = q64.shape
    s = _scale(d, scale)
    keys = np.asarray(keys)
    ak = np.zeros((len(keys), len(heads), d))
    av = np.zeros((len(keys), len(heads), v64.shape[2]))
    for hi, hd in enumerate(heads):
        for r0 in range(0, nq, chunk):
            p, m, ag = _terms(q64[r0:r0 + chunk, hd], k64[:, hd], v64[:, hd], g64[r0:r0 + chunk, hd], s, None)
            ak[:, hi] += s * (m[:, keys].T @ np.abs(q64[r0:r0 + chunk, hd]))
            av[:, hi] += p[:, keys].T @ ag
    return C * U * ak + FLOOR, C * U * av + FLOOR


def check(name, got, ref, allow, unit=True):
    """Every entry within its allowance; at unit-scale inputs also max-abs
    within TOL_UNIT."""
    err = np.abs(np.asarray(got, dtype=np.float64) - ref)
    worst = float(np.max(err)) if err.size else 0.0
    ratio = float(np.max(err / allow)) if err.size else 0.0
    print("%s: max-abs %.3e, max |ref| %.3e, max error / allowance %.3f" % (
        name, worst, float(np.max(np.abs(ref))) if err.size else 0.0, ratio), flush=True)
    assert ratio <= 1.0, (name, ratio)
    if unit:
        assert worst <= TOL_UNIT, (name, worst)
