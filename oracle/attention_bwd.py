"""Oracle: softmax attention for training, fp64 -- the log-sum-exp that the
forward pass keeps, and the gradients of the attention output.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the bench's CPU
baseline may import this module; the product path never does.

Sources:
  * SkyReels-V4 analysis (paper.rainbus.top 2602.21818), workflow step 4:
    the joint model is trained with a flow-matching objective on the
    predicted velocity of the video and audio latents, so every attention of
    the block (joint, video->text, audio<->video) is differentiated in the
    backward pass of a training step.
  * Prism page (xyznot.com 2610.05416), "Resultados", efficiency gains: the
    block-sparse attention is compared with full attention by the time of a
    training step at 2K, i.e. forward plus backward.

What is computed is the plain definition, per head, with s the softmax scale
and, for the block-sparse case, a fixed boolean mask of allowed (query, key)
pairs (the block selection is a piecewise-constant function of Q and K, so
no gradient flows through it):
    S = s Q K^T  (disallowed entries -inf),   P = softmax over each row,
    O = P V,   lse_i = log sum_j exp(S_ij)   (natural log).
For the gradient dO of a scalar loss with respect to O, the chain rule
through O = P V and through the row softmax, whose Jacobian is
d p_j / d x_k = p_j (delta_jk - p_k), gives
    dV = P^T dO
    dP = dO V^T
    D_i = sum_j P_ij dP_ij
    dS = P o (dP - D)          (o: elementwise; D broadcast along the row)
    dQ = s dS K,   dK = s dS^T Q.
Everything is formed from q, k, v and dO alone; this module takes neither
the forward output nor its log-sum-exp as input.
"""
import numpy as np


def _scale(d, scale):
    return np.float64(1.0 / np.sqrt(d)) if scale is None else np.float64(scale)


def _mask(allowed, h, nq, nk):
    if allowed is None:
        return None
    allowed = np.asarray(allowed, dtype=bool)
    if allowed.ndim == 2:
        allowed = np.broadcast_to(allowed, (h,) + allowed.shape)
    assert allowed.shape == (h, nq, nk)
    return allowed


def _probs(qh, kh, s, allow_h):
    """Row softmax of s q k^T (fp64) and the natural-log row log-sum-exp."""
    logits = (qh @ kh.T) * s
    if allow_h is not None:
        logits = np.where(allow_h, logits, -np.inf)
    m = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - m)
    l = e.sum(axis=1, keepdims=True)
    return e / l, (m + np.log(l))[:, 0]


def attention_fwd_lse(q, k, v, scale=None, allowed=None):
    """O [Nq, h, d] and lse [h, Nq] (both fp64) of softmax attention."""
    q64, k64, v64 = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    nq, h, d = q64.shape
    s = _scale(d, scale)
    allow = _mask(allowed, h, nq, k64.shape[0])
    o = np.empty((nq, h, v64.shape[2]))
    lse = np.empty((h, nq))
    for hd in range(h):
        p, lse[hd] = _probs(q64[:, hd], k64[:, hd], s, None if allow is None else allow[hd])
        o[:, hd] = p @ v64[:, hd]
    return o, lse


def attention_bwd(q, k, v, d_o, scale=None, allowed=None):
    """Gradients (dq, dk, dv) of sum(d_o * O) with respect to q, k, v (fp64).

    q, d_o [Nq, h, d]; k, v [Nk, h, d]; allowed None, [Nq, Nk] or [h, Nq, Nk]
    (every query row must allow at least one key).
    """
    q64, k64, v64, g64 = (np.asarray(x, dtype=np.float64) for x in (q, k, v, d_o))
    nq, h, d = q64.shape
    nk = k64.shape[0]
    s = _scale(d, scale)
    allow = _mask(allowed, h, nq, nk)
    dq = np.empty_like(q64)
    dk = np.empty_like(k64)
    dv = np.empty_like(v64)
    for hd in range(h):
        qh, kh, vh, gh = q64[:, hd], k64[:, hd], v64[:, hd], g64[:, hd]
        p, _ = _probs(qh, kh, s, None if allow is None else allow[hd])
        dv[:, hd] = p.T @ gh
        dp = gh @ vh.T
        dd = (p * dp).sum(axis=1, keepdims=True)
        ds = p * (dp - dd)
        dq[:, hd] = s * (ds @ kh)
        dk[:, hd] = s * (ds.T @ qh)
    return dq, dk, dv


def row_dot(o, d_o):
    """D [h, Nq] = <dO_i, O_i> per head, the row term of the softmax
    backward written through the forward output (equal to sum_j P_ij dP_ij
    because O_i = sum_j P_ij v_j)."""
    o64, g64 = np.asarray(o, dtype=np.float64), np.asarray(d_o, dtype=np.float64)
    return np.einsum("qhd,qhd->hq", o64, g64)


def key_rows_grads(q, k, v, d_o, keys, heads, scale=None, chunk=2048):
    """dK and dV rows of the listed keys for the listed heads (fp64), each
    [len(keys), len(heads), d], from the same definitions as attention_bwd.

    A key's gradient needs every query's probabilities, so each query's
    log-sum-exp and D_i = sum_j P_ij dP_ij are formed over all keys first,
    in chunks of `chunk` query rows (the full score matrix never exists).
    """
    q64, k64, v64, g64 = (np.asarray(x, dtype=np.float64) for x in (q, k, v, d_o))
    nq, _, d = q64.shape
    s = _scale(d, scale)
    keys = np.asarray(keys)
    dk = np.zeros((len(keys), len(heads), d))
    dv = np.zeros((len(keys), len(heads), v64.shape[2]))
    for hi, hd in enumerate(heads):
        kh, vh = k64[:, hd], v64[:, hd]
        for r0 in range(0, nq, chunk):
            qh, gh = q64[r0:r0 + chunk, hd], g64[r0:r0 + chunk, hd]
            p, _ = _probs(qh, kh, s, None)
            dd = (p * (gh @ vh.T)).sum(axis=1, keepdims=True)
            pk = p[:, keys]                               # [rows, len(keys)]
            dpk = gh @ vh[keys].T
            dsk = pk * (dpk - dd)
            dv[:, hi] += pk.T @ gh
            dk[:, hi] += s * (dsk.T @ qh)
    return dk, dv
