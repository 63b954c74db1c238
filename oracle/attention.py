"""Oracle: dense softmax attention, fp64.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the bench's CPU
baseline may import this module; the product path never does.

Sources (pages on SkyReels-V4):
  * SkyReels-V4 analysis (paper.rainbus.top 2602.21818), workflow step 3:
    in the dual-stream blocks video/audio tokens and text tokens attend
    jointly; every layer adds a text cross-attention (video queries text
    embeddings) and a bidirectional audio-video cross-attention.
  * trdm.cn SkyReels-V4 article, sections 2.1 and 2.2 (joint self-attention
    in the dual-stream layers; audio attends to video and video to audio in
    every block).

What is computed is the plain definition, per head:
    O_q = sum_k softmax_k(s * <q, k>) v_k,   s = 1/sqrt(d) unless given,
over the stated key set, with no mask (the pages name none).  Two passes:
row maximum first, then exponentials, sums and the weighted value sum.
"""
import numpy as np


def attention(q, k, v, scale=None, rows=None, chunk=1024):
    """Softmax attention of queries q[rows] against all of k, v.

    q [Nq, h, d], k and v [Nk, h, d] (any float dtype, promoted to fp64).
    Returns O [len(rows) or Nq, h, d] fp64.
    """
    q = np.asarray(q)
    k64 = np.asarray(k, dtype=np.float64)
    v64 = np.asarray(v, dtype=np.float64)
    d = q.shape[2]
    s = np.float64(1.0 / np.sqrt(d)) if scale is None else np.float64(scale)
    if rows is not None:
        q = q[np.asarray(rows)]
    q64 = np.asarray(q, dtype=np.float64)
    nq, h = q64.shape[0], q64.shape[1]
    out = np.empty((nq, h, v64.shape[2]), dtype=np.float64)
    for hd in range(h):
        kh = np.ascontiguousarray(k64[:, hd, :])
        vh = np.ascontiguousarray(v64[:, hd, :])
        for r0 in range(0, nq, chunk):
            qh = q64[r0:r0 + chunk, hd, :]
            logits = (qh @ kh.T) * s
            m = logits.max(axis=1, keepdims=True)
            p = np.exp(logits - m)
            l = p.sum(axis=1, keepdims=True)
            out[r0:r0 + chunk, hd, :] = (p @ vh) / l
    return out


def attention_probs(q, k, scale=None):
    """Row-stochastic attention matrix P [h, Nq, Nk] (fp64)."""
    q64 = np.asarray(q, dtype=np.float64)
    k64 = np.asarray(k, dtype=np.float64)
    d = q64.shape[2]
    s = np.float64(1.0 / np.sqrt(d)) if scale is None else np.float64(scale)
    logits = np.einsum("qhd,khd->hqk", q64, k64) * s
    m = logits.max(axis=2, keepdims=True)
    p = np.exp(logits - m)
    return p / p.sum(axis=2, keepdims=True)


def masked_attention(q, k, v, allowed, scale=None):
    """Attention where query i may only see keys j with allowed[i, j] True.

    allowed [Nq, Nk] (shared by heads) or [h, Nq, Nk].  Disallowed logits are
    -inf; every query row must allow at least one key.
    """
    q64 = np.asarray(q, dtype=np.float64)
    k64 = np.asarray(k, dtype=np.float64)
    v64 = np.asarray(v, dtype=np.float64)
    d = q64.shape[2]
    h = q64.shape[1]
    s = np.float64(1.0 / np.sqrt(d)) if scale is None else np.float64(scale)
    allowed = np.asarray(allowed, dtype=bool)
    if allowed.ndim == 2:
        allowed = np.broadcast_to(allowed, (h,) + allowed.shape)
    out = np.empty((q64.shape[0], h, v64.shape[2]), dtype=np.float64)
    for hd in range(h):
        logits = (q64[:, hd, :] @ k64[:, hd, :].T) * s
        logits = np.where(allowed[hd], logits, -np.inf)
        m = logits.max(axis=1, keepdims=True)
        p = np.exp(logits - m)
        out[:, hd, :] = (p @ v64[:, hd, :]) / p.sum(axis=1, keepdims=True)
    return out


def joint_segments(w):
    """Token ranges of the joint sequence [cond | video | audio | text].

    Returns dict name -> (start, stop).  'video_stream' spans cond + video,
    the tokens the audio-video cross-attention sees on the video side.
    """
    frame = w["H"] * w["W"]
    n_c = w.get("n_cond_frames", 0) * frame
    n_v = w["T"] * frame
    n_a = w.get("n_audio", 0)
    n_t = w.get("n_text", 0)
    a0 = n_c + n_v
    return dict(cond=(0, n_c), video=(n_c, a0), video_stream=(0, a0),
                audio=(a0, a0 + n_a), text=(a0 + n_a, a0 + n_a + n_t))
