"""Oracle cross-check: pure-Python loop versions for tiny inputs.

TEST INFRASTRUCTURE.  Written independently of the numpy oracle (no shared
helpers) so that the two can be compared: scalar math.cos / math.sin /
math.exp, explicit loops, Python's sorted() for the block order.  Only for
inputs with a few thousand scalars.
"""
import math


def rope_token(vec, t, h, w, split, theta):
    """Rotate one head vector (list of floats) at position (t, h, w)."""
    out = list(vec)
    base = 0
    for p, width in zip((t, h, w), split):
        for i in range(width // 2):
            ang = p * theta ** (-(2.0 * i) / width)
            c, s = math.cos(ang), math.sin(ang)
            a, b = out[base + 2 * i], out[base + 2 * i + 1]
            out[base + 2 * i] = a * c - b * s
            out[base + 2 * i + 1] = a * s + b * c
        base += width
    return out


def sequence_positions(T, H, W, n_cond_frames, n_audio, n_text, scale_num, scale_den):
    """List of (t, h, w) or None (text) per token in [cond|video|audio|text]."""
    out = []
    for c in range(n_cond_frames):
        for hh in range(H):
            for ww in range(W):
                out.append((float(c - n_cond_frames), float(hh), float(ww)))
    for t in range(T):
        for hh in range(H):
            for ww in range(W):
                out.append((float(t), float(hh), float(ww)))
    for j in range(n_audio):
        out.append((j * scale_num / scale_den, 0.0, 0.0))
    for _ in range(n_text):
        out.append(None)
    return out


def attention_row(qv, keys, vals, scale):
    """One query's attention output over lists of key / value vectors."""
    logits = [scale * sum(a * b for a, b in zip(qv, kv)) for kv in keys]
    m = max(logits)
    e = [math.exp(x - m) for x in logits]
    tot = sum(e)
    d = len(vals[0])
    return [sum(e[j] * vals[j][c] for j in range(len(vals))) / tot for c in range(d)]


def blocks(T, H, W, zone, block):
    """Token lists per block id, built by walking zones then blocks."""
    ZT, ZH, ZW = zone
    BT, BH, BW = block
    res = []
    for zt in range(T // ZT):
        for zh in range(H // ZH):
            for zw in range(W // ZW):
                for bt in range(ZT // BT):
                    for bh in range(ZH // BH):
                        for bw in range(ZW // BW):
                            toks = []
                            for a in range(BT):
                                for b in range(BH):
                                    for c in range(BW):
                                        t = zt * ZT + bt * BT + a
                                        h = zh * ZH + bh * BH + b
                                        w = zw * ZW + bw * BW + c
                                        toks.append((t * H + h) * W + w)
                            res.append(toks)
    return res


def select_row(probs, k, p):
    """Selected block ids of one row: the longer of the top-k and top-p prefixes."""
    n = len(probs)
    order = sorted(range(n), key=lambda j: (-probs[j], j))
    if p >= 1.0:
        n_p = n
    else:
        run = 0.0
        n_p = n
        for r, j in enumerate(order):
            run += probs[j]
            if run >= p:
                n_p = r + 1
                break
    K = max(min(k, n), n_p)
    return set(order[:K])


def block_probs_row(qbar, kbars, scale):
    logits = [scale * sum(a * b for a, b in zip(qbar, kb)) for kb in kbars]
    m = max(logits)
    e = [math.exp(x - m) for x in logits]
    tot = sum(e)
    return [x / tot for x in e]
