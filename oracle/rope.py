"""Oracle: time-shifted 3D rotary position embedding, fp64.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the bench's CPU
baseline may import this module; the product path never does.

Sources (pages on SkyReels-V4):
  * SkyReels-V4 analysis (paper.rainbus.top 2602.21818), workflow step 1:
    conditioning latents are concatenated along time and told apart from the
    generation targets by negative temporal indices.
  * same page, novelty 4 (time-shifted 3D RoPE, extends to several
    references) and novelty 5 (audio RoPE frequency scaled by 21/218 so 218
    audio tokens line up with 21 video frames).
  * trdm.cn SkyReels-V4 article, section 2.2: the frequency scaling of the
    rotary embedding aligns the two temporal resolutions.

Readings where the pages are silent (each one is also listed in the design
notes): base theta = 10000; head_dim is split into t | h | w slices in that
order; each slice rotates adjacent pairs (2i, 2i+1) by p_a * theta^(-2i/d_a);
audio token j sits at temporal position j * T/N_audio with h = w = 0 and uses
the video's temporal bands; conditioning frame c of n sits at t = c - n
(so one frame sits at t = -1); text tokens are not rotated.
"""
import numpy as np


def axis_frequencies(width, theta):
    """omega_i = theta^(-2 i / width) for i < width / 2 (fp64)."""
    i = np.arange(width // 2, dtype=np.float64)
    return np.power(np.float64(theta), -2.0 * i / np.float64(width))


def token_positions(w):
    """Per-token (t, h, w) positions and a rotate flag, in sequence order.

    Order is [cond | video | audio | text].  Returns (pos [N, 3] fp64,
    rotated [N] bool).  Positions of text tokens are 0 and rotated is False.
    """
    T, H, W = w["T"], w["H"], w["W"]
    n_cf = w.get("n_cond_frames", 0)
    n_a = w.get("n_audio", 0)
    n_t = w.get("n_text", 0)
    rows = []
    for c in range(n_cf):
        t = c - n_cf
        for hh in range(H):
            for ww in range(W):
                rows.append((t, hh, ww, True))
    for t in range(T):
        for hh in range(H):
            for ww in range(W):
                rows.append((t, hh, ww, True))
    num, den = w.get("audio_scale", (T, max(n_a, 1)))
    step = np.float64(num) / np.float64(den)
    for j in range(n_a):
        rows.append((np.float64(j) * step, 0.0, 0.0, True))
    for _ in range(n_t):
        rows.append((0.0, 0.0, 0.0, False))
    pos = np.array([r[:3] for r in rows], dtype=np.float64).reshape(-1, 3)
    rot = np.array([r[3] for r in rows], dtype=bool)
    return pos, rot


def rope_angles(pos, split, theta):
    """Angles phi[N, d/2]: pair i of axis a gets p_a * omega_{a,i}."""
    parts = []
    for a, width in enumerate(split):
        if width == 0:
            continue
        om = axis_frequencies(width, theta)
        parts.append(pos[:, a:a + 1] * om[None, :])
    return np.concatenate(parts, axis=1) if parts else np.zeros((pos.shape[0], 0))


def apply_rope(x, pos, rotated, split, theta):
    """Rotate x [N, heads, d] (any float dtype) and return an fp64 copy.

    Pair (2i, 2i+1) of the whole head vector, i < d/2, is turned by angle
    phi[n, i]: (x0, x1) -> (x0 cos - x1 sin, x0 sin + x1 cos).  Tokens with
    rotated == False are copied unchanged.
    """
    out = np.array(x, dtype=np.float64, copy=True)
    d = out.shape[2]
    assert sum(split) == d and all(s % 2 == 0 for s in split)
    phi = rope_angles(pos[rotated], split, theta)          # [n_rot, d/2]
    c = np.cos(phi)[:, None, :]
    s = np.sin(phi)[:, None, :]
    sel = out[rotated]
    x0 = sel[:, :, 0::2]
    x1 = sel[:, :, 1::2]
    y = np.empty_like(sel)
    y[:, :, 0::2] = x0 * c - x1 * s
    y[:, :, 1::2] = x0 * s + x1 * c
    out[rotated] = y
    return out


def rope_table(w):
    """Host table the way the pages' positions define it: per distinct axis
    position, the fp64 (cos, sin) of every pair of that axis.

    Returns a dict of arrays keyed by 'cond_t', 'video_t', 'h', 'w', 'audio_t',
    each [n_positions, width/2, 2] fp64.  Used to pin the library's host table
    builder after its fp32 rounding.
    """
    T, H, W = w["T"], w["H"], w["W"]
    d_t, d_h, d_w = w["split"]
    th = w["theta"]
    n_cf = w.get("n_cond_frames", 0)
    n_a = w.get("n_audio", 0)
    num, den = w.get("audio_scale", (T, max(n_a, 1)))

    def tab(p, width):
        ang = np.asarray(p, dtype=np.float64)[:, None] * axis_frequencies(width, th)[None, :]
        return np.stack([np.cos(ang), np.sin(ang)], axis=-1)

    out = {
        "cond_t": tab([c - n_cf for c in range(n_cf)], d_t),
        "video_t": tab(list(range(T)), d_t),
        "h": tab(list(range(H)), d_h),
        "w": tab(list(range(W)), d_w),
        "audio_t": tab([np.float64(j) * (np.float64(num) / np.float64(den)) for j in range(n_a)], d_t),
    }
    return out
