"""Seeded synthetic inputs for every workload.

This module draws random tensors and nothing else: it holds none of the
method's arithmetic (no positions, no rotations, no attention, no pooling).
Both the product path and the oracle consume the tensors it returns; the
oracle always receives exactly the bytes the GPU consumed.

Draws use a torch.Generator seeded with the workload's seed on the device the
tensors are made on, so a (seed, device type) pair always gives the same bytes.
"""
import math

import torch

from .configs import layout_counts, n_tokens

_DTYPES = {"fp32": torch.float32, "bf16": torch.bfloat16}


def _gen(seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def joint_inputs(w, device="cpu"):
    """Q, K, V of one joint sequence [N, heads, head_dim] in the workload dtype.

    Entries are N(0, 1) drawn in fp32 (Q, then K, then V), multiplied by
    `input_scale`, then rounded to the workload dtype by round-to-nearest-even.
    With `outlier_frac` > 0 a seeded set of round(frac * N) tokens (one set for
    all three tensors, drawn after V) is multiplied by `outlier_gain` before
    rounding.  Returns a dict with q, k, v and the outlier token indices.
    """
    n = n_tokens(w)
    shape = (n, w["heads"], w["head_dim"])
    g = _gen(w["seed"], device)
    q = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    k = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    v = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if w.get("input_scale", 1.0) != 1.0:
        s = float(w["input_scale"])
        q.mul_(s), k.mul_(s), v.mul_(s)
    idx = torch.empty(0, dtype=torch.long, device=device)
    frac = float(w.get("outlier_frac", 0.0))
    if frac > 0.0:
        m = int(round(frac * n))
        idx = torch.randperm(n, generator=g, device=device)[:m]
        gain = float(w["outlier_gain"])
        q[idx] *= gain
        k[idx] *= gain
        v[idx] *= gain
    dt = _DTYPES[w["dtype"]]
    return dict(q=q.to(dt).contiguous(), k=k.to(dt).contiguous(), v=v.to(dt).contiguous(),
                outliers=idx)


def _gaussian_transfer(n, sigma, device):
    """Fourier transfer of a periodic Gaussian blur of std `sigma` samples."""
    f = torch.fft.fftfreq(n, device=device, dtype=torch.float64)
    return torch.exp(-0.5 * (2.0 * math.pi * f * sigma) ** 2).to(torch.float32)


def _smooth_fields(n_ch, T, H, W, length, g, device, chunk=256):
    """Standardised Gaussian random fields, [T*H*W, n_ch] fp32.

    White N(0,1) noise per channel on the periodic T x H x W grid, blurred by
    a Gaussian of std length/sqrt(2) per axis (so the field's covariance is
    exp(-r^2 / (2 length^2))), then shifted and scaled per channel to mean 0,
    variance 1.  `length` is one number or a (t, h, w) triple.
    """
    lt, lh, lw = (length,) * 3 if isinstance(length, (int, float)) else tuple(length)
    ht = _gaussian_transfer(T, lt / math.sqrt(2.0), device)[:, None, None]
    hh = _gaussian_transfer(H, lh / math.sqrt(2.0), device)[None, :, None]
    hw = _gaussian_transfer(W, lw / math.sqrt(2.0), device)[: W // 2 + 1][None, None, :]
    tf = ht * hh * hw
    out = torch.empty((T * H * W, n_ch), dtype=torch.float32, device=device)
    for c0 in range(0, n_ch, chunk):
        c1 = min(n_ch, c0 + chunk)
        white = torch.randn((c1 - c0, T, H, W), generator=g, device=device, dtype=torch.float32)
        spec = torch.fft.rfftn(white, dim=(1, 2, 3))
        spec *= tf
        f = torch.fft.irfftn(spec, s=(T, H, W), dim=(1, 2, 3)).reshape(c1 - c0, -1)
        f -= f.mean(dim=1, keepdim=True)
        f /= f.std(dim=1, keepdim=True)
        out[:, c0:c1] = f.t()
        del white, spec, f
    return out


def sparse_inputs(w, device="cpu"):
    """Q, K, V [T*H*W, heads, head_dim] bf16 in raster (t, h, w) token order.

    Q and K share one smooth field F, V uses an independent field G; each
    tensor adds its own N(0, noise_std^2) noise.  Draw order: F, G, then the
    noise for Q, K, V.  Rounded to bf16 by round-to-nearest-even.
    """
    T, H, W = w["T"], w["H"], w["W"]
    h, d = w["heads"], w["head_dim"]
    n = T * H * W
    g = _gen(w["seed"], device)
    F = _smooth_fields(h * d, T, H, W, w["field_length"], g, device)
    G = _smooth_fields(h * d, T, H, W, w["field_length"], g, device)
    s = float(w["noise_std"])
    dt = _DTYPES[w["dtype"]]
    out = {}
    for name, base in (("q", F), ("k", F), ("v", G)):
        x = torch.randn((n, h * d), generator=g, device=device, dtype=torch.float32)
        x.mul_(s).add_(base)
        out[name] = x.reshape(n, h, d).to(dt).contiguous()
        del x
    del F, G
    return out


def _blob(T, H, W, hc, wc, radius, device):
    """exp(-((h - hc)^2 + (w - wc)^2) / (2 radius^2)) on the grid, [T, H, W] fp32,
    the same in every frame."""
    hh = torch.arange(H, device=device, dtype=torch.float32)[:, None]
    ww = torch.arange(W, device=device, dtype=torch.float32)[None, :]
    b = torch.exp(-((hh - hc) ** 2 + (ww - wc) ** 2) / (2.0 * radius * radius))
    return b[None].expand(T, H, W)


def adaptive_inputs(w, device="cpu"):
    """Q, K, V [T*H*W, heads, head_dim] bf16 in raster order and per-token
    audio norms a [T*H*W] fp32 >= 0 for the content-adaptive block shapes.

    Q and K are as in sparse_inputs (one shared smooth field F of length
    `field_length`, own noise).  V is a quiet background plus a compact
    foreground: `bg_amp` times a smooth field of length `bg_length`, plus a
    Gaussian blob (radius `fg_radius` tokens in h, w, the same in every frame)
    times a field with per-axis lengths `fg_lengths` (t, h, w), plus noise.
    The audio norms are a second blob (radius `audio_radius`, peak
    `audio_gain`) pulsing along t with period `audio_period`:
    a = gain * blob * (1 + cos(2 pi t / period)) / 2, a sound source inside
    the frame.  Draw order: the two blob centres (uniform in h, w), F, the
    background field, the foreground field, then the noise of Q, K and V.
    """
    T, H, W = w["T"], w["H"], w["W"]
    h, d = w["heads"], w["head_dim"]
    n = T * H * W
    g = _gen(w["seed"], device)
    ctr = torch.rand(4, generator=g, device=device, dtype=torch.float64).tolist()
    F = _smooth_fields(h * d, T, H, W, w["field_length"], g, device)
    bg = _smooth_fields(h * d, T, H, W, w["bg_length"], g, device)
    fg = _smooth_fields(h * d, T, H, W, w["fg_lengths"], g, device)
    env = _blob(T, H, W, ctr[0] * H, ctr[1] * W, w["fg_radius"], device).reshape(n, 1)
    V = bg.mul_(float(w["bg_amp"])).add_(fg.mul_(env))
    del fg
    s = float(w["noise_std"])
    dt = _DTYPES[w["dtype"]]
    out = {}
    for name, base in (("q", F), ("k", F), ("v", V)):
        x = torch.randn((n, h * d), generator=g, device=device, dtype=torch.float32)
        x.mul_(s).add_(base)
        out[name] = x.reshape(n, h, d).to(dt).contiguous()
        del x
    del F, V
    tt = torch.arange(T, device=device, dtype=torch.float32)[:, None, None]
    pulse = 0.5 * (1.0 + torch.cos(2.0 * math.pi * tt / float(w["audio_period"])))
    a = _blob(T, H, W, ctr[2] * H, ctr[3] * W, w["audio_radius"], device) * pulse * float(w["audio_gain"])
    out["a"] = a.reshape(n).contiguous()
    return out


def normal_tensors(shapes, seed, dtype="bf16", device="cpu", scale=1.0):
    """One seeded generator, N(0, scale^2) fp32 tensors of the given shapes in
    order, each rounded to `dtype` by round-to-nearest-even."""
    g = _gen(seed, device)
    dt = _DTYPES[dtype]
    out = []
    for shape in shapes:
        x = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
        if scale != 1.0:
            x.mul_(float(scale))
        out.append(x.to(dt).contiguous())
    return out


def upstream_grad(w, device="cpu"):
    """dO of a backward pass over a workload's joint sequence: N(0, 1) entries
    [N, heads, head_dim] from a generator seeded with the workload's seed +
    7919 (a stream separate from Q, K, V), rounded to the workload dtype."""
    shape = (n_tokens(w), w["heads"], w["head_dim"])
    return normal_tensors([shape], int(w["seed"]) + 7919, w["dtype"], device)[0]


def segment_sizes(w):
    """Token counts per modality (re-exported for callers)."""
    return layout_counts(w)
