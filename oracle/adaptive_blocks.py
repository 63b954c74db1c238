"""Oracle: content-adaptive 3D block shapes for block-sparse attention, fp64.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the bench's CPU
baseline may import this module; the product path never does.

Sources (Prism page, xyznot.com 2610.05416):
  * "Ideas clave": the token volume is cut into 8 x 8 x 8 macro-zones; each
    zone measures its directional content variation from the channel variance
    of the video values and from the audio-to-video cross-attention norms
    (the dual-guidance variation indicator); each zone then picks one of 16
    candidate block shapes whose volumes are 64, 128 or 256 tokens.
  * "Metodo" section 1: per axis d in {T, H, W}, the value features averaged
    over the other two axes at each position i along d give the directional
    variance sigma2_{v,d}(m), averaged over the D channels; its share of the
    three axes is r_{v,d}(m).  The audio norms a = ||h_hat||_2 (cached from the
    previous layer) give a coupling strength abar(m) in [0, 1] and a normalised
    directional variance vhat_{a,d}(m); g_d = r_{v,d} + abar * vhat_{a,d} + eps.
  * "Metodo" section 2: the volume B(m) comes from a normalised density rho(m)
    against tau_128 = 0.5 and tau_256 = 0.25; minimising
    sum_d g_d (b_d^2 - 1) subject to prod_d b_d = B gives b_d ~ g_d^(-1/2), in
    log2 space l*_d = -log2(g_d)/2 + (S + sum_d' log2(g_d')/2) / 3 with
    S = log2 B; the zone's shape is the candidate of volume B nearest to l* in
    Euclidean distance.
  * "Limitaciones": self-attention runs before cross-attention in a block, so
    the audio norms are those of the previous layer (an input here).
  * "Metodo" section 3: blocks are mean-pooled and selected exactly as with
    uniform blocks (oracle.block_sparse), only with blocks of 64, 128 or 256
    tokens.

Readings where the page is silent (also listed in the design notes):
  * candidates: the boxes whose edges lie in {2, 4, 8} with volume 64, 128 or
    256 -- exactly 16 (7, 6 and 3); ordered by volume, then by (b_T, b_H, b_W)
    lexicographically; distance ties go to the first in that order;
  * D counts every channel of the values (heads x head_dim);
  * rho(m) = E(m) / max_m' E(m') with E(m) = sum_d sigma2_{v,d}(m), the zone's
    directional variance energy; rho >= 0.5 gives 64, rho >= 0.25 gives 128,
    otherwise 256 (all zones 256 when every E is zero);
  * abar(m) = (mean of a over the zone) / (largest zone mean), 0 when all
    norms are zero or no norms are given;
  * vhat_{a,d}(m) = sigma2_{a,d}(m) / sum_d' sigma2_{a,d'}(m), the directional
    variance of a built as sigma2_{v,d} with one channel, normalised like
    r_{v,d}; a zone whose total variance is zero contributes 0 (for r and vhat);
  * eps = 1e-6;
  * blocks inside a zone are numbered in raster (t, h, w) order of their
    position, tokens inside a block in raster order, zones in raster order.
"""
import numpy as np

ZONE = (8, 8, 8)
TAU_128 = 0.5
TAU_256 = 0.25
EPS = 1e-6
VOLUMES = (64, 128, 256)


def candidate_shapes():
    """The 16 candidate shapes (b_T, b_H, b_W), ordered by volume, then
    lexicographically."""
    out = []
    for vol in VOLUMES:
        for bt in (2, 4, 8):
            for bh in (2, 4, 8):
                for bw in (2, 4, 8):
                    if bt * bh * bw == vol:
                        out.append((bt, bh, bw))
    return out


def zone_grid(T, H, W):
    """Zones along each axis; the grid must be a whole number of zones."""
    ZT, ZH, ZW = ZONE
    assert T % ZT == 0 and H % ZH == 0 and W % ZW == 0, "grid must be whole 8 x 8 x 8 zones"
    return T // ZT, H // ZH, W // ZW


def zone_view(x, T, H, W):
    """x [T*H*W, C] in raster order -> [nz, 8, 8, 8, C], zones in raster order."""
    nzt, nzh, nzw = zone_grid(T, H, W)
    ZT, ZH, ZW = ZONE
    c = x.shape[1]
    y = np.asarray(x, dtype=np.float64).reshape(nzt, ZT, nzh, ZH, nzw, ZW, c)
    return y.transpose(0, 2, 4, 1, 3, 5, 6).reshape(nzt * nzh * nzw, ZT, ZH, ZW, c)


def directional_variance(z):
    """sigma2_d for one zone z [Z_T, Z_H, Z_W, C] ("Metodo" section 1): the
    mean over channels of the variance, over the positions i along axis d, of
    the channel mean over the other two axes at i.  Returns [3] fp64."""
    out = np.empty(3)
    for d in range(3):
        other = tuple(a for a in range(3) if a != d)
        vbar = z.mean(axis=other)                 # [Z_d, C]
        mu = vbar.mean(axis=0)                    # [C], the zone's channel mean
        out[d] = ((vbar - mu) ** 2).mean(axis=0).mean()
    return out


def _share(s2):
    """Rows of s2 [nz, 3] divided by their sum; rows that sum to zero give 0."""
    tot = s2.sum(axis=1, keepdims=True)
    with np.errstate(invalid="ignore", divide="ignore"):
        return np.where(tot > 0.0, s2 / np.where(tot > 0.0, tot, 1.0), 0.0)


def variation_indicator(v, a, T, H, W, eps=EPS):
    """Per zone quantities of "Metodo" sections 1-2 (readings in the header).

    v [T*H*W, heads, hd] (any float dtype, read as fp64); a [T*H*W] audio
    norms or None.  Returns a dict of fp64 arrays over zones: sigma2_v [nz, 3],
    r_v [nz, 3], energy [nz], rho [nz], a_mean [nz], sigma2_a [nz, 3],
    v_hat [nz, 3], a_bar [nz], g [nz, 3]."""
    n = T * H * W
    vz = zone_view(np.asarray(v).reshape(n, -1), T, H, W)
    nz = vz.shape[0]
    s2v = np.stack([directional_variance(vz[m]) for m in range(nz)])
    r_v = _share(s2v)
    energy = s2v.sum(axis=1)
    emax = energy.max()
    rho = energy / emax if emax > 0.0 else np.zeros(nz)
    if a is None:
        a_mean = np.zeros(nz)
        s2a = np.zeros((nz, 3))
    else:
        az = zone_view(np.asarray(a, dtype=np.float64).reshape(n, 1), T, H, W)
        a_mean = az.reshape(nz, -1).mean(axis=1)
        s2a = np.stack([directional_variance(az[m]) for m in range(nz)])
    amax = a_mean.max()
    a_bar = a_mean / amax if amax > 0.0 else np.zeros(nz)
    v_hat = _share(s2a)
    g = r_v + a_bar[:, None] * v_hat + eps
    return dict(sigma2_v=s2v, r_v=r_v, energy=energy, rho=rho, a_mean=a_mean, sigma2_a=s2a, v_hat=v_hat,
                a_bar=a_bar, g=g)


def volume(rho):
    """B(m) from rho(m) against tau_128 and tau_256 ("Metodo" section 2)."""
    rho = np.asarray(rho, dtype=np.float64)
    return np.where(rho >= TAU_128, 64, np.where(rho >= TAU_256, 128, 256)).astype(np.int64)


def ell_star(g, B):
    """Continuous optimum of the edge lengths in log2 space ("Metodo"
    section 2): l*_d = -log2(g_d)/2 + (log2 B + sum_d' log2(g_d')/2) / 3."""
    lg = np.log2(np.asarray(g, dtype=np.float64))
    S = np.log2(np.asarray(B, dtype=np.float64))
    return -0.5 * lg + ((S + 0.5 * lg.sum(axis=-1)) / 3.0)[..., None]


def nearest_shape(ell, B):
    """Index into candidate_shapes() of the volume-B candidate nearest to ell
    (Euclidean distance of log2 edge lengths); ties to the earlier one."""
    cands = candidate_shapes()
    best, best_d = -1, np.inf
    for i, s in enumerate(cands):
        if s[0] * s[1] * s[2] != B:
            continue
        d = sum((np.log2(s[a]) - ell[a]) ** 2 for a in range(3))
        if d < best_d:
            best, best_d = i, d
    return best


def zone_shapes(v, a, T, H, W, eps=EPS):
    """Candidate index of every zone and the indicator it came from."""
    ind = variation_indicator(v, a, T, H, W, eps)
    B = volume(ind["rho"])
    ell = ell_star(ind["g"], B)
    codes = np.array([nearest_shape(ell[m], int(B[m])) for m in range(len(B))], dtype=np.int64)
    ind.update(volume=B, ell=ell)
    return codes, ind


def adaptive_block_tokens(T, H, W, codes):
    """Token lists of the blocks of every zone for the given candidate codes.

    Returns (blocks, zone_of_block): blocks is a list of int64 arrays of
    raster token indices, numbered zone by zone (zones in raster order),
    blocks inside a zone in raster order of their position, tokens inside a
    block in raster order."""
    nzt, nzh, nzw = zone_grid(T, H, W)
    ZT, ZH, ZW = ZONE
    cands = candidate_shapes()
    blocks, zone_of = [], []
    m = 0
    for zt in range(nzt):
        for zh in range(nzh):
            for zw in range(nzw):
                bt, bh, bw = cands[int(codes[m])]
                for pt in range(ZT // bt):
                    for ph in range(ZH // bh):
                        for pw in range(ZW // bw):
                            t0, h0, w0 = zt * ZT + pt * bt, zh * ZH + ph * bh, zw * ZW + pw * bw
                            tt, hh, ww = np.meshgrid(np.arange(t0, t0 + bt), np.arange(h0, h0 + bh),
                                                     np.arange(w0, w0 + bw), indexing="ij")
                            blocks.append(((tt * H + hh) * W + ww).reshape(-1).astype(np.int64))
                            zone_of.append(m)
                m += 1
    return blocks, np.array(zone_of, dtype=np.int64)


def ragged_means(x, blocks):
    """fp64 mean over each block's tokens, per head: [h, nb, d]."""
    x64 = np.asarray(x, dtype=np.float64)
    return np.stack([x64[b].mean(axis=0) for b in blocks], axis=1)


def token_norms(x):
    """a_t = ||x_t||_2 over all heads and channels of one token ("Metodo"
    section 1: the norm of the audio-to-video cross-attention output)."""
    x64 = np.asarray(x, dtype=np.float64)
    return np.sqrt((x64.reshape(x64.shape[0], -1) ** 2).sum(axis=1))


def ragged_sparse_attention(q, k, v, blocks, mask, scale=None, query_blocks=None, heads=None):
    """Attention of each query over the keys of its block's selected blocks.

    blocks from adaptive_block_tokens; mask [h, nb, nb] bool.  Returns
    {(head, qblock): O [len(block), d] fp64}; row r belongs to token
    blocks[qblock][r]."""
    q64 = np.asarray(q, dtype=np.float64)
    k64 = np.asarray(k, dtype=np.float64)
    v64 = np.asarray(v, dtype=np.float64)
    d = q64.shape[2]
    s = np.float64(1.0 / np.sqrt(d)) if scale is None else np.float64(scale)
    hs = range(q64.shape[1]) if heads is None else heads
    qbs = range(len(blocks)) if query_blocks is None else query_blocks
    out = {}
    for hd in hs:
        for i in qbs:
            sel = np.nonzero(mask[hd, i])[0]
            keys = np.concatenate([blocks[j] for j in sel])
            logits = (q64[blocks[i], hd, :] @ k64[keys, hd, :].T) * s
            mx = logits.max(axis=1, keepdims=True)
            p = np.exp(logits - mx)
            out[(hd, i)] = (p @ v64[keys, hd, :]) / p.sum(axis=1, keepdims=True)
    return out
