"""Oracle: block pooling, hybrid top-k / top-p block selection and sparse
attention over the selected key blocks, fp64.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the bench's CPU
baseline may import this module; the product path never does.

Sources (Prism page, xyznot.com 2610.05416):
  * "Ideas clave", macro-zone partitioning: the token volume is cut into
    Z_T x Z_H x Z_W = 8 x 8 x 8 macro-zones.
  * "Ideas clave", hybrid top-k / top-p selection; "Metodo" section 3:
    key blocks are mean-pooled into representatives K_j, scored against the
    query blocks to give block probabilities P_i, and the attended set is
    S_i = TopK(P_i, k) union TopP(P_i, p); sparse attention with an online
    softmax then runs only over S_i.
  * "Problema y motivacion": block representatives come from mean pooling.
SkyReels-V4 analysis (paper.rainbus.top 2602.21818), workflow step 6: the
Refiner uses video sparse attention for about 3x less attention cost.

Steps, in the order the Prism page gives them:
  1. blocks: uniform b_T x b_H x b_W tiles inside each macro-zone;
  2. pool: per head, fp64 mean of each block's query rows and key rows;
  3. score: L_ij = <Qbar_i, Kbar_j> * s, s = 1/sqrt(d);
  4. P_i = softmax_j(L_ij) over all key blocks;
  5. order blocks by P descending, ties to the lower block id;
  6. S_i = the first K_i blocks of that order, K_i = max(min(k, nb), n_p),
     n_p = the smallest n >= 1 whose running sum of P reaches p (all blocks
     when p >= 1 or when rounding keeps the total below p); since top-k and
     top-p are both prefixes of one order, their union is the longer prefix;
  7. attention of each query over the keys of the blocks in S_i only.
Readings where the page is silent are listed in the design notes: query
pooling equals averaging per-query logits (by linearity), the temperature is
1/sqrt(d), the nucleus includes the block that crosses p, no block is forced.
"""
import numpy as np


def block_token_index(T, H, W, zone=(8, 8, 8), block=(4, 4, 4)):
    """Token indices (raster t, h, w order) of every block, [nb, vol] int64.

    Block id j = zone_id * blocks_per_zone + local_id, where zones are
    numbered in raster (zt, zh, zw) order and blocks inside a zone in raster
    (bt, bh, bw) order.  Tokens inside a block are listed in raster order.
    """
    ZT, ZH, ZW = zone
    BT, BH, BW = block
    assert T % ZT == 0 and H % ZH == 0 and W % ZW == 0
    assert ZT % BT == 0 and ZH % BH == 0 and ZW % BW == 0
    nz = (T // ZT, H // ZH, W // ZW)
    nbz = (ZT // BT, ZH // BH, ZW // BW)
    rows = []
    for zt in range(nz[0]):
        for zh in range(nz[1]):
            for zw in range(nz[2]):
                for bt in range(nbz[0]):
                    for bh in range(nbz[1]):
                        for bw in range(nbz[2]):
                            t0 = zt * ZT + bt * BT
                            h0 = zh * ZH + bh * BH
                            w0 = zw * ZW + bw * BW
                            tt, hh, ww = np.meshgrid(np.arange(t0, t0 + BT), np.arange(h0, h0 + BH),
                                                     np.arange(w0, w0 + BW), indexing="ij")
                            rows.append(((tt * H + hh) * W + ww).reshape(-1))
    return np.stack(rows).astype(np.int64)


def block_means(x, idx):
    """fp64 mean over each block's tokens, per head: [h, nb, d]."""
    x64 = np.asarray(x, dtype=np.float64)
    g = x64[idx]                      # [nb, vol, h, d]
    return g.mean(axis=1).transpose(1, 0, 2).copy()


def block_probs(qbar, kbar, scale=None):
    """P [h, nqb, nkb]: row softmax of the pooled block logits (fp64)."""
    d = qbar.shape[2]
    s = np.float64(1.0 / np.sqrt(d)) if scale is None else np.float64(scale)
    logits = np.einsum("hid,hjd->hij", qbar, kbar) * s
    m = logits.max(axis=2, keepdims=True)
    e = np.exp(logits - m)
    return e / e.sum(axis=2, keepdims=True)


def select_blocks(P, top_k, top_p):
    """Hybrid top-k / top-p selection on block probabilities P [h, nqb, nkb].

    Returns (mask [h, nqb, nkb] bool, counts [h, nqb] int64, margin dict).
    margin['cumsum'] is min over rows of |running sum - p| at the two sums
    that bracket the cut (how far rounding is from changing n_p);
    margin['rel_gap'] is min over rows of the relative gap between the last
    selected and first unselected probability (how far rounding is from
    reordering across the cut).
    """
    P = np.asarray(P, dtype=np.float64)
    h, nq, nk = P.shape
    mask = np.zeros((h, nq, nk), dtype=bool)
    counts = np.zeros((h, nq), dtype=np.int64)
    kk = min(max(int(top_k), 0), nk)
    min_cs = np.inf
    min_gap = np.inf
    rows = np.arange(nq)[:, None]
    for hd in range(h):
        # stable sort of -P: descending probability, equal values keep the lower id first
        order = np.argsort(-P[hd], axis=1, kind="stable")
        ps = np.take_along_axis(P[hd], order, axis=1)
        cs = np.cumsum(ps, axis=1)
        if top_p >= 1.0:
            n_p = np.full(nq, nk)
        else:
            reached = cs >= top_p
            hit = reached.any(axis=1)
            first = np.argmax(reached, axis=1)
            n_p = np.where(hit, first + 1, nk)
            r = np.flatnonzero(hit)
            if r.size:
                at = cs[r, n_p[r] - 1]
                min_cs = min(min_cs, float(np.min(np.abs(at - top_p))))
                r2 = r[n_p[r] >= 2]
                if r2.size:
                    before = cs[r2, n_p[r2] - 2]
                    min_cs = min(min_cs, float(np.min(np.abs(before - top_p))))
        K = np.maximum(kk, n_p)
        counts[hd] = K
        sel = np.arange(nk)[None, :] < K[:, None]          # prefix of the order
        mask[hd][np.broadcast_to(rows, order.shape)[sel], order[sel]] = True
        cut = np.flatnonzero(K < nk)
        if cut.size:
            a = ps[cut, K[cut] - 1]
            b = ps[cut, K[cut]]
            with np.errstate(divide="ignore", invalid="ignore"):
                g = np.where(a > 0, (a - b) / a, np.inf)
            min_gap = min(min_gap, float(np.min(g)))
    return mask, counts, dict(cumsum=float(min_cs), rel_gap=float(min_gap))


def pack_mask(mask):
    """Bit j of word j // 32 in row (h, i) is set iff block j is selected.

    Returns uint32 [h, nqb, ceil(nkb / 32)], the layout the library exports.
    """
    h, nq, nk = mask.shape
    nw = (nk + 31) // 32
    words = np.zeros((h, nq, nw), dtype=np.uint64)
    j = np.arange(nk)
    for b in range(nk):
        words[:, :, b // 32] |= mask[:, :, b].astype(np.uint64) << np.uint64(b % 32)
    del j
    return words.astype(np.uint32)


def block_sparse_attention(q, k, v, idx, mask, scale=None, query_blocks=None, heads=None):
    """Attention of each query over the keys of its block's selected blocks.

    q, k, v [N, h, d] in raster order; idx [nb, vol] from block_token_index;
    mask [h, nqb, nkb].  Returns {(head, qblock): O [vol, d] fp64} for the
    requested query blocks (all by default) and heads (all by default); row r
    of O belongs to token idx[qblock, r].
    """
    q64 = np.asarray(q, dtype=np.float64)
    k64 = np.asarray(k, dtype=np.float64)
    v64 = np.asarray(v, dtype=np.float64)
    d = q64.shape[2]
    s = np.float64(1.0 / np.sqrt(d)) if scale is None else np.float64(scale)
    nb = idx.shape[0]
    hs = range(q64.shape[1]) if heads is None else heads
    qbs = range(nb) if query_blocks is None else query_blocks
    out = {}
    for hd in hs:
        for i in qbs:
            sel = np.nonzero(mask[hd, i])[0]
            keys = idx[sel].reshape(-1)
            qi = q64[idx[i], hd, :]
            logits = (qi @ k64[keys, hd, :].T) * s
            m = logits.max(axis=1, keepdims=True)
            p = np.exp(logits - m)
            out[(hd, i)] = (p @ v64[keys, hd, :]) / p.sum(axis=1, keepdims=True)
    return out
