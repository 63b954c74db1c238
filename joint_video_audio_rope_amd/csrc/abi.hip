// C ABI: argument checks, workspace plans, the host RoPE table builder and
// kernel dispatch.  Every check runs before the first HIP call so a failed
// call enqueues nothing.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>
#include <vector>

#include "internal.hpp"

using namespace mmdit;

namespace {

thread_local std::string g_err;

mmdit_status fail(mmdit_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return st;
}

mmdit_status hip_fail(hipError_t e, const char* what) {
    return fail(MMDIT_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    const char* x = static_cast<const char*>(a);
    const char* y = static_cast<const char*>(b);
    return x < y + nb && y < x + na;
}

size_t elem_size(int dtype) { return dtype == MMDIT_BF16 ? 2 : 4; }

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// softmax_scale 0 selects the usual 1/sqrt(head_dim) (the scale of the
// attention the pages describe; SkyReels-V4 analysis, workflow step 3).
double resolve_scale(double s, int hd) { return s == 0.0 ? 1.0 / std::sqrt((double)hd) : s; }
float resolve_scale(float s, int hd) { return s == 0.f ? (float)(1.0 / std::sqrt((double)hd)) : s; }

bool scale_ok(double s) { return std::isfinite(s) && s >= 0.0 && std::isfinite((float)s); }

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// ---- dense attention plan ----------------------------------------------------
// Workspace of a bf16 attention: fp16 V^T, the partial maxima of V (its
// prescale exponents) and, for split key ranges, the partial O and (m, l).
struct AttnPlan {
    int64_t n_pad, n_q_pad;
    int32_t q_tile, q_tiles, kv_tiles, splits, tiles_per_split;
    size_t vt_bytes, vmax_bytes, part_o_bytes, part_ml_bytes;
    size_t total() const { return vt_bytes + vmax_bytes + part_o_bytes + part_ml_bytes; }
};

AttnPlan plan_attn(int64_t n_q, int64_t n_kv, int heads, int hd, int dtype) {
    AttnPlan p{};
    if (dtype != MMDIT_BF16) return p;   // the fp32 kernel needs no workspace
    p.n_pad = round_up(n_kv, kTileN);
    p.q_tile = (n_kv <= kShortKv || n_q <= kDenseQ) ? kShortQ : kDenseQ;
    p.q_tiles = (int32_t)((n_q + p.q_tile - 1) / p.q_tile);
    p.n_q_pad = (int64_t)p.q_tiles * p.q_tile;
    p.kv_tiles = (int32_t)(p.n_pad / kTileN);
    const int64_t base = (int64_t)p.q_tiles * heads;
    int splits = 1;
    if (base > 0 && base < 512) {
        const int64_t want = (1024 + base - 1) / base;
        const int64_t cap = std::max<int64_t>(1, p.kv_tiles / 4);
        splits = (int)std::min(want, cap);
    }
    p.tiles_per_split = (p.kv_tiles + splits - 1) / splits;
    p.splits = (p.kv_tiles + p.tiles_per_split - 1) / p.tiles_per_split;
    p.vt_bytes = align256((size_t)heads * hd * p.n_pad * 2);
    p.vmax_bytes = align256((size_t)heads * kVmaxParts * 4);
    if (p.splits > 1) {
        p.part_o_bytes = align256((size_t)p.splits * heads * p.n_q_pad * hd * 4);
        p.part_ml_bytes = align256((size_t)p.splits * heads * p.n_q_pad * 2 * 4);
    }
    return p;
}

mmdit_status check_attn_args(const void* q, int64_t n_q, const void* k, const void* v,
                             int64_t n_kv, int heads, int hd, int dtype, float scale,
                             const float* o, const char* who) {
    if (dtype != MMDIT_FP32 && dtype != MMDIT_BF16)
        return fail(MMDIT_ERR_INVALID_ARG, "%s: dtype %d is neither MMDIT_FP32 nor MMDIT_BF16", who,
                    dtype);
    if (hd != 64 && hd != 128)
        return fail(MMDIT_ERR_UNSUPPORTED, "%s: head_dim %d (supported: 64, 128)", who, hd);
    if (heads < 1) return fail(MMDIT_ERR_INVALID_ARG, "%s: heads %d < 1", who, heads);
    if (n_q < 0) return fail(MMDIT_ERR_INVALID_ARG, "%s: n_q %lld < 0", who, (long long)n_q);
    if (n_kv < 1) return fail(MMDIT_ERR_INVALID_ARG, "%s: n_kv %lld < 1", who, (long long)n_kv);
    if (!scale_ok(scale))
        return fail(MMDIT_ERR_INVALID_ARG, "%s: softmax_scale must be finite and >= 0 (0: 1/sqrt(head_dim))",
                    who);
    const int64_t lim = (int64_t)1 << 31;
    if (n_q * heads >= lim || n_kv * heads >= lim)
        return fail(MMDIT_ERR_UNSUPPORTED, "%s: tokens * heads must stay below 2^31", who);
    // per-lane byte offsets into the [heads][head_dim][tokens] operands are 32-bit
    if (n_q >= ((int64_t)1 << 24) || n_kv >= ((int64_t)1 << 24))
        return fail(MMDIT_ERR_UNSUPPORTED, "%s: at most 2^24 - 1 tokens per side", who);
    if (!k || !v) return fail(MMDIT_ERR_INVALID_ARG, "%s: null k or v", who);
    if (!aligned16(k) || !aligned16(v))
        return fail(MMDIT_ERR_INVALID_ARG, "%s: k and v must be 16-byte aligned", who);
    if (n_q > 0) {
        if (!q || !o) return fail(MMDIT_ERR_INVALID_ARG, "%s: null q or o", who);
        if (!aligned16(q) || !aligned16(o))
            return fail(MMDIT_ERR_INVALID_ARG, "%s: q and o must be 16-byte aligned", who);
        const size_t es = elem_size(dtype);
        const size_t ob = (size_t)n_q * heads * hd * 4;
        if (overlaps(o, ob, q, (size_t)n_q * heads * hd * es) ||
            overlaps(o, ob, k, (size_t)n_kv * heads * hd * es) ||
            overlaps(o, ob, v, (size_t)n_kv * heads * hd * es))
            return fail(MMDIT_ERR_INVALID_ARG, "%s: output aliases an input", who);
    }
    return MMDIT_OK;
}

// Enqueue one attention after its arguments and workspace were checked.
mmdit_status run_attn(const void* q, int64_t n_q, const void* k, const void* v, int64_t n_kv,
                      int heads, int hd, int dtype, float scale, float* o, float* lse, char* ws,
                      const AttnPlan& p, hipStream_t s, const char* who) {
    if (n_q == 0) return MMDIT_OK;
    hipError_t e;
    if (dtype == MMDIT_FP32) {
        e = launch_attn_fp32((const float*)q, n_q, (const float*)k, (const float*)v, n_kv, heads,
                             hd, scale, o, lse, s);
        return e == hipSuccess ? MMDIT_OK : hip_fail(e, who);
    }
    AttnArgs a{};
    a.q = (const __bf16*)q;
    a.k = (const __bf16*)k;
    a.vt = (const _Float16*)ws;
    a.o = o;
    a.lse = lse;
    uint32_t* vmax = (uint32_t*)(ws + p.vt_bytes);
    a.vmax = vmax;
    a.part_o = p.splits > 1 ? (float*)(ws + p.vt_bytes + p.vmax_bytes) : nullptr;
    a.part_ml = p.splits > 1 ? (float*)(ws + p.vt_bytes + p.vmax_bytes + p.part_o_bytes) : nullptr;
    a.n_q = n_q;
    a.n_kv = n_kv;
    a.n_pad = p.n_pad;
    a.n_q_pad = p.n_q_pad;
    a.heads = heads;
    a.q_tile = p.q_tile;
    a.q_tiles = p.q_tiles;
    a.splits = p.splits;
    a.tiles_per_split = p.tiles_per_split;
    a.kv_tiles = p.kv_tiles;
    a.scale_log2 = (float)((double)scale * 1.4426950408889634);
    e = launch_v_absmax((const __bf16*)v, n_kv, heads, hd, vmax, s);
    if (e != hipSuccess) return hip_fail(e, who);
    e = launch_vt_dense((const __bf16*)v, n_kv, p.n_pad, heads, hd, vmax, (_Float16*)ws, s);
    if (e != hipSuccess) return hip_fail(e, who);
    e = launch_attn_bf16(a, hd, s);
    if (e != hipSuccess) return hip_fail(e, who);
    if (p.splits > 1) {
        e = launch_attn_combine(a, hd, s);
        if (e != hipSuccess) return hip_fail(e, who);
    }
    return MMDIT_OK;
}

// The RoPE-fused joint attention: the attention workspace, then room for the
// rotated K when the caller does not take it.
size_t rope_attn_ws_bytes(int64_t n, int heads, int hd) {
    return plan_attn(n, n, heads, hd, MMDIT_BF16).total() + align256((size_t)n * heads * hd * 2);
}

// ---- dense attention backward plan -------------------------------------------------
struct BwdPlan {
    int64_t n_q_pad = 0, n_kv_pad = 0;
    size_t off_dd = 0, off_ls2 = 0, off_qt = 0, off_dot = 0, off_kt = 0, total = 0;
};

// bf16: D and lse2 [heads][n_q_pad] fp32, Q^T and dO^T [heads][hd][n_q_pad] and
// K^T [heads][hd][n_kv_pad] bf16 (pads: multiples of 64).  fp32: D [heads][n_q].
BwdPlan plan_bwd(int64_t n_q, int64_t n_kv, int heads, int hd, int dtype) {
    BwdPlan p;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off += align256(bytes);
        return o;
    };
    if (dtype == MMDIT_FP32) {
        p.n_q_pad = n_q;
        p.off_dd = take((size_t)heads * n_q * 4);
    } else {
        p.n_q_pad = round_up(n_q, kTileN);
        p.n_kv_pad = round_up(n_kv, kTileN);
        p.off_dd = take((size_t)heads * p.n_q_pad * 4);
        p.off_ls2 = take((size_t)heads * p.n_q_pad * 4);
        p.off_qt = take((size_t)heads * hd * p.n_q_pad * 2);
        p.off_dot = take((size_t)heads * hd * p.n_q_pad * 2);
        p.off_kt = take((size_t)heads * hd * p.n_kv_pad * 2);
    }
    p.total = off;
    return p;
}

// ---- RoPE ----------------------------------------------------------------------
struct RopePlan {
    size_t floats = 0;
    RopeArgs args{};
};

mmdit_status plan_rope(const mmdit_rope_desc* d, int dtype, RopePlan* out) {
    if (!d) return fail(MMDIT_ERR_INVALID_ARG, "rope: null descriptor");
    if (d->heads < 1) return fail(MMDIT_ERR_INVALID_ARG, "rope: heads %d < 1", d->heads);
    if (d->head_dim < 8 || d->head_dim % 8)
        return fail(MMDIT_ERR_INVALID_ARG, "rope: head_dim %d must be a positive multiple of 8",
                    d->head_dim);
    if (d->d_t < 0 || d->d_h < 0 || d->d_w < 0 || d->d_t % 8 || d->d_h % 8 || d->d_w % 8)
        return fail(MMDIT_ERR_UNSUPPORTED, "rope: slice widths (%d, %d, %d) must be multiples of 8",
                    d->d_t, d->d_h, d->d_w);
    if (d->d_t + d->d_h + d->d_w != d->head_dim)
        return fail(MMDIT_ERR_INVALID_ARG, "rope: d_t + d_h + d_w != head_dim");
    if (!(d->theta > 0.0) || !std::isfinite(d->theta))
        return fail(MMDIT_ERR_INVALID_ARG, "rope: theta must be positive and finite");
    if (d->n_segs < 1 || d->n_segs > MMDIT_MAX_SEGMENTS)
        return fail(MMDIT_ERR_INVALID_ARG, "rope: n_segs %d outside 1..%d", d->n_segs,
                    MMDIT_MAX_SEGMENTS);
    if (!d->segs) return fail(MMDIT_ERR_INVALID_ARG, "rope: null segment array");
    if (d->n_tokens < 0) return fail(MMDIT_ERR_INVALID_ARG, "rope: n_tokens < 0");
    if (dtype != MMDIT_FP32 && dtype != MMDIT_BF16)
        return fail(MMDIT_ERR_INVALID_ARG, "rope: bad dtype %d", dtype);

    std::vector<std::pair<int64_t, int64_t>> ranges;
    RopeArgs& a = out->args;
    a.heads = d->heads;
    a.head_dim = d->head_dim;
    a.d_t = d->d_t;
    a.d_h = d->d_h;
    a.d_w = d->d_w;
    const int epc = dtype == MMDIT_BF16 ? 8 : 4;
    a.chunks_per_token = d->heads * d->head_dim / epc;
    int64_t pairs = 0;   // float2 entries
    int64_t chunks = 0;
    int ns = 0;
    for (int i = 0; i < d->n_segs; ++i) {
        const mmdit_segment& s = d->segs[i];
        if (s.offset < 0 || s.count < 0 || s.offset + s.count > d->n_tokens)
            return fail(MMDIT_ERR_INVALID_ARG, "rope: segment %d outside the token range", i);
        if (s.count > 0) ranges.push_back({s.offset, s.offset + s.count});
        if (s.kind == MMDIT_SEG_TEXT) continue;
        if (s.kind != MMDIT_SEG_VIDEO && s.kind != MMDIT_SEG_AUDIO)
            return fail(MMDIT_ERR_INVALID_ARG, "rope: segment %d has unknown kind %d", i, s.kind);
        RopeSeg rs{};
        rs.kind = s.kind;
        rs.offset = s.offset;
        if (s.kind == MMDIT_SEG_VIDEO) {
            if (s.T < 1 || s.H < 1 || s.W < 1 || (int64_t)s.T * s.H * s.W != s.count)
                return fail(MMDIT_ERR_INVALID_ARG, "rope: video segment %d needs count == T*H*W >= 1",
                            i);
            rs.T = s.T, rs.H = s.H, rs.W = s.W;
            rs.tab_t = (int32_t)pairs;
            pairs += (int64_t)s.T * (d->d_t / 2);
            rs.tab_h = (int32_t)pairs;
            pairs += (int64_t)s.H * (d->d_h / 2);
            rs.tab_w = (int32_t)pairs;
            pairs += (int64_t)s.W * (d->d_w / 2);
        } else {
            if (!std::isfinite(s.t_scale))
                return fail(MMDIT_ERR_INVALID_ARG, "rope: audio segment %d t_scale not finite", i);
            rs.T = rs.H = rs.W = 1;
            rs.tab_t = (int32_t)pairs;
            pairs += s.count * (d->d_t / 2);
        }
        const int64_t c = s.count * a.chunks_per_token;
        if (c >= ((int64_t)1 << 31))
            return fail(MMDIT_ERR_UNSUPPORTED, "rope: segment %d has 2^31 or more chunks", i);
        rs.chunk_begin = chunks;
        chunks += c;
        rs.chunk_end = chunks;
        if (c > 0) a.seg[ns++] = rs;
    }
    if (pairs >= ((int64_t)1 << 30)) return fail(MMDIT_ERR_UNSUPPORTED, "rope: table too large");
    std::sort(ranges.begin(), ranges.end());
    for (size_t i = 1; i < ranges.size(); ++i)
        if (ranges[i].first < ranges[i - 1].second)
            return fail(MMDIT_ERR_INVALID_ARG, "rope: segments overlap");
    a.n_segs = ns;
    a.total_chunks = chunks;
    out->floats = (size_t)pairs * 2;
    return MMDIT_OK;
}

// ---- block sparse plan ------------------------------------------------------------
struct SparsePlan {
    SparseGeom g{};
    int32_t chunk_rows;   // query blocks whose logits are computed and selected at once
    size_t off_qbar, off_kbar, off_scores, off_mask, off_count, off_base, off_vt, off_kimg, off_vmax, off_order,
        total;
};

// Query blocks per chunk of block logits: whole 128-row tiles of the score
// GEMM within kScoreChunkBytes for all heads, or every block when they fit.
int32_t score_chunk_rows(int64_t nb, int32_t heads) {
    int64_t c = (int64_t)kScoreChunkBytes / ((int64_t)heads * nb * 8);
    c = c / 128 * 128;
    if (c < 128) c = 128;
    return (int32_t)(c < nb ? c : nb);
}

// Workspace layout of a block-sparse call (shared by the plan and the size
// query): fp64 block means, fp64 scores, selection bitmask and counts, block
// first tokens, per-block fp16 V^T and per-block K tile images, the partial
// maxima of V (its prescale exponents), the attention kernel's group order.
void sparse_layout(int64_t nb, int32_t heads, int32_t hd, SparsePlan* p) {
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off += align256(bytes);
        return o;
    };
    p->off_qbar = take((size_t)heads * nb * hd * 8);
    p->off_kbar = take((size_t)heads * nb * hd * 8);
    p->chunk_rows = score_chunk_rows(nb, heads);
    p->off_scores = take((size_t)heads * p->chunk_rows * nb * 8);
    p->off_mask = take((size_t)heads * nb * ((nb + 31) / 32) * 4);
    p->off_count = take((size_t)heads * nb * 4);
    p->off_base = take((size_t)nb * 4);
    p->off_vt = take((size_t)heads * nb * hd * kTileN * 2);
    p->off_kimg = take((size_t)heads * nb * hd * kTileN * 2);
    p->off_vmax = take((size_t)heads * kVmaxParts * 4);
    p->off_order = take((size_t)heads * stream_groups(nb) * 4);
    p->total = off;
}

mmdit_status plan_sparse(int T, int H, int W, int heads, int hd, const mmdit_sparse_desc* sp,
                         SparsePlan* p) {
    if (!sp) return fail(MMDIT_ERR_INVALID_ARG, "block_sparse: null sparse descriptor");
    if (T < 1 || H < 1 || W < 1 || heads < 1)
        return fail(MMDIT_ERR_INVALID_ARG, "block_sparse: T, H, W and heads must be >= 1");
    if (hd != 128) return fail(MMDIT_ERR_UNSUPPORTED, "block_sparse: head_dim %d (supported: 128)", hd);
    for (int a = 0; a < 3; ++a)
        if (sp->zone[a] < 1 || sp->block[a] < 1 || sp->zone[a] % sp->block[a])
            return fail(MMDIT_ERR_INVALID_ARG,
                        "block_sparse: zone sizes must be positive multiples of block sizes");
    if (T % sp->zone[0] || H % sp->zone[1] || W % sp->zone[2])
        return fail(MMDIT_ERR_INVALID_ARG, "block_sparse: T, H, W must be multiples of the zone");
    if (sp->block[0] * sp->block[1] * sp->block[2] != kTileN)
        return fail(MMDIT_ERR_UNSUPPORTED, "block_sparse: block volume must be %d", kTileN);
    if (sp->top_k < 0) return fail(MMDIT_ERR_INVALID_ARG, "block_sparse: top_k < 0");
    if (!(sp->top_p >= 0.0 && sp->top_p <= 1.0))
        return fail(MMDIT_ERR_INVALID_ARG, "block_sparse: top_p must lie in [0, 1]");
    if (sp->wait_limit < 0 || sp->wait_limit > kSpinLimit)
        return fail(MMDIT_ERR_INVALID_ARG, "block_sparse: wait_limit must lie in [0, %d]", kSpinLimit);
    const int64_t n = (int64_t)T * H * W;
    if (n * heads >= ((int64_t)1 << 31))
        return fail(MMDIT_ERR_UNSUPPORTED, "block_sparse: tokens * heads must stay below 2^31");
    const int64_t nb = n / kTileN;
    if (nb > kSelMax)
        return fail(MMDIT_ERR_UNSUPPORTED, "block_sparse: %lld blocks per head (max %d)", (long long)nb, kSelMax);
    SparseGeom& g = p->g;
    g.T = T, g.H = H, g.W = W;
    g.ZT = sp->zone[0], g.ZH = sp->zone[1], g.ZW = sp->zone[2];
    g.BT = sp->block[0], g.BH = sp->block[1], g.BW = sp->block[2];
    g.nzh = H / g.ZH, g.nzw = W / g.ZW;
    g.bz_t = g.ZT / g.BT, g.bz_h = g.ZH / g.BH, g.bz_w = g.ZW / g.BW;
    g.nb = (int32_t)nb;
    g.heads = heads;
    sparse_layout(nb, heads, hd, p);
    return MMDIT_OK;
}

mmdit_status check_ws(const void* ws, size_t ws_bytes, size_t need, const char* who) {
    if (need == 0) return MMDIT_OK;
    if (!ws) return fail(MMDIT_ERR_WORKSPACE, "%s: workspace of %zu bytes required, got null", who, need);
    if (ws_bytes < need)
        return fail(MMDIT_ERR_WORKSPACE, "%s: workspace %zu bytes < required %zu", who, ws_bytes, need);
    if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0)
        return fail(MMDIT_ERR_INVALID_ARG, "%s: workspace must be 256-byte aligned", who);
    return MMDIT_OK;
}

// Content-adaptive blocks: the extra workspace after the uniform layout of
// the nt = T*H*W / 64 tiles (zone statistics, shape codes, tile tables).
struct AdaptivePlan {
    size_t off_part, off_audio, off_code, off_tdim, off_lead, off_tblock, off_nblocks, total;
};

AdaptivePlan adaptive_layout(size_t start, int64_t nt, int32_t heads, int32_t hd) {
    AdaptivePlan p{};
    size_t off = start;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off += align256(bytes);
        return o;
    };
    const int64_t nz = nt / kZoneTiles;
    p.off_part = take((size_t)nz * zone_stat_chunks(heads, hd) * 3 * 8);
    p.off_audio = take((size_t)nz * 4 * 8);
    p.off_code = take((size_t)nz);
    p.off_tdim = take((size_t)nt);
    p.off_lead = take((size_t)nt * 4);
    p.off_tblock = take((size_t)nt * 4);
    p.off_nblocks = take(4);
    p.total = off;
    return p;
}

// Outputs and the audio input of an adaptive call (all optional).
struct AdaptiveCall {
    const float* a;
    uint8_t* zone_shape;
    int32_t* tile_block;
    int32_t* n_blocks;
};

mmdit_status run_sparse(const void* q, const void* k, const void* v, int32_t T, int32_t H, int32_t W,
                        int32_t heads, int32_t head_dim, const mmdit_sparse_desc* sp, double softmax_scale,
                        float* o, float* lse, uint32_t* sel_mask, int32_t* sel_count, void* ws, size_t ws_bytes,
                        void* stream, const char* who, const AdaptiveCall* ad = nullptr) {
    SparsePlan p{};
    mmdit_status st = plan_sparse(T, H, W, heads, head_dim, sp, &p);
    if (st != MMDIT_OK) return st;
    AdaptivePlan ap{};
    if (ad) {
        if ((int64_t)p.g.nb / kZoneTiles > kMaxZones)
            return fail(MMDIT_ERR_UNSUPPORTED, "%s: %d zones (max %d)", who, p.g.nb / kZoneTiles, kMaxZones);
        ap = adaptive_layout(p.total, p.g.nb, heads, head_dim);
        p.total = ap.total;
    }
    if (!scale_ok(softmax_scale))
        return fail(MMDIT_ERR_INVALID_ARG, "%s: softmax_scale must be finite and >= 0 (0: 1/sqrt(head_dim))",
                    who);
    softmax_scale = resolve_scale(softmax_scale, head_dim);
    if (!q || !k || !v || !o) return fail(MMDIT_ERR_INVALID_ARG, "%s: null q, k, v or o", who);
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
        return fail(MMDIT_ERR_INVALID_ARG, "%s: q, k, v, o must be 16-byte aligned", who);
    if ((sel_mask && !aligned16(sel_mask)) || (sel_count && (reinterpret_cast<uintptr_t>(sel_count) & 3u)))
        return fail(MMDIT_ERR_INVALID_ARG, "%s: misaligned sel_mask or sel_count", who);
    const size_t n = (size_t)T * H * W;
    const size_t ib = n * heads * head_dim * 2, ob = n * heads * head_dim * 4;
    if (overlaps(o, ob, q, ib) || overlaps(o, ob, k, ib) || overlaps(o, ob, v, ib))
        return fail(MMDIT_ERR_INVALID_ARG, "%s: output aliases an input", who);
    if (lse) {
        const size_t lb = n * heads * 4;
        if (overlaps(lse, lb, o, ob) || overlaps(lse, lb, q, ib) || overlaps(lse, lb, k, ib) ||
            overlaps(lse, lb, v, ib))
            return fail(MMDIT_ERR_INVALID_ARG, "%s: lse aliases o or an input", who);
    }
    if (ad) {
        const size_t n4 = n * 4, nt = (size_t)p.g.nb;
        if ((ad->a && (reinterpret_cast<uintptr_t>(ad->a) & 3u)) ||
            (ad->tile_block && (reinterpret_cast<uintptr_t>(ad->tile_block) & 3u)) ||
            (ad->n_blocks && (reinterpret_cast<uintptr_t>(ad->n_blocks) & 3u)))
            return fail(MMDIT_ERR_INVALID_ARG, "%s: a_norm, tile_block and n_blocks must be 4-byte aligned", who);
        if (ad->a && (overlaps(o, ob, ad->a, n4) || (lse && overlaps(lse, n * heads * 4, ad->a, n4))))
            return fail(MMDIT_ERR_INVALID_ARG, "%s: an output aliases a_norm", who);
        const void* outs[3] = {ad->zone_shape, ad->tile_block, ad->n_blocks};
        const size_t sizes[3] = {nt / kZoneTiles, nt * 4, 4};
        for (int i = 0; i < 3; ++i)
            if (outs[i] && (overlaps(outs[i], sizes[i], o, ob) || overlaps(outs[i], sizes[i], q, ib) ||
                            overlaps(outs[i], sizes[i], k, ib) || overlaps(outs[i], sizes[i], v, ib) ||
                            (ad->a && overlaps(outs[i], sizes[i], ad->a, n4))))
                return fail(MMDIT_ERR_INVALID_ARG, "%s: zone_shape, tile_block or n_blocks aliases a tensor", who);
    }
    if ((st = check_ws(ws, ws_bytes, p.total, who)) != MMDIT_OK) return st;
    char* w = (char*)ws;
    SparseWs sw{};
    sw.qbar = (double*)(w + p.off_qbar);
    sw.kbar = (double*)(w + p.off_kbar);
    sw.scores = (double*)(w + p.off_scores);
    sw.mask = (uint32_t*)(w + p.off_mask);
    sw.count = (int32_t*)(w + p.off_count);
    sw.base = (int32_t*)(w + p.off_base);
    sw.vt = (_Float16*)(w + p.off_vt);
    sw.kimg = (__bf16*)(w + p.off_kimg);
    sw.vmax = (uint32_t*)(w + p.off_vmax);
    sw.order = (int32_t*)(w + p.off_order);
    hipStream_t s = (hipStream_t)stream;
    hipError_t e;
    if (ad) {
        AdaptiveWs aw{};
        aw.part = (double*)(w + ap.off_part);
        aw.audio = (double*)(w + ap.off_audio);
        aw.code = ad->zone_shape ? ad->zone_shape : (uint8_t*)(w + ap.off_code);
        aw.base = sw.base;
        aw.tdim = (uint8_t*)(w + ap.off_tdim);
        aw.lead = (int32_t*)(w + ap.off_lead);
        aw.tblock = ad->tile_block ? ad->tile_block : (int32_t*)(w + ap.off_tblock);
        aw.nblocks = ad->n_blocks ? ad->n_blocks : (int32_t*)(w + ap.off_nblocks);
        sw.tdim = aw.tdim;
        sw.lead = aw.lead;
        if ((e = launch_zone_stats(p.g, (const __bf16*)v, ad->a, head_dim, aw, s)) != hipSuccess)
            return hip_fail(e, "block_sparse_adaptive zone statistics");
        if ((e = launch_zone_shapes(p.g, head_dim, aw, s)) != hipSuccess)
            return hip_fail(e, "block_sparse_adaptive shapes");
    }
    if ((e = launch_block_pool(p.g, (const __bf16*)q, (const __bf16*)k, head_dim, sw, s)) != hipSuccess)
        return hip_fail(e, "block_sparse pool");
    if ((e = launch_v_absmax((const __bf16*)v, (int64_t)T * H * W, heads, head_dim, sw.vmax, s)) != hipSuccess)
        return hip_fail(e, "block_sparse v prescale");
    if ((e = launch_vt_blocks(p.g, (const __bf16*)k, (const __bf16*)v, head_dim, sw, s)) != hipSuccess)
        return hip_fail(e, "block_sparse vt");
    for (int r0 = 0; r0 < p.g.nb; r0 += p.chunk_rows) {
        const int rows = std::min(p.chunk_rows, p.g.nb - r0);
        if ((e = launch_block_scores(p.g, head_dim, softmax_scale, sw, r0, rows, s)) != hipSuccess)
            return hip_fail(e, "block_sparse scores");
        if ((e = launch_block_select(p.g, sp->top_k, sp->top_p, sw, r0, rows, sel_mask, sel_count, s)) !=
            hipSuccess)
            return hip_fail(e, "block_sparse select");
    }
    if ((e = launch_group_order(p.g, kStreamGroup, sw.mask, sw.order, s)) != hipSuccess)
        return hip_fail(e, "block_sparse group order");
    if ((e = launch_sparse_attn(p.g, (const __bf16*)q, head_dim,
                                (float)(softmax_scale * 1.4426950408889634), sw, o, lse,
                                sp->wait_limit ? sp->wait_limit : kSpinLimit, s)) != hipSuccess)
        return hip_fail(e, "block_sparse attention");
    return MMDIT_OK;
}

// Workspace of a block-sparse backward: D and lse2 [heads][n] fp32, the
// transposed block images Q^T, dO^T, K^T [heads][nb][hd * 64] bf16, the
// transposed selection bitmask [heads][nb][ceil(nb/32)], the dispatch
// orders of the query-block and key-block groups [heads][groups] i32, and
// the block row images Q, dO, K, V [heads][nb][64 * hd] bf16.
struct SparseBwdPlan {
    size_t off_dd, off_ls2, off_qt, off_dot, off_kt, off_maskt, off_order_q, off_order_k, off_qi, off_doi, off_ki,
        off_vi, total;
};

SparseBwdPlan plan_sparse_bwd(int64_t n, int64_t nb, int32_t heads, int32_t hd) {
    SparseBwdPlan p{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off += align256(bytes);
        return o;
    };
    p.off_dd = take((size_t)heads * n * 4);
    p.off_ls2 = take((size_t)heads * n * 4);
    p.off_qt = take((size_t)heads * nb * hd * kTileN * 2);
    p.off_dot = take((size_t)heads * nb * hd * kTileN * 2);
    p.off_kt = take((size_t)heads * nb * hd * kTileN * 2);
    p.off_maskt = take((size_t)heads * nb * ((nb + 31) / 32) * 4);
    p.off_order_q = take((size_t)heads * ((nb + kBwdGroup - 1) / kBwdGroup) * 4);
    p.off_order_k = take((size_t)heads * ((nb + kBwdGroup - 1) / kBwdGroup) * 4);
    p.off_qi = take((size_t)heads * nb * hd * kTileN * 2);
    p.off_doi = take((size_t)heads * nb * hd * kTileN * 2);
    p.off_ki = take((size_t)heads * nb * hd * kTileN * 2);
    p.off_vi = take((size_t)heads * nb * hd * kTileN * 2);
    p.total = off;
    return p;
}

// Adaptive-shape backward: the tile table (first token and log2 edges of
// every 64-token tile), then the uniform backward's workspace over the tiles.
struct AdaptiveBwdPlan {
    size_t off_tbase, off_tdim, off_bwd, total;
    SparseBwdPlan bwd;
};

AdaptiveBwdPlan plan_adaptive_bwd(int64_t n, int32_t heads, int32_t hd) {
    AdaptiveBwdPlan p{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off += align256(bytes);
        return o;
    };
    p.off_tbase = take((size_t)(n / kTileN) * 4);
    p.off_tdim = take((size_t)(n / kTileN));
    p.bwd = plan_sparse_bwd(n, n / kTileN, heads, hd);
    p.off_bwd = take(p.bwd.total);
    p.total = off;
    return p;
}

// The kernels of a block-sparse backward over geometry g: uniform blocks, or
// (tbase, tdim set) the content-adaptive tiles of the grid.
mmdit_status run_sparse_bwd(const SparseGeom& g, const SparseBwdPlan& bp, const void* q, const void* k,
                            const void* v, const float* o, const float* lse, const void* d_o,
                            const uint32_t* sel_mask, float* dq, float* dk, float* dv, double softmax_scale,
                            const int32_t* tbase, const uint8_t* tdim, char* w, hipStream_t s, const char* who) {
    const int64_t n = (int64_t)g.T * g.H * g.W;
    const int heads = g.heads;
    const int head_dim = 128;
    SparseBwdArgs a{};
    a.q = (const __bf16*)q;
    a.k = (const __bf16*)k;
    a.v = (const __bf16*)v;
    a.d_o = (const __bf16*)d_o;
    a.qt_img = (const __bf16*)(w + bp.off_qt);
    a.dot_img = (const __bf16*)(w + bp.off_dot);
    a.kt_img = (const __bf16*)(w + bp.off_kt);
    a.q_img = (const __bf16*)(w + bp.off_qi);
    a.do_img = (const __bf16*)(w + bp.off_doi);
    a.k_img = (const __bf16*)(w + bp.off_ki);
    a.v_img = (const __bf16*)(w + bp.off_vi);
    a.mask = sel_mask;
    a.maskt = (const uint32_t*)(w + bp.off_maskt);
    a.ls2 = (const float*)(w + bp.off_ls2);
    a.dd = (const float*)(w + bp.off_dd);
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.tbase = tbase;
    a.tdim = tdim;
    a.order_q = (const int32_t*)(w + bp.off_order_q);
    a.order_k = (const int32_t*)(w + bp.off_order_k);
    a.scale = (float)softmax_scale;
    a.scale_log2 = (float)(softmax_scale * 1.4426950408889634);
    hipError_t e;
    if ((e = launch_bwd_rowterm(o, d_o, MMDIT_BF16, lse, n, n, heads, head_dim, (float*)a.dd, (float*)a.ls2, s)) !=
            hipSuccess ||
        (e = launch_block_timg(g, a.q, (__bf16*)a.qt_img, tbase, tdim, s)) != hipSuccess ||
        (e = launch_block_timg(g, a.d_o, (__bf16*)a.dot_img, tbase, tdim, s)) != hipSuccess ||
        (e = launch_block_timg(g, a.k, (__bf16*)a.kt_img, tbase, tdim, s)) != hipSuccess ||
        (e = launch_block_rimg(g, a.q, (__bf16*)a.q_img, tbase, tdim, s)) != hipSuccess ||
        (e = launch_block_rimg(g, a.d_o, (__bf16*)a.do_img, tbase, tdim, s)) != hipSuccess ||
        (e = launch_block_rimg(g, a.k, (__bf16*)a.k_img, tbase, tdim, s)) != hipSuccess ||
        (e = launch_block_rimg(g, a.v, (__bf16*)a.v_img, tbase, tdim, s)) != hipSuccess ||
        (e = launch_mask_transpose(g, sel_mask, (uint32_t*)a.maskt, s)) != hipSuccess ||
        (e = launch_group_order(g, kBwdGroup, sel_mask, (int32_t*)a.order_q, s)) != hipSuccess ||
        (e = launch_group_order(g, kBwdGroup, a.maskt, (int32_t*)a.order_k, s)) != hipSuccess ||
        (e = launch_sparse_bwd(g, a, s)) != hipSuccess)
        return hip_fail(e, who);
    return MMDIT_OK;
}

// ---- scratch of the allocation-free joint attention -------------------------------
// One array per GPU, in the library's code object: it exists on every device
// the library has launched a kernel on, until the process ends.  In host code
// `scratch` names a host-side stand-in, never the device memory; the device
// address comes from hipGetSymbolAddress, taken once per device (with that
// device current) and kept.
static __device__ __align__(256) char scratch[MMDIT_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

// The calling thread's current device's address of `scratch`.
mmdit_status scratch_address(void** out, const char* who) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, who);
    if (dev < 0 || dev >= kMaxDevices)
        return fail(MMDIT_ERR_UNSUPPORTED, "%s: device %d (at most %d devices)", who, dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, who);
        if (!p) return fail(MMDIT_ERR_HIP, "%s: no device address for the scratch array", who);
        g_scratch_dev[dev] = p;
    }
    *out = g_scratch_dev[dev];
    return MMDIT_OK;
}

}  // namespace

extern "C" {

int32_t mmdit_abi_version(void) { return MMDIT_ABI_VERSION; }

const char* mmdit_last_error(void) { return g_err.c_str(); }

size_t mmdit_rope3d_table_floats(const mmdit_rope_desc* desc) {
    RopePlan p;
    if (plan_rope(desc, MMDIT_BF16, &p) != MMDIT_OK) return 0;
    return p.floats;
}

mmdit_status mmdit_rope3d_build_table(const mmdit_rope_desc* d, float* host_table) {
    RopePlan p;
    mmdit_status st = plan_rope(d, MMDIT_BF16, &p);
    if (st != MMDIT_OK) return st;
    if (p.floats > 0 && !host_table) return fail(MMDIT_ERR_INVALID_ARG, "rope table: null output");
    size_t at = 0;
    // pair i of an axis of width w turns at position * theta^(-2i/w)
    auto axis = [&](double pos, int width) {
        for (int i = 0; i < width / 2; ++i) {
            const double om = std::pow(d->theta, -2.0 * i / (double)width);
            const double ang = pos * om;
            host_table[at++] = (float)std::cos(ang);
            host_table[at++] = (float)std::sin(ang);
        }
    };
    for (int i = 0; i < d->n_segs; ++i) {
        const mmdit_segment& s = d->segs[i];
        if (s.kind == MMDIT_SEG_VIDEO) {
            for (int t = 0; t < s.T; ++t) axis((double)(s.t0 + t), d->d_t);
            for (int h = 0; h < s.H; ++h) axis((double)h, d->d_h);
            for (int w = 0; w < s.W; ++w) axis((double)w, d->d_w);
        } else if (s.kind == MMDIT_SEG_AUDIO) {
            for (int64_t j = 0; j < s.count; ++j) axis((double)j * s.t_scale, d->d_t);
        }
    }
    return MMDIT_OK;
}

size_t mmdit_workspace_bytes(int32_t op, int64_t n_q, int64_t n_kv, int32_t heads,
                             int32_t head_dim, int32_t dtype, const mmdit_sparse_desc* sp) {
    if (heads < 1 || head_dim < 1 || n_q < 0 || n_kv < 0) return 0;
    if (op == MMDIT_OP_JOINT_ATTN) {
        if (n_kv < 1) return 0;
        return plan_attn(n_q, n_kv, heads, head_dim, dtype).total();
    }
    if (op == MMDIT_OP_JOINT_ATTN_ROPE) {
        if (n_q < 1) return 0;
        return rope_attn_ws_bytes(n_q, heads, head_dim);
    }
    if (op == MMDIT_OP_AV_CROSS_ATTN) {
        if (n_q < 1 || n_kv < 1) return 0;
        return plan_attn(n_q, n_kv, heads, head_dim, dtype).total() +
               plan_attn(n_kv, n_q, heads, head_dim, dtype).total();
    }
    if (op == MMDIT_OP_JOINT_ATTN_BWD) {
        if (n_kv < 1) return 0;
        return plan_bwd(n_q, n_kv, heads, head_dim, dtype).total;
    }
    if (op == MMDIT_OP_BLOCK_SPARSE_ATTN_BWD) {
        if (!sp) return 0;
        return plan_sparse_bwd(n_q, n_q / kTileN, heads, head_dim).total;
    }
    if (op == MMDIT_OP_BLOCK_SPARSE_ATTN) {
        if (!sp) return 0;
        // T, H, W are not known here; the layout depends on them only through nb.
        SparsePlan p;
        sparse_layout(n_q / kTileN, heads, head_dim, &p);
        return p.total;
    }
    if (op == MMDIT_OP_BLOCK_SPARSE_ATTN_ADAPTIVE_BWD) return plan_adaptive_bwd(n_q, heads, head_dim).total;
    if (op == MMDIT_OP_BLOCK_SPARSE_ATTN_ADAPTIVE) {
        SparsePlan p;
        sparse_layout(n_q / kTileN, heads, head_dim, &p);
        return adaptive_layout(p.total, n_q / kTileN, heads, head_dim).total;
    }
    return 0;
}

mmdit_status mmdit_rope3d(const mmdit_rope_desc* desc, const float* dev_table, void* q, void* k,
                          int32_t dtype, void* stream) {
    RopePlan p;
    mmdit_status st = plan_rope(desc, dtype, &p);
    if (st != MMDIT_OK) return st;
    if (p.args.total_chunks == 0) return MMDIT_OK;
    if (!q || !k || !dev_table) return fail(MMDIT_ERR_INVALID_ARG, "rope: null q, k or table");
    if (!aligned16(q) || !aligned16(k) || (reinterpret_cast<uintptr_t>(dev_table) & 7u))
        return fail(MMDIT_ERR_INVALID_ARG, "rope: q, k must be 16-byte and the table 8-byte aligned");
    const size_t bytes = (size_t)desc->n_tokens * desc->heads * desc->head_dim * elem_size(dtype);
    if (overlaps(q, bytes, k, bytes)) return fail(MMDIT_ERR_INVALID_ARG, "rope: q and k overlap");
    hipError_t e = launch_rope(p.args, dev_table, q, k, dtype, (hipStream_t)stream);
    return e == hipSuccess ? MMDIT_OK : hip_fail(e, "rope");
}

mmdit_status mmdit_joint_attn(const void* q, int64_t n_q, const void* k, const void* v,
                              int64_t n_kv, int32_t heads, int32_t head_dim, int32_t dtype,
                              float softmax_scale, float* o, void* ws, size_t ws_bytes,
                              void* stream) {
    mmdit_status st = check_attn_args(q, n_q, k, v, n_kv, heads, head_dim, dtype, softmax_scale,
                                      o, "joint_attn");
    if (st != MMDIT_OK) return st;
    const AttnPlan p = plan_attn(n_q, n_kv, heads, head_dim, dtype);
    if (n_q > 0 && (st = check_ws(ws, ws_bytes, p.total(), "joint_attn")) != MMDIT_OK) return st;
    softmax_scale = resolve_scale(softmax_scale, head_dim);
    return run_attn(q, n_q, k, v, n_kv, heads, head_dim, dtype, softmax_scale, o, nullptr, (char*)ws, p,
                    (hipStream_t)stream, "joint_attn");
}

mmdit_status mmdit_joint_attn_noalloc(const void* q, int64_t n_q, const void* k, const void* v, int64_t n_kv,
                                      int32_t heads, int32_t head_dim, int32_t dtype, float softmax_scale, float* o,
                                      void* stream) {
    const char* who = "joint_attn_noalloc";
    mmdit_status st = check_attn_args(q, n_q, k, v, n_kv, heads, head_dim, dtype, softmax_scale, o, who);
    if (st != MMDIT_OK) return st;
    const AttnPlan p = plan_attn(n_q, n_kv, heads, head_dim, dtype);
    if (p.total() > (size_t)MMDIT_NOALLOC_SCRATCH_BYTES)
        return fail(MMDIT_ERR_WORKSPACE,
                    "%s: these sizes need %zu bytes of scratch, more than its fixed %zu (use mmdit_joint_attn "
                    "with a workspace)", who, p.total(), (size_t)MMDIT_NOALLOC_SCRATCH_BYTES);
    if (n_q == 0) return MMDIT_OK;
    void* ws = nullptr;
    if (p.total() > 0 && (st = scratch_address(&ws, who)) != MMDIT_OK) return st;
    softmax_scale = resolve_scale(softmax_scale, head_dim);
    return run_attn(q, n_q, k, v, n_kv, heads, head_dim, dtype, softmax_scale, o, nullptr, (char*)ws, p,
                    (hipStream_t)stream, who);
}

mmdit_status mmdit_joint_attn_rope(const mmdit_rope_desc* desc, const float* dev_table, const void* q,
                                   const void* k, const void* v, int32_t dtype, float softmax_scale, float* o,
                                   void* q_rot, void* k_rot, void* ws, size_t ws_bytes, void* stream) {
    const char* who = "joint_attn_rope";
    RopePlan rp;
    mmdit_status st = plan_rope(desc, dtype, &rp);
    if (st != MMDIT_OK) return st;
    if (dtype != MMDIT_BF16)
        return fail(MMDIT_ERR_UNSUPPORTED, "%s: bf16 only (fp32: mmdit_rope3d, then mmdit_joint_attn)", who);
    const int64_t n = desc->n_tokens;
    const int heads = desc->heads, hd = desc->head_dim;
    if (n < 1) return fail(MMDIT_ERR_INVALID_ARG, "%s: n_tokens must be >= 1", who);
    if ((st = check_attn_args(q, n, k, v, n, heads, hd, dtype, softmax_scale, o, who)) != MMDIT_OK) return st;
    if (rp.floats > 0 && (!dev_table || (reinterpret_cast<uintptr_t>(dev_table) & 7u)))
        return fail(MMDIT_ERR_INVALID_ARG, "%s: the table must be a non-null 8-byte aligned device pointer", who);
    const size_t tb = (size_t)n * heads * hd * 2;
    if ((q_rot && !aligned16(q_rot)) || (k_rot && !aligned16(k_rot)))
        return fail(MMDIT_ERR_INVALID_ARG, "%s: q_rot and k_rot must be 16-byte aligned", who);
    const void* ins[4] = {q, k, v, o};
    const size_t isz[4] = {tb, tb, tb, tb * 2};
    for (void* out : {q_rot, k_rot}) {
        if (!out) continue;
        for (int j = 0; j < 4; ++j)
            if (overlaps(out, tb, ins[j], isz[j]))
                return fail(MMDIT_ERR_INVALID_ARG, "%s: q_rot and k_rot must not overlap q, k, v or o", who);
    }
    if (q_rot && k_rot && overlaps(q_rot, tb, k_rot, tb))
        return fail(MMDIT_ERR_INVALID_ARG, "%s: q_rot and k_rot overlap", who);
    const AttnPlan p = plan_attn(n, n, heads, hd, dtype);
    if ((st = check_ws(ws, ws_bytes, rope_attn_ws_bytes(n, heads, hd), who)) != MMDIT_OK) return st;
    if (ws_bytes && (overlaps(ws, rope_attn_ws_bytes(n, heads, hd), q_rot ? q_rot : ws, q_rot ? tb : 0) ||
                     overlaps(ws, rope_attn_ws_bytes(n, heads, hd), k_rot ? k_rot : ws, k_rot ? tb : 0)))
        return fail(MMDIT_ERR_INVALID_ARG, "%s: the workspace overlaps q_rot or k_rot", who);
    softmax_scale = resolve_scale(softmax_scale, hd);
    char* w = (char*)ws;
    hipStream_t s = (hipStream_t)stream;
    RopeFused rf{};
    rf.a = rp.args;
    rf.tab = reinterpret_cast<const float2*>(dev_table);
    rf.k = (const __bf16*)k;
    rf.k_out = k_rot ? (__bf16*)k_rot : (__bf16*)(w + p.total());
    rf.q_out = (__bf16*)q_rot;
    AttnArgs a{};
    a.q = (const __bf16*)q;
    a.k = rf.k_out;
    a.vt = (const _Float16*)w;
    uint32_t* vmax = (uint32_t*)(w + p.vt_bytes);
    a.vmax = vmax;
    a.part_o = p.splits > 1 ? (float*)(w + p.vt_bytes + p.vmax_bytes) : nullptr;
    a.part_ml = p.splits > 1 ? (float*)(w + p.vt_bytes + p.vmax_bytes + p.part_o_bytes) : nullptr;
    a.o = o;
    a.n_q = a.n_kv = n;
    a.n_pad = p.n_pad;
    a.n_q_pad = p.n_q_pad;
    a.heads = heads;
    a.q_tile = p.q_tile;
    a.q_tiles = p.q_tiles;
    a.splits = p.splits;
    a.tiles_per_split = p.tiles_per_split;
    a.kv_tiles = p.kv_tiles;
    a.scale_log2 = (float)((double)softmax_scale * 1.4426950408889634);
    hipError_t e;
    if ((e = launch_v_absmax((const __bf16*)v, n, heads, hd, vmax, s)) != hipSuccess ||
        (e = launch_vt_dense_rope((const __bf16*)v, n, p.n_pad, heads, hd, vmax, (_Float16*)w, rf, s)) !=
            hipSuccess ||
        (e = launch_attn_bf16_rope(a, hd, rf, s)) != hipSuccess ||
        (p.splits > 1 && (e = launch_attn_combine(a, hd, s)) != hipSuccess))
        return hip_fail(e, who);
    return MMDIT_OK;
}

mmdit_status mmdit_joint_attn_fwd(const void* q, int64_t n_q, const void* k, const void* v,
                                  int64_t n_kv, int32_t heads, int32_t head_dim, int32_t dtype,
                                  float softmax_scale, float* o, float* lse, void* ws, size_t ws_bytes,
                                  void* stream) {
    mmdit_status st = check_attn_args(q, n_q, k, v, n_kv, heads, head_dim, dtype, softmax_scale,
                                      o, "joint_attn_fwd");
    if (st != MMDIT_OK) return st;
    if (n_q > 0) {
        if (!lse || (reinterpret_cast<uintptr_t>(lse) & 3u))
            return fail(MMDIT_ERR_INVALID_ARG, "joint_attn_fwd: lse must be a 4-byte aligned pointer");
        const size_t lb = (size_t)n_q * heads * 4, es = elem_size(dtype);
        if (overlaps(lse, lb, o, (size_t)n_q * heads * head_dim * 4) ||
            overlaps(lse, lb, q, (size_t)n_q * heads * head_dim * es) ||
            overlaps(lse, lb, k, (size_t)n_kv * heads * head_dim * es) ||
            overlaps(lse, lb, v, (size_t)n_kv * heads * head_dim * es))
            return fail(MMDIT_ERR_INVALID_ARG, "joint_attn_fwd: lse aliases o or an input");
    }
    const AttnPlan p = plan_attn(n_q, n_kv, heads, head_dim, dtype);
    if (n_q > 0 && (st = check_ws(ws, ws_bytes, p.total(), "joint_attn_fwd")) != MMDIT_OK) return st;
    softmax_scale = resolve_scale(softmax_scale, head_dim);
    return run_attn(q, n_q, k, v, n_kv, heads, head_dim, dtype, softmax_scale, o, lse, (char*)ws, p,
                    (hipStream_t)stream, "joint_attn_fwd");
}

mmdit_status mmdit_joint_attn_bwd(const void* q, int64_t n_q, const void* k, const void* v,
                                  int64_t n_kv, int32_t heads, int32_t head_dim, int32_t dtype,
                                  float softmax_scale, const float* o, const float* lse, const void* d_o,
                                  float* dq, float* dk, float* dv, void* ws, size_t ws_bytes, void* stream) {
    const char* who = "joint_attn_bwd";
    mmdit_status st = check_attn_args(q, n_q, k, v, n_kv, heads, head_dim, dtype, softmax_scale, dq, who);
    if (st != MMDIT_OK) return st;
    if (!dk || !dv || !aligned16(dk) || !aligned16(dv))
        return fail(MMDIT_ERR_INVALID_ARG, "%s: dk and dv must be non-null and 16-byte aligned", who);
    const size_t es = elem_size(dtype);
    const size_t qb = (size_t)n_q * heads * head_dim, kb = (size_t)n_kv * heads * head_dim;
    if (n_q > 0) {
        if (!o || !d_o || !aligned16(o) || !aligned16(d_o))
            return fail(MMDIT_ERR_INVALID_ARG, "%s: o and d_o must be non-null and 16-byte aligned", who);
        if (!lse || (reinterpret_cast<uintptr_t>(lse) & 3u))
            return fail(MMDIT_ERR_INVALID_ARG, "%s: lse must be a 4-byte aligned pointer", who);
    }
    // outputs against each other and against every input
    const void* outs[3] = {dq, dk, dv};
    const size_t osz[3] = {qb * 4, kb * 4, kb * 4};
    const void* ins[6] = {q, k, v, o, lse, d_o};
    const size_t isz[6] = {qb * es, kb * es, kb * es, qb * 4, (size_t)n_q * heads * 4, qb * es};
    for (int i = 0; i < 3; ++i) {
        if (!outs[i] || osz[i] == 0) continue;
        for (int j = i + 1; j < 3; ++j)
            if (outs[j] && overlaps(outs[i], osz[i], outs[j], osz[j]))
                return fail(MMDIT_ERR_INVALID_ARG, "%s: dq, dk and dv must not overlap", who);
        for (int j = 0; j < 6; ++j)
            if (ins[j] && isz[j] && overlaps(outs[i], osz[i], ins[j], isz[j]))
                return fail(MMDIT_ERR_INVALID_ARG, "%s: a gradient aliases an input", who);
    }
    const BwdPlan p = plan_bwd(n_q, n_kv, heads, head_dim, dtype);
    if ((st = check_ws(ws, ws_bytes, p.total, who)) != MMDIT_OK) return st;
    softmax_scale = resolve_scale(softmax_scale, head_dim);
    char* w = (char*)ws;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e;
    float* dd = (float*)(w + p.off_dd);
    if (dtype == MMDIT_FP32) {
        if ((e = launch_bwd_rowterm(o, d_o, dtype, lse, n_q, n_q, heads, head_dim, dd, nullptr, s)) != hipSuccess)
            return hip_fail(e, who);
        e = launch_bwd_fp32((const float*)q, (const float*)k, (const float*)v, (const float*)d_o, lse, dd, n_q,
                            n_kv, heads, head_dim, softmax_scale, dq, dk, dv, s);
        return e == hipSuccess ? MMDIT_OK : hip_fail(e, who);
    }
    BwdArgs a{};
    a.q = (const __bf16*)q;
    a.k = (const __bf16*)k;
    a.v = (const __bf16*)v;
    a.d_o = (const __bf16*)d_o;
    a.qt = (const __bf16*)(w + p.off_qt);
    a.dot = (const __bf16*)(w + p.off_dot);
    a.kt = (const __bf16*)(w + p.off_kt);
    a.ls2 = (const float*)(w + p.off_ls2);
    a.dd = dd;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.n_q = n_q;
    a.n_kv = n_kv;
    a.n_q_pad = p.n_q_pad;
    a.n_kv_pad = p.n_kv_pad;
    a.heads = heads;
    a.scale = softmax_scale;
    a.scale_log2 = (float)((double)softmax_scale * 1.4426950408889634);
    if ((e = launch_bwd_rowterm(o, d_o, dtype, lse, n_q, p.n_q_pad, heads, head_dim, dd, (float*)a.ls2, s)) !=
            hipSuccess ||
        (e = launch_transpose(a.q, n_q, p.n_q_pad, heads, head_dim, (__bf16*)a.qt, s)) != hipSuccess ||
        (e = launch_transpose(a.d_o, n_q, p.n_q_pad, heads, head_dim, (__bf16*)a.dot, s)) != hipSuccess ||
        (e = launch_transpose(a.k, n_kv, p.n_kv_pad, heads, head_dim, (__bf16*)a.kt, s)) != hipSuccess ||
        (e = launch_bwd_keys(a, head_dim, s)) != hipSuccess || (e = launch_bwd_dq(a, head_dim, s)) != hipSuccess)
        return hip_fail(e, who);
    return MMDIT_OK;
}

mmdit_status mmdit_av_cross_attn(const void* q_v, const void* k_v, const void* v_v,
                                 int64_t n_video, const void* q_a, const void* k_a,
                                 const void* v_a, int64_t n_audio, int32_t heads,
                                 int32_t head_dim, int32_t dtype, float softmax_scale,
                                 float* o_video, float* o_audio, void* ws, size_t ws_bytes,
                                 void* stream) {
    if (n_video < 1 || n_audio < 1)
        return fail(MMDIT_ERR_INVALID_ARG, "av_cross_attn: n_video and n_audio must be >= 1");
    mmdit_status st = check_attn_args(q_v, n_video, k_a, v_a, n_audio, heads, head_dim, dtype,
                                      softmax_scale, o_video, "av_cross_attn (video->audio)");
    if (st != MMDIT_OK) return st;
    st = check_attn_args(q_a, n_audio, k_v, v_v, n_video, heads, head_dim, dtype, softmax_scale,
                         o_audio, "av_cross_attn (audio->video)");
    if (st != MMDIT_OK) return st;
    const size_t ob_v = (size_t)n_video * heads * head_dim * 4;
    const size_t ob_a = (size_t)n_audio * heads * head_dim * 4;
    const size_t es = elem_size(dtype);
    if (overlaps(o_video, ob_v, o_audio, ob_a) ||
        overlaps(o_video, ob_v, q_a, (size_t)n_audio * heads * head_dim * es) ||
        overlaps(o_video, ob_v, k_v, (size_t)n_video * heads * head_dim * es) ||
        overlaps(o_video, ob_v, v_v, (size_t)n_video * heads * head_dim * es) ||
        overlaps(o_audio, ob_a, q_v, (size_t)n_video * heads * head_dim * es) ||
        overlaps(o_audio, ob_a, k_a, (size_t)n_audio * heads * head_dim * es) ||
        overlaps(o_audio, ob_a, v_a, (size_t)n_audio * heads * head_dim * es))
        return fail(MMDIT_ERR_INVALID_ARG, "av_cross_attn: an output aliases an input or the other output");
    const AttnPlan pva = plan_attn(n_video, n_audio, heads, head_dim, dtype);
    const AttnPlan pav = plan_attn(n_audio, n_video, heads, head_dim, dtype);
    if ((st = check_ws(ws, ws_bytes, pva.total() + pav.total(), "av_cross_attn")) != MMDIT_OK)
        return st;
    softmax_scale = resolve_scale(softmax_scale, head_dim);
    char* w = (char*)ws;
    st = run_attn(q_v, n_video, k_a, v_a, n_audio, heads, head_dim, dtype, softmax_scale, o_video,
                  nullptr, w, pva, (hipStream_t)stream, "av_cross_attn (video->audio)");
    if (st != MMDIT_OK) return st;
    return run_attn(q_a, n_audio, k_v, v_v, n_video, heads, head_dim, dtype, softmax_scale,
                    o_audio, nullptr, w ? w + pva.total() : nullptr, pav, (hipStream_t)stream,
                    "av_cross_attn (audio->video)");
}

mmdit_status mmdit_block_sparse_attn(const void* q, const void* k, const void* v, int32_t T,
                                     int32_t H, int32_t W, int32_t heads, int32_t head_dim,
                                     const mmdit_sparse_desc* sp, double softmax_scale, float* o,
                                     uint32_t* sel_mask, int32_t* sel_count, void* ws,
                                     size_t ws_bytes, void* stream) {
    return run_sparse(q, k, v, T, H, W, heads, head_dim, sp, softmax_scale, o, nullptr, sel_mask, sel_count, ws,
                      ws_bytes, stream, "block_sparse");
}

mmdit_status mmdit_block_sparse_attn_fwd(const void* q, const void* k, const void* v, int32_t T, int32_t H,
                                         int32_t W, int32_t heads, int32_t head_dim, const mmdit_sparse_desc* sp,
                                         double softmax_scale, float* o, float* lse, uint32_t* sel_mask,
                                         int32_t* sel_count, void* ws, size_t ws_bytes, void* stream) {
    if (!lse || (reinterpret_cast<uintptr_t>(lse) & 3u))
        return fail(MMDIT_ERR_INVALID_ARG, "block_sparse_fwd: lse must be a 4-byte aligned pointer");
    if (!sel_mask)
        return fail(MMDIT_ERR_INVALID_ARG, "block_sparse_fwd: sel_mask is required (the backward takes it)");
    return run_sparse(q, k, v, T, H, W, heads, head_dim, sp, softmax_scale, o, lse, sel_mask, sel_count, ws,
                      ws_bytes, stream, "block_sparse_fwd");
}

mmdit_status mmdit_adaptive_tile_table(int32_t T, int32_t H, int32_t W, const uint8_t* zone_shape,
                                       int32_t* tile_base, uint8_t* tile_dims, int32_t* tile_block) {
    if (T < 1 || H < 1 || W < 1 || T % kZoneEdge || H % kZoneEdge || W % kZoneEdge)
        return fail(MMDIT_ERR_INVALID_ARG, "adaptive_tile_table: T, H, W must be positive multiples of %d",
                    kZoneEdge);
    const int64_t n = (int64_t)T * H * W;
    if (n >= ((int64_t)1 << 31)) return fail(MMDIT_ERR_UNSUPPORTED, "adaptive_tile_table: grid too large");
    if (!zone_shape) return fail(MMDIT_ERR_INVALID_ARG, "adaptive_tile_table: null zone_shape");
    const int64_t nz = n / (kZoneTiles * kTileN);
    for (int64_t m = 0; m < nz; ++m)
        if (zone_shape[m] > 15)
            return fail(MMDIT_ERR_INVALID_ARG, "adaptive_tile_table: zone %lld has shape code %d (0..15)",
                        (long long)m, (int)zone_shape[m]);
    SparseGeom g{};
    g.T = T, g.H = H, g.W = W;
    g.nzh = H / kZoneEdge, g.nzw = W / kZoneEdge;
    int32_t blocks = 0;
    for (int64_t m = 0; m < nz; ++m) {
        for (int u = 0; u < kZoneTiles; ++u) {
            const int s = (int)(m * kZoneTiles + u);
            const TileGeom tg = tile_geom(g, s, zone_shape[m]);
            if (tile_base) tile_base[s] = (int32_t)tg.base;
            if (tile_dims) tile_dims[s] = (uint8_t)tg.dims;
            if (tile_block) tile_block[s] = blocks + tg.blk;
        }
        int lt, lh, lw;
        adaptive_candidate(zone_shape[m], lt, lh, lw);
        blocks += 1 << (9 - (lt + lh + lw));
    }
    return MMDIT_OK;
}

mmdit_status mmdit_token_norms(const float* x, int64_t n, int64_t width, float* out, void* stream) {
    if (n < 0 || width < 4 || width % 4)
        return fail(MMDIT_ERR_INVALID_ARG, "token_norms: n >= 0 and width a positive multiple of 4 required");
    if (n >= ((int64_t)1 << 31)) return fail(MMDIT_ERR_UNSUPPORTED, "token_norms: n must stay below 2^31");
    if (n == 0) return MMDIT_OK;
    if (!x || !out || !aligned16(x) || (reinterpret_cast<uintptr_t>(out) & 3u))
        return fail(MMDIT_ERR_INVALID_ARG, "token_norms: x must be 16-byte and out 4-byte aligned, non-null");
    if (overlaps(out, (size_t)n * 4, x, (size_t)n * width * 4))
        return fail(MMDIT_ERR_INVALID_ARG, "token_norms: out aliases x");
    const hipError_t e = launch_token_norms(x, n, width, out, (hipStream_t)stream);
    return e == hipSuccess ? MMDIT_OK : hip_fail(e, "token_norms");
}

mmdit_status mmdit_block_sparse_attn_adaptive(const void* q, const void* k, const void* v, const float* a_norm,
                                              int32_t T, int32_t H, int32_t W, int32_t heads, int32_t head_dim,
                                              int32_t top_k, double top_p, double softmax_scale, float* o,
                                              float* lse, uint8_t* zone_shape, int32_t* tile_block,
                                              int32_t* n_blocks, uint32_t* sel_mask, int32_t* sel_count, void* ws,
                                              size_t ws_bytes, void* stream) {
    const char* who = "block_sparse_adaptive";
    if (T % kZoneEdge || H % kZoneEdge || W % kZoneEdge || T < 1 || H < 1 || W < 1)
        return fail(MMDIT_ERR_INVALID_ARG, "%s: T, H, W must be positive multiples of %d", who, kZoneEdge);
    if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u))
        return fail(MMDIT_ERR_INVALID_ARG, "%s: lse must be 4-byte aligned", who);
    mmdit_sparse_desc sp{};
    for (int i = 0; i < 3; ++i) sp.zone[i] = kZoneEdge, sp.block[i] = 4;
    sp.top_k = top_k;
    sp.top_p = top_p;
    const AdaptiveCall ad{a_norm, zone_shape, tile_block, n_blocks};
    return run_sparse(q, k, v, T, H, W, heads, head_dim, &sp, softmax_scale, o, lse, sel_mask, sel_count, ws,
                      ws_bytes, stream, who, &ad);
}

mmdit_status mmdit_block_sparse_attn_bwd(const void* q, const void* k, const void* v, int32_t T, int32_t H,
                                         int32_t W, int32_t heads, int32_t head_dim, const mmdit_sparse_desc* sp,
                                         double softmax_scale, const float* o, const float* lse, const void* d_o,
                                         const uint32_t* sel_mask, float* dq, float* dk, float* dv, void* ws,
                                         size_t ws_bytes, void* stream) {
    const char* who = "block_sparse_bwd";
    SparsePlan p{};
    mmdit_status st = plan_sparse(T, H, W, heads, head_dim, sp, &p);
    if (st != MMDIT_OK) return st;
    if (!scale_ok(softmax_scale))
        return fail(MMDIT_ERR_INVALID_ARG, "%s: softmax_scale must be finite and >= 0 (0: 1/sqrt(head_dim))",
                    who);
    softmax_scale = resolve_scale(softmax_scale, head_dim);
    const void* al16[8] = {q, k, v, o, d_o, dq, dk, dv};
    for (const void* ptr : al16)
        if (!ptr || !aligned16(ptr))
            return fail(MMDIT_ERR_INVALID_ARG, "%s: q, k, v, o, d_o, dq, dk, dv must be non-null and 16-byte aligned",
                        who);
    if (!lse || (reinterpret_cast<uintptr_t>(lse) & 3u) || !sel_mask ||
        (reinterpret_cast<uintptr_t>(sel_mask) & 3u))
        return fail(MMDIT_ERR_INVALID_ARG, "%s: lse and sel_mask must be non-null and 4-byte aligned", who);
    const int64_t n = (int64_t)T * H * W;
    const int64_t nb = p.g.nb, nw = (nb + 31) / 32;
    const size_t ib = (size_t)n * heads * head_dim * 2, fb = (size_t)n * heads * head_dim * 4;
    const void* outs[3] = {dq, dk, dv};
    const void* ins[6] = {q, k, v, o, lse, d_o};
    const size_t isz[6] = {ib, ib, ib, fb, (size_t)n * heads * 4, ib};
    for (int i = 0; i < 3; ++i) {
        for (int j = i + 1; j < 3; ++j)
            if (overlaps(outs[i], fb, outs[j], fb))
                return fail(MMDIT_ERR_INVALID_ARG, "%s: dq, dk and dv must not overlap", who);
        for (int j = 0; j < 6; ++j)
            if (overlaps(outs[i], fb, ins[j], isz[j]))
                return fail(MMDIT_ERR_INVALID_ARG, "%s: a gradient aliases an input", who);
        if (overlaps(outs[i], fb, sel_mask, (size_t)heads * nb * nw * 4))
            return fail(MMDIT_ERR_INVALID_ARG, "%s: a gradient aliases sel_mask", who);
    }
    const SparseBwdPlan bp = plan_sparse_bwd(n, nb, heads, head_dim);
    if ((st = check_ws(ws, ws_bytes, bp.total, who)) != MMDIT_OK) return st;
    return run_sparse_bwd(p.g, bp, q, k, v, o, lse, d_o, sel_mask, dq, dk, dv, softmax_scale, nullptr, nullptr,
                          (char*)ws, (hipStream_t)stream, who);
}

mmdit_status mmdit_block_sparse_attn_adaptive_bwd(const void* q, const void* k, const void* v, int32_t T, int32_t H,
                                                  int32_t W, int32_t heads, int32_t head_dim, double softmax_scale,
                                                  const float* o, const float* lse, const void* d_o,
                                                  const uint8_t* zone_shape, const uint32_t* sel_mask, float* dq,
                                                  float* dk, float* dv, void* ws, size_t ws_bytes, void* stream) {
    const char* who = "block_sparse_adaptive_bwd";
    if (T < 1 || H < 1 || W < 1 || T % kZoneEdge || H % kZoneEdge || W % kZoneEdge)
        return fail(MMDIT_ERR_INVALID_ARG, "%s: T, H, W must be positive multiples of %d", who, kZoneEdge);
    const int64_t n = (int64_t)T * H * W;
    if (n / kTileN / kZoneTiles > kMaxZones)
        return fail(MMDIT_ERR_UNSUPPORTED, "%s: %lld zones (max %d)", who, (long long)(n / 512), kMaxZones);
    // the grid in tile order: one row of tokens, a block per 64 of them
    mmdit_sparse_desc flat{};
    flat.zone[0] = flat.zone[1] = flat.block[0] = flat.block[1] = 1;
    flat.zone[2] = flat.block[2] = kTileN;
    flat.top_k = 0;
    flat.top_p = 1.0;
    SparsePlan p{};
    mmdit_status st = plan_sparse(1, 1, (int)std::min<int64_t>(n, INT32_MAX), heads, head_dim, &flat, &p);
    if (st != MMDIT_OK) return st;
    if (!scale_ok(softmax_scale))
        return fail(MMDIT_ERR_INVALID_ARG, "%s: softmax_scale must be finite and >= 0 (0: 1/sqrt(head_dim))",
                    who);
    softmax_scale = resolve_scale(softmax_scale, head_dim);
    const void* al16[8] = {q, k, v, o, d_o, dq, dk, dv};
    for (const void* ptr : al16)
        if (!ptr || !aligned16(ptr))
            return fail(MMDIT_ERR_INVALID_ARG, "%s: q, k, v, o, d_o, dq, dk, dv must be non-null and 16-byte aligned",
                        who);
    if (!lse || (reinterpret_cast<uintptr_t>(lse) & 3u) || !sel_mask ||
        (reinterpret_cast<uintptr_t>(sel_mask) & 3u) || !zone_shape)
        return fail(MMDIT_ERR_INVALID_ARG, "%s: lse, sel_mask (4-byte aligned) and zone_shape are required", who);
    const int64_t nb = p.g.nb, nw = (nb + 31) / 32;
    const size_t ib = (size_t)n * heads * head_dim * 2, fb = (size_t)n * heads * head_dim * 4;
    const void* outs[3] = {dq, dk, dv};
    const void* ins[8] = {q, k, v, o, lse, d_o, sel_mask, zone_shape};
    const size_t isz[8] = {ib, ib, ib, fb, (size_t)n * heads * 4, ib, (size_t)heads * nb * nw * 4,
                           (size_t)(n / 512)};
    for (int i = 0; i < 3; ++i) {
        for (int j = i + 1; j < 3; ++j)
            if (overlaps(outs[i], fb, outs[j], fb))
                return fail(MMDIT_ERR_INVALID_ARG, "%s: dq, dk and dv must not overlap", who);
        for (int j = 0; j < 8; ++j)
            if (overlaps(outs[i], fb, ins[j], isz[j]))
                return fail(MMDIT_ERR_INVALID_ARG, "%s: a gradient aliases an input", who);
    }
    const AdaptiveBwdPlan ap = plan_adaptive_bwd(n, heads, head_dim);
    if ((st = check_ws(ws, ws_bytes, ap.total, who)) != MMDIT_OK) return st;
    char* w = (char*)ws;
    hipStream_t s = (hipStream_t)stream;
    // the grid and the tiles of the shapes the forward chose; the backward
    // reads and writes the raster tensors in place
    SparseGeom grid{};
    grid.T = T, grid.H = H, grid.W = W;
    grid.nzh = H / kZoneEdge, grid.nzw = W / kZoneEdge;
    grid.nb = (int32_t)nb;
    grid.heads = heads;
    int32_t* tbase = (int32_t*)(w + ap.off_tbase);
    uint8_t* tdim = (uint8_t*)(w + ap.off_tdim);
    hipError_t e;
    if ((e = launch_tile_table(grid, zone_shape, tbase, tdim, s)) != hipSuccess) return hip_fail(e, who);
    st = run_sparse_bwd(grid, ap.bwd, q, k, v, o, lse, d_o, sel_mask, dq, dk, dv, softmax_scale, tbase, tdim,
                        w + ap.off_bwd, s, who);
    if (st != MMDIT_OK) return st;
    return MMDIT_OK;
}

}  // extern "C"
