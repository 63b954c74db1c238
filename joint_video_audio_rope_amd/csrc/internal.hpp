// Internal declarations shared by the library's translation units (not part
// of the ABI).  Everything here is gfx950 HIP.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mmdit.h"

namespace mmdit {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4v __attribute__((ext_vector_type(4)));

constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLog2e = 1.4426950408889634f;

// Threads per 64-lane wavefront on CDNA.
constexpr int kWave = 64;
// Keys per K/V tile of the attention kernels.
constexpr int kTileN = 64;
// Dense bf16 attention workgroup: 256 queries, each wave holding kDenseQB
// blocks of 32 queries (so 8 / kDenseQB waves).  Two blocks per wave halve
// the LDS fragment reads per MFMA but need ~420 registers, i.e. one wave per
// SIMD with Q and O in AGPRs.  With the compiler placing the accumulators it
// measured 1.5x slower than one block per wave with two waves per SIMD; with
// Q and O pinned to AGPRs (matrix-core products in inline assembly) still
// 1.1x slower: at the 256-VGPR limit the scheduler issues each fragment read
// just before its product, and a lone wave per SIMD waits out every LDS
// latency that the second wave hides here.
constexpr int kDenseQ = 256;
constexpr int kDenseQB = 1;
constexpr int dense_threads(int qb) { return kDenseQ / (32 * qb) * kWave; }
// Calls with at most kShortKv keys (video -> text, video -> audio) use
// workgroups of kShortQ queries (4 waves), two per CU at the same two waves
// per SIMD: with only a few key tiles per workgroup, one workgroup's Q loads
// and O stores then overlap the other's products.  So do calls with at most
// kDenseQ queries (audio -> video), whose keys are split across workgroups.
constexpr int kShortQ = 128;
constexpr int kShortKv = 1024;

// ---- RoPE ------------------------------------------------------------------
struct RopeSeg {
    int32_t kind;
    int32_t T, H, W;
    int64_t offset;        // first token
    int64_t chunk_begin;   // first 16-byte chunk id of this segment (global numbering)
    int64_t chunk_end;
    int32_t tab_t, tab_h, tab_w;   // float2 index of each axis sub-table in the table
};

struct RopeArgs {
    RopeSeg seg[MMDIT_MAX_SEGMENTS];
    int32_t n_segs;
    int32_t heads, head_dim, d_t, d_h, d_w;
    int32_t chunks_per_token;      // heads * head_dim / elems per chunk
    int64_t total_chunks;
};

hipError_t launch_rope(const RopeArgs& a, const float* table, void* q, void* k, int dtype,
                       hipStream_t s);

// Rotation of one adjacent pair (x0, x1) by the angle whose (cos, sin) is
// (c, s), with the roundings spelled out (one product, then one fused
// multiply-add per output) so that every kernel that rotates produces the
// same bits.
__device__ __forceinline__ void rope_pair(float x0, float x1, float c, float s, float& y0, float& y1) {
    y0 = __builtin_fmaf(x0, c, -(x1 * s));
    y1 = __builtin_fmaf(x0, s, x1 * c);
}

// float2 index into the (cos, sin) table of the first pair of the 8-element
// chunk that starts at element `dim` (a multiple of 8) of token `tok` (an
// index into the [n_tokens][heads][head_dim] buffer), or -1 when that chunk
// is not rotated (text and other tokens outside every segment, and the h and
// w slices of audio tokens, which sit at position 0).
__device__ __forceinline__ int rope_table_index(const RopeArgs& a, int64_t tok, int dim) {
    for (int i = 0; i < a.n_segs; ++i) {
        const RopeSeg& sg = a.seg[i];
        const int64_t count = (sg.chunk_end - sg.chunk_begin) / a.chunks_per_token;
        if (tok < sg.offset || tok >= sg.offset + count) continue;
        const int t = (int)(tok - sg.offset);
        if (dim < a.d_t) {
            const int p = sg.kind == MMDIT_SEG_VIDEO ? t / (sg.H * sg.W) : t;
            return sg.tab_t + p * (a.d_t >> 1) + (dim >> 1);
        }
        if (sg.kind != MMDIT_SEG_VIDEO) return -1;
        if (dim < a.d_t + a.d_h) return sg.tab_h + ((t / sg.W) % sg.H) * (a.d_h >> 1) + ((dim - a.d_t) >> 1);
        return sg.tab_w + (t % sg.W) * (a.d_w >> 1) + ((dim - a.d_t - a.d_h) >> 1);
    }
    return -1;
}

// Rotate 8 bf16 values (elements dim .. dim + 7 of one token row) in fp32
// with table pairs tab[ti .. ti + 3]; results rounded to bf16 (nearest even).
__device__ __forceinline__ bf16x8 rope_chunk_bf16(bf16x8 x, const float2* __restrict__ tab, int ti) {
    if (ti < 0) return x;
    bf16x8 y;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float2 cs = tab[ti + i];
        float y0, y1;
        rope_pair((float)x[2 * i], (float)x[2 * i + 1], cs.x, cs.y, y0, y1);
        y[2 * i] = (__bf16)y0;
        y[2 * i + 1] = (__bf16)y1;
    }
    return y;
}

// ---- fp16 staging of V -----------------------------------------------------------
// V enters the P V products as fp16 (three more mantissa bits than bf16, for
// P).  A bf16 value converts to fp16 exactly only inside fp16's normal range,
// so each head's V is first scaled by a power of two 2^e chosen from the
// head's largest magnitude: the largest entry lands in [2^14, 2^15), nothing
// overflows whatever the range of V, every entry within 2^-28 of the largest
// converts exactly, and O is scaled back by 2^-e (also exact).  For values
// that are already inside fp16's range the results are bitwise those of an
// unscaled conversion.
constexpr int kVmaxParts = 64;   // partial maxima per head, reduced by one wave

// vmax [heads][kVmaxParts]: the largest bf16 magnitude (bits & 0x7FFF) of
// each head over kVmaxParts slices of the n tokens of v [n][heads][hd].
hipError_t launch_v_absmax(const __bf16* v, int64_t n, int heads, int hd, uint32_t* vmax, hipStream_t s);

// Exponent e of the prescale for the largest bf16 magnitude m (bits): 0 for
// an all-zero head or one holding inf / NaN (they propagate as in the
// definition), else 14 - floor(log2(max)), at most 100 (V below 2^-86 is left
// partly subnormal in fp16).
__host__ __device__ __forceinline__ int v_exp_from_max(uint32_t m) {
    if (m == 0u || m >= 0x7F80u) return 0;
    const int e = 14 - ((int)(m >> 7) - 127);
    return e < 100 ? e : 100;
}

// The head's exponent from its partial maxima, computed by a whole wave
// (every lane loads one partial); wave-uniform.
__device__ __forceinline__ int v_scale_exp(const uint32_t* vmax, int head) {
    uint32_t m = vmax[(int64_t)head * kVmaxParts + (threadIdx.x & 63)];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const uint32_t x = (uint32_t)__shfl_xor((int)m, o);
        m = m > x ? m : x;
    }
    return v_exp_from_max(__builtin_amdgcn_readfirstlane(m));
}

// ---- dense attention ---------------------------------------------------------
// V of one key range transposed to fp16 [heads][head_dim][n_pad] (pad keys
// zero), each head scaled by its prescale 2^e (from vmax).
hipError_t launch_vt_dense(const __bf16* v, int64_t n_kv, int64_t n_pad, int heads, int hd,
                           const uint32_t* vmax, _Float16* vt, hipStream_t s);

struct AttnArgs {
    const __bf16* q;
    const __bf16* k;
    const _Float16* vt;    // [heads][hd][n_pad], head h scaled by 2^e(h)
    const uint32_t* vmax;  // [heads][kVmaxParts] partial maxima of V (the prescale exponents)
    float* o;              // [n_q][heads][hd], used when splits == 1
    float* part_o;         // [splits][heads][n_q_pad][hd], splits > 1
    float* part_ml;        // [splits][heads][n_q_pad][2]
    float* lse;            // [heads][n_q] natural-log log-sum-exp, or null
    int64_t n_q, n_kv, n_pad, n_q_pad;
    int32_t heads;
    int32_t q_tiles;       // ceil(n_q / q_tile)
    int32_t splits;
    int32_t tiles_per_split;
    int32_t kv_tiles;
    float scale_log2;      // softmax scale * log2(e)
    int32_t q_tile;        // queries per workgroup: kDenseQ or kShortQ
};

hipError_t launch_attn_bf16(const AttnArgs& a, int hd, hipStream_t s);
hipError_t launch_attn_combine(const AttnArgs& a, int hd, hipStream_t s);

// RoPE fused into the joint attention: the staging pass also rotates K (all
// n_kv tokens, those outside every rotated segment copied) into k_out, and
// the attention kernel rotates each Q row in registers as it loads it,
// optionally storing the rotated row to q_out.  Token indices are those of
// the [n][heads][hd] buffers the RoPE descriptor describes.
struct RopeFused {
    RopeArgs a;
    const float2* tab;     // device (cos, sin) table of the descriptor
    const __bf16* k;       // K before rotation
    __bf16* k_out;         // rotated K (the attention reads it)
    __bf16* q_out;         // rotated Q, or null
};
hipError_t launch_vt_dense_rope(const __bf16* v, int64_t n_kv, int64_t n_pad, int heads, int hd,
                                const uint32_t* vmax, _Float16* vt, const RopeFused& r, hipStream_t s);
hipError_t launch_attn_bf16_rope(const AttnArgs& a, int hd, const RopeFused& r, hipStream_t s);

hipError_t launch_attn_fp32(const float* q, int64_t n_q, const float* k, const float* v,
                            int64_t n_kv, int heads, int hd, float scale, float* o, float* lse,
                            hipStream_t s);

// ---- dense attention backward --------------------------------------------------
// dK and dV workgroups: kBwdKvWaves waves of 32 keys, two waves per SIMD.
constexpr int kBwdKvWaves = 8;
constexpr int kBwdKvKeys = 32 * kBwdKvWaves;
// dQ workgroup: kBwdDqWaves waves of 32 queries, two waves per SIMD.
constexpr int kBwdDqWaves = 8;
constexpr int kBwdDqQueries = 32 * kBwdDqWaves;

struct BwdArgs {
    const __bf16* q;       // [n_q][heads][hd]
    const __bf16* k;       // [n_kv][heads][hd]
    const __bf16* v;
    const __bf16* d_o;     // [n_q][heads][hd]
    const __bf16* qt;      // [heads][hd][n_q_pad]
    const __bf16* dot;     // [heads][hd][n_q_pad]
    const __bf16* kt;      // [heads][hd][n_kv_pad]
    const float* ls2;      // [heads][n_q_pad] lse * log2(e), +inf past n_q
    const float* dd;       // [heads][n_q_pad] <dO_i, O_i>, 0 past n_q
    float* dq;             // [n_q][heads][hd]
    float* dk;             // [n_kv][heads][hd]
    float* dv;
    int64_t n_q, n_kv, n_q_pad, n_kv_pad;   // pads: multiples of 64
    int32_t heads;
    float scale;           // softmax scale
    float scale_log2;      // softmax scale * log2(e)
    int32_t q_tile;        // queries per workgroup: kDenseQ or kShortQ
};

// D = <dO, O> (and, when ls2 is not null, lse * log2(e)) per (head, query),
// written [heads][n_q_pad] with D = 0 and +inf past n_q.
hipError_t launch_bwd_rowterm(const float* o, const void* d_o, int dtype, const float* lse, int64_t n_q,
                              int64_t n_q_pad, int heads, int hd, float* dd, float* ls2, hipStream_t s);
// [n][heads][hd] bf16 -> [heads][hd][n_pad] bf16, zero past n.
hipError_t launch_transpose(const __bf16* src, int64_t n, int64_t n_pad, int heads, int hd, __bf16* dst,
                            hipStream_t s);
// The two key-owned passes: dV, then dK.
hipError_t launch_bwd_keys(const BwdArgs& a, int hd, hipStream_t s);
hipError_t launch_bwd_dq(const BwdArgs& a, int hd, hipStream_t s);
hipError_t launch_bwd_fp32(const float* q, const float* k, const float* v, const float* d_o, const float* lse,
                           const float* dd, int64_t n_q, int64_t n_kv, int heads, int hd, float scale, float* dq,
                           float* dk, float* dv, hipStream_t s);

// ---- block sparse -------------------------------------------------------------
struct SparseGeom {
    int32_t T, H, W;
    int32_t ZT, ZH, ZW;        // zone
    int32_t BT, BH, BW;        // block
    int32_t nzh, nzw;          // zones along h and w
    int32_t bz_t, bz_h, bz_w;  // blocks per zone along each axis
    int32_t nb;                // blocks in the grid
    int32_t heads;
};

// Query blocks per workgroup of the block-sparse attention kernel.  Measured
// on the 24 x 64 x 112 grid (density 27.6 %), where a block selects 742 key
// blocks on average: a group of G consecutive blocks stages the union of
// their selections, 1488 tiles for G = 4 and 1951 for G = 7, so the gathered
// K/V tiles per call fall from 786 GB to 589 GB and the copies alone from
// 95 ms to 69 ms.  The consumers' compute bounds the kernel, and more waves
// per SIMD keep more of them busy: the call went from 133.3 ms (G = 4,
// whole-tile steps at 168 registers) to 129.4 ms (G = 7, half-tile steps at
// 128).  With workgroup barriers per tile instead of producer waves, pairs
// took 164 ms and groups of 4 205 ms.
constexpr int kStreamGroup = 7;
__host__ __device__ constexpr int64_t stream_groups(int64_t nb) { return (nb + kStreamGroup - 1) / kStreamGroup; }

struct SparseWs {
    double* qbar;       // [heads][nb][hd]
    double* kbar;       // [heads][nb][hd]
    double* scores;     // [heads][chunk rows][nb] (logits, scaled) of the chunk of query blocks being selected
    uint32_t* mask;     // [heads][nb][ceil(nb/32)] selected key blocks, bit j of word j/32
    int32_t* count;     // [heads][nb]
    int32_t* base;      // [nb] raster token index of each block's first token
    _Float16* vt;       // [heads][nb][hd * 64]: each key block's V^T (prescaled) in LDS tile order
    __bf16* kimg;       // [heads][nb][64 * hd]: each key block's K rows in LDS tile order
    uint32_t* vmax;     // [heads][kVmaxParts] partial maxima of V (the prescale exponents)
    int32_t* order;     // [heads][stream_groups(nb)] group ids in the attention kernel's dispatch order
    // Content-adaptive blocks (null for uniform blocks).  "Blocks" above are
    // then 64-token tiles; a block of 128 or 256 tokens is 2 or 4 consecutive
    // tiles, and base[] is filled by the shape pass.
    const uint8_t* tdim;  // [nb] log2 edges of each tile: t | h << 2 | w << 4
    const int32_t* lead;  // [nb] first tile of the tile's block
};

hipError_t launch_block_pool(const SparseGeom& g, const __bf16* q, const __bf16* k, int hd,
                             const SparseWs& w, hipStream_t s);
hipError_t launch_vt_blocks(const SparseGeom& g, const __bf16* k, const __bf16* v, int hd, const SparseWs& w,
                            hipStream_t s);
// The block logits and the selection run in chunks of query blocks: the
// scores of query blocks row0 .. row0 + rows - 1 (all heads) are computed
// into w.scores ([heads][rows][nb]) and selected from there.
hipError_t launch_block_scores(const SparseGeom& g, int hd, double scale, const SparseWs& w, int row0, int rows,
                               hipStream_t s);
hipError_t launch_block_select(const SparseGeom& g, int top_k, double top_p, const SparseWs& w, int row0, int rows,
                               uint32_t* sel_mask, int32_t* sel_count, hipStream_t s);
// Blocks per workgroup of the block-sparse backward passes (a 2 x 2 square).
constexpr int kBwdGroup = 4;

// Per head, the groups of `group` consecutive blocks (kStreamGroup or
// kBwdGroup) ranked by an estimate of their walk's time from the bitmask rows
// [heads][nb][ceil(nb/32)], costliest first, into order [heads][groups].
hipError_t launch_group_order(const SparseGeom& g, int group, const uint32_t* mask, int32_t* order, hipStream_t s);

// Workgroups of a walk kernel over `groups` groups per head: 8 per rank slot
// of every head (one per XCD), head-major.
__host__ __device__ constexpr int64_t group_workgroups(int64_t groups, int64_t heads) {
    return 8 * ((groups + 7) / 8) * heads;
}

// The (head, group) of this workgroup: head-major, so the tiles in flight
// stay those of one head; within a head, rank 8 j + x of the order table to
// XCD x (blockIdx % 8) for even j and to XCD 7 - x for odd j.  False for the
// padding workgroups past the last rank.
__device__ __forceinline__ bool group_of_workgroup(int groups, int heads, const int32_t* order, int& head,
                                                   int& grp) {
    const int per = (groups + 7) >> 3;
    const int xcd = (int)(blockIdx.x & 7);
    const int slot = (int)(blockIdx.x >> 3);
    head = slot / per;
    const int j = slot - head * per;
    const int rank = 8 * j + ((j & 1) ? 7 - xcd : xcd);
    if (head >= heads || rank >= groups) return false;
    grp = order[(int64_t)head * groups + rank];
    return true;
}
// wait_limit: bound of each of the kernel's internal waits, in sleeps of
// about 64 cycles (1 .. kSpinLimit).  A wait that reaches it gives up and the
// workgroup writes NaN to its o rows and lse entries.
// K and V come from the staged block images in w.
hipError_t launch_sparse_attn(const SparseGeom& g, const __bf16* q, int hd,
                              float scale_log2, const SparseWs& w, float* o, float* lse, int wait_limit,
                              hipStream_t s);
constexpr int kSpinLimit = 1 << 18;

// Largest number of blocks (64-token tiles) per head: selection rows of up to
// 4096 blocks are held by one wave, longer ones by 2, 4 or 8 waves; the
// attention kernels stage their blocks' selection rows in LDS.
constexpr int kSelMax = 32768;
// Bytes of block logits computed and selected at once (the chunk of query
// blocks is sized to stay within it).
constexpr size_t kScoreChunkBytes = size_t(1) << 30;

// ---- content-adaptive block shapes ----------------------------------------------
constexpr int kZoneEdge = 8;       // macro-zone edge in tokens along t, h and w
constexpr int kZoneTiles = 8;      // 64-token tiles per zone
constexpr int kStatPairs = 256;    // channel pairs per zone-statistics workgroup
constexpr int kMaxZones = kSelMax / kZoneTiles;

struct AdaptiveWs {
    double* part;      // [nz][nchunk][3] per-chunk sums over channels of the directional variances
    double* audio;     // [nz][4] zone mean of the audio norms, then their three directional variances
    uint8_t* code;     // [nz] candidate shape of each zone
    int32_t* base;     // [nt] first raster token of each tile (SparseWs::base)
    uint8_t* tdim;     // [nt] log2 edges of each tile
    int32_t* lead;     // [nt] first tile of the tile's block
    int32_t* tblock;   // [nt] block id of each tile
    int32_t* nblocks;  // [1] number of blocks
};

// log2 edges (t, h, w) of content-adaptive candidate `code`: volume 64 (codes
// 0-6), 128 (7-12), 256 (13-15), each group in lexicographic (b_T, b_H, b_W)
// order of the boxes with edges in {2, 4, 8}.
__host__ __device__ __forceinline__ void adaptive_candidate(int code, int& lt, int& lh, int& lw) {
    constexpr uint8_t kCand[16] = {0x39, 0x2D, 0x36, 0x2A, 0x1E, 0x27, 0x1B,   // t | h << 2 | w << 4
                                   0x3D, 0x3A, 0x2E, 0x37, 0x2B, 0x1F, 0x3E, 0x3B, 0x2F};
    const int c = kCand[code];
    lt = c & 3, lh = (c >> 2) & 3, lw = (c >> 4) & 3;
}

// Geometry of tile s (zone s / 8, tile s % 8 of the zone, zones in raster
// order over a grid of whole 8 x 8 x 8 zones) for zone shape `code`: the
// raster index of its first token, its log2 edges (t | h << 2 | w << 4), its
// index inside its block and its block's index inside the zone.  A block of
// B tokens is B / 64 tiles: its longest edge halved (the first of t, h, w
// among equals) once per factor of two, tiles in raster order inside the
// block, blocks in raster order of their position in the zone.
struct TileGeom {
    int64_t base;
    uint32_t dims;
    int sub, blk;
};

__host__ __device__ __forceinline__ TileGeom tile_geom(const SparseGeom& g, int s, int code) {
    const int zm = s / kZoneTiles, u = s - zm * kZoneTiles;
    int lbt, lbh, lbw;
    adaptive_candidate(code, lbt, lbh, lbw);
    const int split = lbt + lbh + lbw - 6;   // tiles per block = 2^split
    const int blk = u >> split, sub = u & ((1 << split) - 1);
    // position of the block inside the zone, raster over (8 >> lbt, 8 >> lbh, 8 >> lbw)
    const int nbh = 8 >> lbh, nbw = 8 >> lbw;
    const int pt = blk / (nbh * nbw), ph = (blk / nbw) % nbh, pw = blk % nbw;
    // tile edges: halve the longest edge (first of t, h, w) split times
    int lt = lbt, lh = lbh, lw = lbw;
    for (int i = 0; i < split; ++i) {
        if (lt >= lh && lt >= lw) --lt;
        else if (lh >= lw) --lh;
        else --lw;
    }
    const int qh_n = 1 << (lbh - lh), qw_n = 1 << (lbw - lw);
    const int qt = sub / (qh_n * qw_n), qh = (sub / qw_n) % qh_n, qw = sub % qw_n;
    const int t = (pt << lbt) + (qt << lt), h = (ph << lbh) + (qh << lh), w = (pw << lbw) + (qw << lw);
    const int zt = zm / (g.nzh * g.nzw);
    const int zr = zm - zt * (g.nzh * g.nzw);
    const int zh = zr / g.nzw;
    const int zw = zr - zh * g.nzw;
    TileGeom r;
    r.base = ((int64_t)(zt * kZoneEdge + t) * g.H + zh * kZoneEdge + h) * g.W + zw * kZoneEdge + w;
    r.dims = (uint32_t)(lt | (lh << 2) | (lw << 4));
    r.sub = sub;
    r.blk = blk;
    return r;
}

// Per zone channel statistics of V and the audio norms a (may be null), then
// the one-workgroup pass that turns them into volumes, shapes and tile tables.
hipError_t launch_zone_stats(const SparseGeom& g, const __bf16* v, const float* a, int hd, const AdaptiveWs& w,
                             hipStream_t s);
hipError_t launch_zone_shapes(const SparseGeom& g, int hd, const AdaptiveWs& w, hipStream_t s);
int zone_stat_chunks(int heads, int hd);
// Per tile of the tiling the zone shape codes of a forward call define: its
// first raster token and log2 edges.
hipError_t launch_tile_table(const SparseGeom& g, const uint8_t* codes, int32_t* tbase, uint8_t* tdim,
                             hipStream_t s);
// out[t] = ||x[t][0 .. width)||_2 for t < n; width a multiple of 4.
hipError_t launch_token_norms(const float* x, int64_t n, int64_t width, float* out, hipStream_t s);

// ---- block-sparse backward ------------------------------------------------------
struct SparseBwdArgs {
    const __bf16* q;         // [n][heads][hd] raster tokens
    const __bf16* k;
    const __bf16* v;
    const __bf16* d_o;
    const __bf16* qt_img;    // [heads][nb][hd * 64] transposed block images
    const __bf16* dot_img;
    const __bf16* kt_img;
    const __bf16* q_img;     // [heads][nb][64 * hd] block row images (row-major tile order)
    const __bf16* do_img;
    const __bf16* k_img;
    const __bf16* v_img;
    const uint32_t* mask;    // [heads][nb][ceil(nb/32)] query block -> selected key blocks
    const uint32_t* maskt;   // [heads][nb][ceil(nb/32)] key block -> query blocks that selected it
    const float* ls2;        // [heads][n] lse * log2(e)
    const float* dd;         // [heads][n] <dO_i, O_i>
    float* dq;               // [n][heads][hd]
    float* dk;
    float* dv;
    // Content-adaptive tiles (null for uniform blocks): "blocks" are then the
    // 64-token tiles, tile j's local token r is raster token tbase[j] +
    // tile_local(g, tdim[j], r), and g holds the grid (T, H, W, nb tiles).
    const int32_t* tbase;
    const uint8_t* tdim;
    const int32_t* order_q;  // [heads][groups] dispatch order of the dQ pass's groups of query blocks
    const int32_t* order_k;  // [heads][groups] dispatch order of the key passes' groups of key blocks
    float scale;
    float scale_log2;
};

hipError_t launch_block_timg(const SparseGeom& g, const __bf16* src, __bf16* dst, const int32_t* tbase,
                             const uint8_t* tdim, hipStream_t s);
hipError_t launch_block_rimg(const SparseGeom& g, const __bf16* src, __bf16* dst, const int32_t* tbase,
                             const uint8_t* tdim, hipStream_t s);
hipError_t launch_mask_transpose(const SparseGeom& g, const uint32_t* mask, uint32_t* maskt, hipStream_t s);
hipError_t launch_sparse_bwd(const SparseGeom& g, const SparseBwdArgs& a, hipStream_t s);

// Offset from a tile's first token of its local token r (raster inside the
// tile) for a tile with log2 edges code = lt | lh << 2 | lw << 4.
__host__ __device__ __forceinline__ int64_t tile_local(const SparseGeom& g, uint32_t code, int r) {
    const int lh = (code >> 2) & 3, lw = (code >> 4) & 3;
    const int a = r >> (lh + lw);
    const int b = (r >> lw) & ((1 << lh) - 1);
    const int c = r & ((1 << lw) - 1);
    return ((int64_t)a * g.H + b) * g.W + c;
}

// Token index (raster t, h, w) of local token r (0..63, raster inside the
// 4x4x4 block) of block j.
__device__ __forceinline__ int64_t block_token(const SparseGeom& g, int j, int r) {
    const int bpz = g.bz_t * g.bz_h * g.bz_w;
    const int zone = j / bpz;
    const int loc = j - zone * bpz;
    const int zt = zone / (g.nzh * g.nzw);
    const int zrem = zone - zt * (g.nzh * g.nzw);
    const int zh = zrem / g.nzw;
    const int zw = zrem - zh * g.nzw;
    const int bt = loc / (g.bz_h * g.bz_w);
    const int brem = loc - bt * (g.bz_h * g.bz_w);
    const int bh = brem / g.bz_w;
    const int bw = brem - bh * g.bz_w;
    const int a = r / (g.BH * g.BW);
    const int rr = r - a * (g.BH * g.BW);
    const int b = rr / g.BW;
    const int c = rr - b * g.BW;
    const int t = zt * g.ZT + bt * g.BT + a;
    const int h = zh * g.ZH + bh * g.BH + b;
    const int w = zw * g.ZW + bw * g.BW + c;
    return ((int64_t)t * g.H + h) * g.W + w;
}

}  // namespace mmdit
