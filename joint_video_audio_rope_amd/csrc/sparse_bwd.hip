// Backward pass of the block-sparse video self-attention (training).
//
// The Prism page ("Resultados", efficiency gains) measures the block-sparse
// attention by the time of a training step at 2K; its "Metodo" section 3
// defines the attention as softmax attention of each query block over the
// key blocks of S_i only.  The selection is a piecewise-constant function of
// Q and K, so the backward holds it fixed: the gradients are those of masked
// softmax attention, with P_ij = exp(s <q_i, k_j> - lse_i) on the selected
// pairs (lse_i from the sparse forward, over S_i) and 0 elsewhere.
//
// Passes (bf16 products, fp32 accumulation), mirroring the dense backward:
//   block_timg   per-block transposed images Q^T, dO^T, K^T [heads][nb][hd x 64]
//                in the LDS order of a transposed tile (the operands that
//                contract over tokens; a block's 64 tokens are not contiguous
//                in the raster layout, so these are staged once);
//   block_rimg   per-block row images Q, dO, K, V [heads][nb][64 x hd] in the
//                LDS order of a row-major tile;
//   mask_transpose  the selection bitmask transposed: for each key block, the
//                query blocks that selected it;
//   dq           a workgroup owns 4 query blocks (8 waves of 32 queries) and
//                walks the union of their selections: S^T = K Q^T, dP^T =
//                V dO^T, dQ^T += K^T dS^T for each selected key block;
//   key (dV, dK) a workgroup owns 4 key blocks (8 waves of 32 keys) and walks
//                the union of the query blocks that selected them: S = Q K^T
//                -> P -> dV^T += dO^T P, and S, dP = dO V^T -> dS -> dK^T +=
//                Q^T dS.
// Every tile is staged by contiguous 1 KB copies of these images.  Walks are
// synchronous (one
// workgroup barrier per tile, double-buffered copies); a wave whose block did
// not select the tile skips its products.  With content-adaptive tiles
// (SparseBwdArgs::tdim set) the same passes run over the 64-token tiles, each
// tile's tokens found from its first token and shape.
#include "attn_core.hpp"

namespace mmdit {

namespace {

// Block (of the workgroup's four) served by wave w; waves w and w + 4 share
// a SIMD.  A group is a 2 x 2 (h, w) square of neighbouring blocks, and each
// SIMD gets one wave of each block of a diagonal pair (blocks 0 and 3 on
// SIMDs 0-1, 1 and 2 on SIMDs 2-3), as in the forward: on the 24 x 64 x 112
// smooth-field selections a lockstep walk then leaves a SIMD with a single
// busy wave less often than with edge neighbours paired (measured 1.2 %
// faster over the three passes).
__device__ __forceinline__ int simd_pair_side(int w) { return w < 4 ? (w >> 1) : 3 - ((w - 4) >> 1); }

// Token offset of block-local token r (raster inside the block) from the
// block's first token.
__device__ __forceinline__ int block_off(const SparseGeom& g, int r) {
    const int a = r / (g.BH * g.BW);
    const int rr = r - a * (g.BH * g.BW);
    const int b = rr / g.BW;
    const int c = rr - b * g.BW;
    return (a * g.H + b) * g.W + c;
}

// Raster token of local token r of block (or adaptive tile) j.
__device__ __forceinline__ int64_t bwd_token(const SparseGeom& g, const int32_t* tbase, const uint8_t* tdim, int j,
                                             int r) {
    return tdim ? (int64_t)tbase[j] + tile_local(g, tdim[j], r) : block_token(g, j, 0) + block_off(g, r);
}

// One workgroup per (block, head): the block's 64 tokens of src, transposed
// to [HD][64] bf16 and laid out as the LDS image of a transposed tile (chunk
// u of the image holds (d, c) = v_at(u): tokens 8c .. 8c + 7 of row d).  The
// 16-bit values move as halves of 32-bit words.
template <int HD>
__global__ __launch_bounds__(256) void block_timg_kernel(SparseGeom g, const __bf16* __restrict__ src,
                                                         __bf16* __restrict__ dst, const int32_t* __restrict__ tbase,
                                                         const uint8_t* __restrict__ tdim) {
    using L = TileLayout<HD>;
    __shared__ uint16_t tile[kTileN][HD + 2];
    const int j = blockIdx.x, head = blockIdx.y;
    const int64_t rs = (int64_t)g.heads * HD;
    constexpr int CPR = HD / 8;
    for (int u = threadIdx.x; u < kTileN * CPR; u += 256) {
        const int r = u / CPR, c = u % CPR;
        const int64_t tok = bwd_token(g, tbase, tdim, j, r);
        const uint4 x = *reinterpret_cast<const uint4*>(src + tok * rs + head * HD + c * 8);
        const uint32_t wv[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) tile[r][c * 8 + i] = (uint16_t)(wv[i >> 1] >> (16 * (i & 1)));
    }
    __syncthreads();
    __bf16* out = dst + ((int64_t)head * g.nb + j) * (HD * kTileN);
    for (int u = threadIdx.x; u < HD * (kTileN / 8); u += 256) {
        int d, c;
        L::v_at(u, d, c);
        auto pair = [&](int i) { return (uint32_t)tile[c * 8 + i][d] | ((uint32_t)tile[c * 8 + i + 1][d] << 16); };
        *reinterpret_cast<uint4*>(out + u * 8) = make_uint4(pair(0), pair(2), pair(4), pair(6));
    }
}

// One workgroup per (block, head): the block's 64 rows of src laid out as
// the LDS image of a row-major tile (chunk u of the image holds chunk c of
// tile row r, (r, c) = k_at(u), and tile row r holds block-local token
// (r & ~31) | perm_row(r & 31), the order the products take).  The walks
// then stage a tile with contiguous 1 KB copies: gathering the 64 scattered
// 256-byte rows per tile in the walk itself cost ~14 % of the backward.
template <int HD>
__global__ __launch_bounds__(256) void block_rimg_kernel(SparseGeom g, const __bf16* __restrict__ src,
                                                         __bf16* __restrict__ dst, const int32_t* __restrict__ tbase,
                                                         const uint8_t* __restrict__ tdim) {
    using L = TileLayout<HD>;
    const int j = blockIdx.x, head = blockIdx.y;
    const int64_t rs = (int64_t)g.heads * HD;
    __bf16* out = dst + ((int64_t)head * g.nb + j) * (HD * kTileN);
    for (int u = threadIdx.x; u < kTileN * L::kKChunks; u += 256) {
        int row, c;
        L::k_at(u, row, c);
        const int64_t tok = bwd_token(g, tbase, tdim, j, (row & ~31) | perm_row(row & 31));
        *reinterpret_cast<uint4*>(out + u * 8) = *reinterpret_cast<const uint4*>(src + tok * rs + head * HD + c * 8);
    }
}

// maskT[head][j][w] bit b = mask[head][32 w + b][j / 32] bit j % 32 (0 past nb).
__global__ __launch_bounds__(256) void mask_transpose_kernel(const uint32_t* __restrict__ mask, int nb, int heads,
                                                             uint32_t* __restrict__ maskt) {
    const int nw = (nb + 31) >> 5;
    const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (id >= (int64_t)heads * nb * nw) return;
    const int wi = (int)(id % nw);
    const int64_t hj = id / nw;
    const int j = (int)(hj % nb);
    const int head = (int)(hj / nb);
    const uint32_t* col = mask + (int64_t)head * nb * nw + (j >> 5);
    uint32_t word = 0u;
    for (int b = 0; b < 32; ++b) {
        const int i = 32 * wi + b;
        if (i >= nb) break;
        word |= ((col[(int64_t)i * nw] >> (j & 31)) & 1u) << b;
    }
    maskt[id] = word;
}

constexpr int kSG = kBwdGroup;   // blocks per workgroup (2 waves of 32 tokens each)

// Cursor over the union of kSG bitmask rows staged in LDS (the same walk in
// every wave; values are wave-uniform).
struct UnionWalk {
    const uint32_t (*rows)[kSelMax / 32];
    int nw, word;
    uint32_t bits;
    __device__ uint32_t union_word(int wd) const {
        uint32_t u = 0u;
#pragma unroll
        for (int sd = 0; sd < kSG; ++sd) u |= rows[sd][wd];
        return __builtin_amdgcn_readfirstlane(u);
    }
    __device__ void init(const uint32_t (*r)[kSelMax / 32], int n_words) {
        rows = r;
        nw = n_words;
        word = 0;
        bits = nw > 0 ? union_word(0) : 0u;
    }
    __device__ int next() {
        while (bits == 0u) {
            if (++word >= nw) return -1;
            bits = union_word(word);
        }
        const int b = __builtin_ctz(bits);
        bits &= bits - 1u;
        return word * 32 + b;
    }
};

__device__ __forceinline__ void dma4(const void* gp, char* lds_wave_base) {
    __builtin_amdgcn_global_load_lds(gp, MMDIT_LDS(lds_wave_base), 4, 0, 0);
}


template <int HD>
__global__ __launch_bounds__(8 * kWave) void sparse_bwd_dq_kernel(SparseGeom g, SparseBwdArgs a) {
    using L = TileLayout<HD>;
    constexpr int NW = 8;
    constexpr int KS = HD / 16;
    constexpr int DB = HD / 32;
    constexpr int CK = kTileN * L::kKChunks / (kWave * NW);
    constexpr int CV = HD * 8 / (kWave * NW);
    static_assert(CK >= 1 && CV >= 1, "tile copies");
    constexpr int kBuf = 2 * L::kKBytes + L::kVBytes;   // K rows | V rows | K^T
    __shared__ __attribute__((aligned(16))) char lds[2 * kBuf];
    __shared__ uint32_t msk[kSG][kSelMax / 32];

    const int groups = (g.nb + kSG - 1) / kSG;
    int head, grp;
    if (!group_of_workgroup(groups, g.heads, a.order_q, head, grp)) return;
    const int b0 = kSG * grp;
    const int nw = (g.nb + 31) >> 5;
    const int64_t n = (int64_t)g.T * g.H * g.W;

    const uint32_t* mrow = a.mask + ((int64_t)head * g.nb + b0) * nw;
    for (int i = threadIdx.x; i < kSG * nw; i += NW * kWave) {
        const int sd = i / nw, wd = i - (i / nw) * nw;
        msk[sd][wd] = (b0 + sd < g.nb) ? mrow[sd * nw + wd] : 0u;
    }
    __syncthreads();

    const int w = wave_id();
    const int lane = threadIdx.x & 63;
    const int hh = lane >> 5;
    const int m = lane & 31;
    const int side = simd_pair_side(w);
    const int64_t rstride = (int64_t)g.heads * HD;
    const bool own_ok = b0 + side < g.nb;
    const int qb = min(b0 + side, g.nb - 1);
    const int64_t qtok = bwd_token(g, a.tbase, a.tdim, qb, (w & 1) * 32 + m);
    bf16x8 qr[KS], gr[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        qr[ks] = load_bf16x8(a.q + qtok * rstride + head * HD + 16 * ks + 8 * hh, true);
        gr[ks] = load_bf16x8(a.d_o + qtok * rstride + head * HD + 16 * ks + 8 * hh, true);
    }
    const float lq2 = a.ls2[(int64_t)head * n + qtok];
    const float dq_d = a.dd[(int64_t)head * n + qtok];

    // this lane's 16 bytes of each 1 KB copy of the per-block images
    const int64_t img = (int64_t)head * g.nb * (HD * kTileN);
    const char* kig = reinterpret_cast<const char*>(a.k_img + img) + 16 * lane;
    const char* vig = reinterpret_cast<const char*>(a.v_img + img) + 16 * lane;
    const char* ktg = reinterpret_cast<const char*>(a.kt_img + img) + 16 * lane;

    auto buf = [&](int t) { return lds + (t & 1) * kBuf; };
    auto issue = [&](int j, char* b) {
        const int64_t jb = (int64_t)j * (HD * kTileN * 2);
#pragma unroll
        for (int i = 0; i < CK; ++i) {
            dma16(kig + jb + (w * CK + i) * 1024, b + (w * CK + i) * 1024);
            dma16(vig + jb + (w * CK + i) * 1024, b + L::kKBytes + (w * CK + i) * 1024);
        }
        const char* src = ktg + jb;
#pragma unroll
        for (int i = 0; i < CV; ++i)
            dma16(src + (w * CV + i) * 1024, b + 2 * L::kKBytes + (w * CV + i) * 1024);
    };

    FragAddr<HD> fa;
    fa.init();
    f32x16 dqt[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) dqt[db][r] = 0.f;

    UnionWalk walk;
    walk.init(msk, nw);
    int cur = walk.next();
    if (cur >= 0) issue(cur, buf(0));
    wait_dma();
    __syncthreads();
    int own_word = -1;
    uint32_t own = 0u;
    for (int t = 0; cur >= 0; ++t) {
        const int nxt = walk.next();
        if (nxt >= 0) issue(nxt, buf(t + 1));
        if ((cur >> 5) != own_word) {
            own_word = cur >> 5;
            own = __builtin_amdgcn_readfirstlane(msk[side][own_word]);
        }
        if ((own >> (cur & 31)) & 1u) {
            const char* lk = buf(t);
            const char* lv = lk + L::kKBytes;
            const char* lkt = lk + 2 * L::kKBytes;
            // One stream of LDS fragments read two products ahead: the S^T
            // and dP^T operands (i = 2 KS kb + 2 ks + {0: K, 1: V}), then
            // the K^T operands of dQ^T (i = NA + 4 db + g).
            constexpr int PD = 2;
            constexpr int NA = 4 * KS, NT = NA + 4 * DB;
            auto frag = [&](int i) -> bf16x8 {
                if (i < NA) return k_frag<HD>((i & 1) ? lv : lk, fa, 2 * ((i >> 1) % KS) + i / (2 * KS));
                const int c = i - NA;
                return *reinterpret_cast<const bf16x8*>(lkt + fa.v[c & 3] + (c >> 2) * 32 * L::kVRowBytes);
            };
            bf16x8 fr[PD];
#pragma unroll
            for (int j = 0; j < PD; ++j) fr[j] = frag(j);
            f32x16 s[2], dp[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) s[kb][r] = dp[kb][r] = 0.f;
#pragma unroll
            for (int i = 0; i < NA; ++i) {
                const int kb = i / (2 * KS), ks = (i >> 1) % KS;
                if (i & 1)
                    dp[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[i % PD], gr[ks], dp[kb], 0, 0, 0);
                else
                    s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[i % PD], qr[ks], s[kb], 0, 0, 0);
                fr[i % PD] = frag(i + PD);
            }
            bf16x8 sb[4];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], a.scale_log2, -lq2));
                    sb[2 * kb + (r >> 3)][r & 7] = (__bf16)(p * (dp[kb][r] - dq_d));
                }
#pragma unroll
            for (int c = 0; c < 4 * DB; ++c) {
                const int i = NA + c;
                dqt[c >> 2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[i % PD], sb[c & 3], dqt[c >> 2], 0, 0, 0);
                if (i + PD < NT) fr[i % PD] = frag(i + PD);
            }
            order_fragment_stream<PD, NT>();
        }
        wait_dma();
        __syncthreads();
        cur = nxt;
    }
    if (!own_ok) return;
    store_o<HD>(a.dq + qtok * rstride + head * HD, dqt, a.scale);
}

// Key-owned pass.  DK = false: S = Q K^T -> P -> dV^T += dO^T P.  DK = true:
// S and dP = dO V^T -> dS -> dK^T += Q^T dS.
template <int HD, bool DK>
__global__ __launch_bounds__(8 * kWave) __attribute__((amdgpu_waves_per_eu(2, 2)))
void sparse_bwd_key_kernel(SparseGeom g, SparseBwdArgs a) {
    using L = TileLayout<HD>;
    constexpr int NW = 8;
    constexpr int KS = HD / 16;
    constexpr int DB = HD / 32;
    constexpr int CK = kTileN * L::kKChunks / (kWave * NW);
    constexpr int CV = HD * 8 / (kWave * NW);
    static_assert(CK >= 1 && CV >= 1, "tile copies");
    // one buffer: Q rows | [dO rows] | (DK ? Q^T : dO^T) | lse2[64] | [D[64]]
    constexpr int kRow = DK ? 2 : 1;
    constexpr int kOffT = kRow * L::kKBytes;
    constexpr int kOffL = kOffT + L::kVBytes;
    constexpr int kBuf = kOffL + (DK ? 2 : 1) * kTileN * 4;
    __shared__ __attribute__((aligned(16))) char lds[2 * kBuf];
    __shared__ uint32_t msk[kSG][kSelMax / 32];

    const int groups = (g.nb + kSG - 1) / kSG;
    int head, grp;
    if (!group_of_workgroup(groups, g.heads, a.order_k, head, grp)) return;
    const int c0 = kSG * grp;
    const int nw = (g.nb + 31) >> 5;
    const int64_t n = (int64_t)g.T * g.H * g.W;

    const uint32_t* mrow = a.maskt + ((int64_t)head * g.nb + c0) * nw;
    for (int i = threadIdx.x; i < kSG * nw; i += NW * kWave) {
        const int sd = i / nw, wd = i - (i / nw) * nw;
        msk[sd][wd] = (c0 + sd < g.nb) ? mrow[sd * nw + wd] : 0u;
    }
    __syncthreads();

    const int w = wave_id();
    const int lane = threadIdx.x & 63;
    const int hh = lane >> 5;
    const int m = lane & 31;
    const int side = simd_pair_side(w);
    const int64_t rstride = (int64_t)g.heads * HD;
    const bool own_ok = c0 + side < g.nb;
    const int kb_own = min(c0 + side, g.nb - 1);
    const int64_t ktok = bwd_token(g, a.tbase, a.tdim, kb_own, (w & 1) * 32 + m);
    bf16x8 kr[KS], vr[DK ? KS : 1];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        kr[ks] = load_bf16x8(a.k + ktok * rstride + head * HD + 16 * ks + 8 * hh, true);
        if (DK) vr[ks] = load_bf16x8(a.v + ktok * rstride + head * HD + 16 * ks + 8 * hh, true);
    }

    const int loff = a.tdim ? 0 : block_off(g, lane);   // this lane's query of the lse / D copies
    // this lane's 16 bytes of each 1 KB copy of the per-block images
    const int64_t img = (int64_t)head * g.nb * (HD * kTileN);
    const char* qig = reinterpret_cast<const char*>(a.q_img + img) + 16 * lane;
    const char* oig = reinterpret_cast<const char*>(a.do_img + img) + 16 * lane;
    const char* tg = reinterpret_cast<const char*>((DK ? a.qt_img : a.dot_img) + img) + 16 * lane;
    const float* lsg = a.ls2 + (int64_t)head * n;
    const float* ddg = a.dd + (int64_t)head * n;

    auto buf = [&](int t) { return lds + (t & 1) * kBuf; };
    auto issue = [&](int i, char* b) {
        // raster token of this lane's query of the lse / D copies
        const int64_t lt = a.tdim ? (int64_t)a.tbase[i] + tile_local(g, a.tdim[i], lane) : block_token(g, i, 0) + loff;
        const int64_t ib = (int64_t)i * (HD * kTileN * 2);
#pragma unroll
        for (int c = 0; c < CK; ++c) {
            dma16(qig + ib + (w * CK + c) * 1024, b + (w * CK + c) * 1024);
            if (DK) dma16(oig + ib + (w * CK + c) * 1024, b + L::kKBytes + (w * CK + c) * 1024);
        }
        const char* src = tg + ib;
#pragma unroll
        for (int c = 0; c < CV; ++c) dma16(src + (w * CV + c) * 1024, b + kOffT + (w * CV + c) * 1024);
        if (w == 0) dma4(lsg + lt, b + kOffL);
        if (DK && w == 1) dma4(ddg + lt, b + kOffL + kTileN * 4);
    };

    FragAddr<HD> fa;
    fa.init();
    f32x16 acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;

    UnionWalk walk;
    walk.init(msk, nw);
    int cur = walk.next();
    if (cur >= 0) issue(cur, buf(0));
    wait_dma();
    __syncthreads();
    int own_word = -1;
    uint32_t own = 0u;
    for (int t = 0; cur >= 0; ++t) {
        const int nxt = walk.next();
        if (nxt >= 0) issue(nxt, buf(t + 1));
        if ((cur >> 5) != own_word) {
            own_word = cur >> 5;
            own = __builtin_amdgcn_readfirstlane(msk[side][own_word]);
        }
        if ((own >> (cur & 31)) & 1u) {
            const char* lq = buf(t);
            const char* lo = lq + L::kKBytes;
            const char* lt = lq + kOffT;
            const float* lls = reinterpret_cast<const float*>(lq + kOffL);
            const float* ldd = lls + kTileN;
            // One stream of LDS fragments over both query halves, read two
            // products ahead: per half the S (and dP) operands, ks-major,
            // then the transposed-tile operands of dV^T / dK^T.
            constexpr int PD = 2;
            constexpr int NA = (DK ? 2 : 1) * KS, NQ = NA + 2 * DB, NT = 2 * NQ;
            auto frag = [&](int i) -> bf16x8 {
                const int qb = i / NQ, u = i % NQ;
                if (u < NA) return k_frag<HD>((DK && (u & 1)) ? lo : lq, fa, 2 * (DK ? u >> 1 : u) + qb);
                const int c = u - NA;   // product (db, g) = (c / 2, c % 2)
                return *reinterpret_cast<const bf16x8*>(lt + fa.v[2 * qb + (c & 1)] + (c >> 1) * 32 * L::kVRowBytes);
            };
            bf16x8 fr[PD];
#pragma unroll
            for (int j = 0; j < PD; ++j) fr[j] = frag(j);
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                f32x16 s, dp;
#pragma unroll
                for (int r = 0; r < 16; ++r) s[r] = dp[r] = 0.f;
#pragma unroll
                for (int u = 0; u < NA; ++u) {
                    const int i = qb * NQ + u, ks = DK ? u >> 1 : u;
                    if (DK && (u & 1))
                        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[i % PD], vr[ks], dp, 0, 0, 0);
                    else
                        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[i % PD], kr[ks], s, 0, 0, 0);
                    fr[i % PD] = frag(i + PD);
                }
                // register r holds block-local query 32 qb + 16 (r / 8) + 8 hh + r % 8
                bf16x8 xb[2];
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int h4 = 0; h4 < 2; ++h4) {
                        const int qi = 32 * qb + 16 * j + 8 * hh + 4 * h4;
                        const float4 x = *reinterpret_cast<const float4*>(lls + qi);
                        const float lsv[4] = {x.x, x.y, x.z, x.w};
                        float ddv[4] = {0.f, 0.f, 0.f, 0.f};
                        if (DK) {
                            const float4 y = *reinterpret_cast<const float4*>(ldd + qi);
                            ddv[0] = y.x, ddv[1] = y.y, ddv[2] = y.z, ddv[3] = y.w;
                        }
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int r = 8 * j + 4 * h4 + e;
                            const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], a.scale_log2, -lsv[e]));
                            xb[j][4 * h4 + e] = (__bf16)(DK ? p * (dp[r] - ddv[e]) : p);
                        }
                    }
#pragma unroll
                for (int c = 0; c < 2 * DB; ++c) {
                    const int i = qb * NQ + NA + c;
                    acc[c >> 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[i % PD], xb[c & 1], acc[c >> 1], 0, 0, 0);
                    if (i + PD < NT) fr[i % PD] = frag(i + PD);
                }
            }
            // the half's lse (and D) reads join the stream before its dV^T / dK^T products
            order_fragment_stream<PD, NT, NQ, NA - 1, DK ? 8 : 4>();
        }
        wait_dma();
        __syncthreads();
        cur = nxt;
    }
    if (!own_ok) return;
    if (DK)
        store_o<HD>(a.dk + ktok * rstride + head * HD, acc, a.scale);
    else
        store_o<HD>(a.dv + ktok * rstride + head * HD, acc, 1.f);
}

}  // namespace

hipError_t launch_block_timg(const SparseGeom& g, const __bf16* src, __bf16* dst, const int32_t* tbase,
                             const uint8_t* tdim, hipStream_t s) {
    hipLaunchKernelGGL(block_timg_kernel<128>, dim3(g.nb, g.heads), dim3(256), 0, s, g, src, dst, tbase, tdim);
    return hipGetLastError();
}

hipError_t launch_block_rimg(const SparseGeom& g, const __bf16* src, __bf16* dst, const int32_t* tbase,
                             const uint8_t* tdim, hipStream_t s) {
    hipLaunchKernelGGL(block_rimg_kernel<128>, dim3(g.nb, g.heads), dim3(256), 0, s, g, src, dst, tbase, tdim);
    return hipGetLastError();
}

hipError_t launch_mask_transpose(const SparseGeom& g, const uint32_t* mask, uint32_t* maskt, hipStream_t s) {
    const int64_t words = (int64_t)g.heads * g.nb * ((g.nb + 31) / 32);
    hipLaunchKernelGGL(mask_transpose_kernel, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, s, mask, g.nb,
                       g.heads, maskt);
    return hipGetLastError();
}

hipError_t launch_sparse_bwd(const SparseGeom& g, const SparseBwdArgs& a, hipStream_t s) {
    const unsigned blocks = (unsigned)group_workgroups((g.nb + kSG - 1) / kSG, g.heads);
    const dim3 block(8 * kWave);
    hipLaunchKernelGGL(sparse_bwd_dq_kernel<128>, dim3(blocks), block, 0, s, g, a);
    hipLaunchKernelGGL((sparse_bwd_key_kernel<128, false>), dim3(blocks), block, 0, s, g, a);
    hipLaunchKernelGGL((sparse_bwd_key_kernel<128, true>), dim3(blocks), block, 0, s, g, a);
    return hipGetLastError();
}

}  // namespace mmdit
