// Backward pass of dense softmax attention (training).
//
// The joint model is trained with a flow-matching objective (SkyReels-V4
// analysis, paper.rainbus.top 2602.21818, workflow step 4), so each attention
// of the block is differentiated; the Prism page ("Resultados", efficiency
// gains) compares attention variants by the time of a whole training step.
//
// Per head, with S = s Q K^T, P = softmax over each row, O = P V and the
// upstream gradient dO:
//   dV = P^T dO,  dP = dO V^T,  D_i = <dO_i, O_i>,  dS = P o (dP - D),
//   dQ = s dS K,  dK = s dS^T Q.
// P is recomputed from Q, K and the forward's log-sum-exp, never stored.
//
// bf16 path (products on bf16 matrix cores, fp32 accumulation):
//   bwd_rowterm  D and lse * log2(e) per (head, query), padded to 64 queries
//                with D = 0 and +inf (so padded queries get P = 0);
//   transpose    bf16 Q^T, dO^T [heads][hd][n_q_pad] and K^T [heads][hd][n_kv_pad]
//                (zero padded), the k-contiguous operands of the products
//                that contract over tokens;
//   bwd_key      a workgroup owns 256 keys (8 waves of 32, each wave's K (and
//                V) rows held in registers) and streams the queries in
//                64-query tiles: S = Q K^T (and dP = dO V^T) with the queries
//                as MFMA rows, permuted within each 32-row half as in the
//                forward so that every lane's P (dS) registers come out as the
//                8 consecutive queries the next product takes; then dV^T +=
//                dO^T P in one pass and dK^T += Q^T dS in a second, whose
//                accumulators store like the forward's O^T (one key per lane,
//                d along registers);
//   bwd_dq       a workgroup owns 256 queries (8 waves of 32, Q and dO rows in
//                registers) and streams the keys in 64-key tiles: S^T = K Q^T,
//                dP^T = V dO^T, dQ^T += K^T dS^T.
// dQ is not summed in the key-owned passes: that takes fp32 atomics on dQ
// from every key tile.  The query-owned pass recomputes S and dP instead (8
// products per (query, key) block against the 5 of the definition), and
// every result is deterministic.
#include "attn_core.hpp"

namespace mmdit {

namespace {

// Rows of 16 lanes: row (head-major over queries) = D and lse2 of one (query,
// head); lanes of the row sum HD/16 products each, then reduce by xor.
template <int HD, typename TG>
__global__ __launch_bounds__(256) void bwd_rowterm_kernel(const float* __restrict__ o,
                                                          const TG* __restrict__ d_o,
                                                          const float* __restrict__ lse, int64_t n_q,
                                                          int64_t n_q_pad, int heads,
                                                          float* __restrict__ dd, float* __restrict__ ls2) {
    constexpr int EPL = HD / 16;   // elements per lane
    const int64_t row = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 4;   // = head * n_q_pad + q
    const int part = threadIdx.x & 15;
    if (row >= (int64_t)heads * n_q_pad) return;   // whole 16-lane rows leave together
    const int head = (int)(row / n_q_pad);
    const int64_t q = row - (int64_t)head * n_q_pad;
    float acc = 0.f;
    if (q < n_q) {
        const int64_t base = (q * heads + head) * HD + part * EPL;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc = fmaf(o[base + e], (float)d_o[base + e], acc);
    }
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 16);
    if (part == 0) {
        dd[row] = acc;
        if (ls2) ls2[row] = q < n_q ? lse[(int64_t)head * n_q + q] * kLog2e : __builtin_inff();
    }
}

// [n][heads][HD] bf16 -> [heads][HD][n_pad] bf16, zero past n.  The 16-bit
// values move as halves of 32-bit words (element-wise bit casts of a bf16
// vector have compiled to a copy of its first element).
template <int HD>
__global__ __launch_bounds__(256) void transpose_kernel(const __bf16* __restrict__ src, int64_t n,
                                                        int64_t n_pad, int heads, __bf16* __restrict__ dst) {
    __shared__ uint16_t tile[kTileN][HD + 2];
    const int head = blockIdx.y;
    const int64_t t0 = (int64_t)blockIdx.x * kTileN;
    constexpr int CPR = HD / 8;
    for (int u = threadIdx.x; u < kTileN * CPR; u += 256) {
        const int r = u / CPR, c = u % CPR;
        const int64_t tok = t0 + r;
        uint4 x = make_uint4(0u, 0u, 0u, 0u);
        if (tok < n) x = *reinterpret_cast<const uint4*>(src + (tok * heads + head) * HD + c * 8);
        const uint32_t wv[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) tile[r][c * 8 + i] = (uint16_t)(wv[i >> 1] >> (16 * (i & 1)));
    }
    __syncthreads();
    for (int u = threadIdx.x; u < HD * (kTileN / 8); u += 256) {
        const int d = u / (kTileN / 8), c = u % (kTileN / 8);
        auto pair = [&](int i) { return (uint32_t)tile[c * 8 + i][d] | ((uint32_t)tile[c * 8 + i + 1][d] << 16); };
        *reinterpret_cast<uint4*>(dst + ((int64_t)head * HD + d) * n_pad + t0 + c * 8) =
            make_uint4(pair(0), pair(2), pair(4), pair(6));
    }
}

// Transposed-tile fragment i = 4 db + g as bf16 (same addressing as v_frag).
template <int HD>
__device__ __forceinline__ bf16x8 t_frag(const char* lt, const FragAddr<HD>& fa, int i) {
    return *reinterpret_cast<const bf16x8*>(lt + fa.v[i & 3] + (i >> 2) * 32 * TileLayout<HD>::kVRowBytes);
}

// Asynchronous 4-byte global -> LDS copy: lane i writes lds_wave_base + 4 i.
__device__ __forceinline__ void dma4(const void* g, char* lds_wave_base) {
    __builtin_amdgcn_global_load_lds(g, MMDIT_LDS(lds_wave_base), 4, 0, 0);
}

__device__ __forceinline__ int xcd_logical(int total) {
    const int per_xcd = (total + 7) >> 3;
    return (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
}

// Key-owned pass.  DK = false: S = Q K^T -> P -> dV^T += dO^T P.  DK = true:
// S = Q K^T and dP = dO V^T -> dS -> dK^T += Q^T dS.  Two passes at two waves
// per SIMD (each wave holds one fp32 accumulator block set) instead of one
// pass at one wave per SIMD: the fused pass needs K, V, dK^T and dV^T in
// registers (~380), and with four waves a 64-query tile brought only half
// the matrix-core work per copied byte of the forward, so the waves waited on
// the copies; the split recomputes S once more.
template <int HD, bool DK>
__global__ __launch_bounds__(kBwdKvWaves * kWave) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_key_kernel(BwdArgs a) {
    using L = TileLayout<HD>;
    constexpr int NW = kBwdKvWaves;
    constexpr int KS = HD / 16;
    constexpr int DB = HD / 32;
    constexpr int CK = kTileN * L::kKChunks / (kWave * NW);   // copies per wave of a row-major tile
    constexpr int CV = HD * 8 / (kWave * NW);                 // copies per wave of a transposed tile
    static_assert(NW >= 2 && CK >= 1 && CV >= 1, "tile copies");
    // one buffer: Q | [dO] | (DK ? Q^T : dO^T) | lse2[64] | [D[64]]
    constexpr int kRow = DK ? 2 : 1;                           // row-major tiles
    constexpr int kOffT = kRow * L::kKBytes;                   // the transposed tile
    constexpr int kOffL = kOffT + L::kVBytes;                  // lse2, then D
    constexpr int kBuf = kOffL + (DK ? 2 : 1) * kTileN * 4;
    __shared__ __attribute__((aligned(16))) char lds[2 * kBuf];

    const int kv_tiles = (int)((a.n_kv + kBwdKvKeys - 1) / kBwdKvKeys);
    const int total = kv_tiles * a.heads;
    const int logical = xcd_logical(total);
    if (logical >= total) return;
    const int kt = logical % kv_tiles;
    const int head = logical / kv_tiles;

    const int w = wave_id();
    const int lane = threadIdx.x & 63;
    const int hh = lane >> 5;
    const int m = lane & 31;
    const int64_t rstride = (int64_t)a.heads * HD;
    const int64_t rb = rstride * 2;   // bytes per token row

    // the key this lane holds in the B operands of S and dP (column m of the
    // wave's 32-key block), and its 8 d values per k-step
    const int64_t key = (int64_t)kt * kBwdKvKeys + w * 32 + m;
    const bool kok = key < a.n_kv;
    bf16x8 kr[KS], vr[DK ? KS : 1];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        kr[ks] = load_bf16x8(a.k + key * rstride + head * HD + 16 * ks + 8 * hh, kok);
        if (DK) vr[ks] = load_bf16x8(a.v + key * rstride + head * HD + 16 * ks + 8 * hh, kok);
    }

    auto q_slot = [&](int i, int& qrow, int& c) {
        int row;
        L::k_at((w * CK + i) * kWave + lane, row, c);
        qrow = (row & ~31) | perm_row(row & 31);
    };
    uint32_t roff[CK];
#pragma unroll
    for (int i = 0; i < CK; ++i) {
        int r, c;
        q_slot(i, r, c);
        roff[i] = (uint32_t)(r * rb + c * 16);
    }
    uint32_t toff[CV];
#pragma unroll
    for (int i = 0; i < CV; ++i) {
        int d, c;
        L::v_at((w * CV + i) * kWave + lane, d, c);
        toff[i] = (uint32_t)((d * a.n_q_pad + c * 8) * 2);
    }
    const char* qg = reinterpret_cast<const char*>(a.q + head * HD);
    const char* og = reinterpret_cast<const char*>(a.d_o + head * HD);
    const char* tg = reinterpret_cast<const char*>((DK ? a.qt : a.dot) + (int64_t)head * HD * a.n_q_pad);
    const float* lsg = a.ls2 + (int64_t)head * a.n_q_pad;
    const float* ddg = a.dd + (int64_t)head * a.n_q_pad;

    auto buf = [&](int t) { return lds + (t & 1) * kBuf; };
    auto issue = [&](int t, char* b) {
        const int64_t q0 = (int64_t)t * kTileN;
        if (q0 + kTileN <= a.n_q) {
#pragma unroll
            for (int i = 0; i < CK; ++i) {
                dma16(qg + q0 * rb + roff[i], b + (w * CK + i) * 1024);
                if (DK) dma16(og + q0 * rb + roff[i], b + L::kKBytes + (w * CK + i) * 1024);
            }
        } else {   // rows past n_q re-read the last real row; their P is 0 (lse2 = +inf)
            const int last = (int)(a.n_q - q0) - 1;
#pragma unroll
            for (int i = 0; i < CK; ++i) {
                int r, c;
                q_slot(i, r, c);
                const int64_t off = (q0 + min(r, last)) * rb + c * 16;
                dma16(qg + off, b + (w * CK + i) * 1024);
                if (DK) dma16(og + off, b + L::kKBytes + (w * CK + i) * 1024);
            }
        }
#pragma unroll
        for (int i = 0; i < CV; ++i) dma16(tg + q0 * 2 + toff[i], b + kOffT + (w * CV + i) * 1024);
        if (w == 0) dma4(lsg + q0 + lane, b + kOffL);
        if (DK && w == 1) dma4(ddg + q0 + lane, b + kOffL + kTileN * 4);
    };

    FragAddr<HD> fa;
    fa.init();
    f32x16 acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;

    const int q_tiles = (int)(a.n_q_pad / kTileN);
    if (q_tiles > 0) {
        issue(0, buf(0));
        wait_dma();
        __syncthreads();
    }
    for (int t = 0; t < q_tiles; ++t) {
        if (t + 1 < q_tiles) issue(t + 1, buf(t + 1));
        const char* lq = buf(t);
        const char* lo = lq + L::kKBytes;
        const char* lt = lq + kOffT;
        const float* lls = reinterpret_cast<const float*>(lq + kOffL);
        const float* ldd = lls + kTileN;
        // One stream of LDS fragments over both query halves, read two
        // products ahead: per half the S (and dP) operands, ks-major, then
        // the transposed-tile operands of dV^T / dK^T.
        constexpr int PD = 2;
        constexpr int NA = (DK ? 2 : 1) * KS, NQ = NA + 2 * DB, NT = 2 * NQ;
        auto frag = [&](int i) -> bf16x8 {
            const int qb = i / NQ, u = i % NQ;
            if (u < NA) return k_frag<HD>((DK && (u & 1)) ? lo : lq, fa, 2 * (DK ? u >> 1 : u) + qb);
            const int c = u - NA;   // product (db, g) = (c / 2, c % 2)
            return t_frag<HD>(lt, fa, 4 * (c >> 1) + 2 * qb + (c & 1));
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
            // register r holds query 32 qb + 16 (r / 8) + 8 hh + r % 8 of the tile
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
        wait_dma();
        __syncthreads();
    }
    if (!kok) return;
    if (DK)
        store_o<HD>(a.dk + key * rstride + head * HD, acc, a.scale);
    else
        store_o<HD>(a.dv + key * rstride + head * HD, acc, 1.f);
}

template <int HD>
__global__ __launch_bounds__(kBwdDqWaves * kWave) void bwd_dq_kernel(BwdArgs a) {
    using L = TileLayout<HD>;
    constexpr int NW = kBwdDqWaves;
    constexpr int KS = HD / 16;
    constexpr int DB = HD / 32;
    constexpr int CK = kTileN * L::kKChunks / (kWave * NW);   // copies per wave of a K or V tile
    constexpr int CV = HD * 8 / (kWave * NW);                 // copies per wave of a K^T tile
    static_assert(CK >= 1 && CV >= 1, "tile copies");
    // one buffer: K tile | V tile | K^T tile
    constexpr int kBuf = 2 * L::kKBytes + L::kVBytes;
    __shared__ __attribute__((aligned(16))) char lds[2 * kBuf];

    const int q_tiles = (int)((a.n_q + kBwdDqQueries - 1) / kBwdDqQueries);
    const int total = q_tiles * a.heads;
    const int logical = xcd_logical(total);
    if (logical >= total) return;
    const int qt = logical % q_tiles;
    const int head = logical / q_tiles;

    const int w = wave_id();
    const int lane = threadIdx.x & 63;
    const int hh = lane >> 5;
    const int m = lane & 31;
    const int64_t rstride = (int64_t)a.heads * HD;
    const int64_t rb = rstride * 2;

    const int64_t query = (int64_t)qt * kBwdDqQueries + w * 32 + m;
    const bool qok = query < a.n_q;
    bf16x8 qr[KS], gr[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        qr[ks] = load_bf16x8(a.q + query * rstride + head * HD + 16 * ks + 8 * hh, qok);
        gr[ks] = load_bf16x8(a.d_o + query * rstride + head * HD + 16 * ks + 8 * hh, qok);
    }
    const float lq2 = qok ? a.ls2[(int64_t)head * a.n_q_pad + query] : __builtin_inff();
    const float dq_d = qok ? a.dd[(int64_t)head * a.n_q_pad + query] : 0.f;

    auto k_slot = [&](int i, int& krow, int& c) {
        int row;
        L::k_at((w * CK + i) * kWave + lane, row, c);
        krow = (row & ~31) | perm_row(row & 31);
    };
    uint32_t roff[CK];
#pragma unroll
    for (int i = 0; i < CK; ++i) {
        int r, c;
        k_slot(i, r, c);
        roff[i] = (uint32_t)(r * rb + c * 16);
    }
    uint32_t toff[CV];
#pragma unroll
    for (int i = 0; i < CV; ++i) {
        int d, c;
        L::v_at((w * CV + i) * kWave + lane, d, c);
        toff[i] = (uint32_t)((d * a.n_kv_pad + c * 8) * 2);
    }
    const char* kg = reinterpret_cast<const char*>(a.k + head * HD);
    const char* vg = reinterpret_cast<const char*>(a.v + head * HD);
    const char* ktg = reinterpret_cast<const char*>(a.kt + (int64_t)head * HD * a.n_kv_pad);

    auto buf = [&](int t) { return lds + (t & 1) * kBuf; };
    auto issue = [&](int t, char* b) {
        const int64_t k0 = (int64_t)t * kTileN;
        if (k0 + kTileN <= a.n_kv) {
#pragma unroll
            for (int i = 0; i < CK; ++i) {
                dma16(kg + k0 * rb + roff[i], b + (w * CK + i) * 1024);
                dma16(vg + k0 * rb + roff[i], b + L::kKBytes + (w * CK + i) * 1024);
            }
        } else {   // rows past n_kv re-read the last real row; their scores are masked
            const int last = (int)(a.n_kv - k0) - 1;
#pragma unroll
            for (int i = 0; i < CK; ++i) {
                int r, c;
                k_slot(i, r, c);
                const int64_t off = (k0 + min(r, last)) * rb + c * 16;
                dma16(kg + off, b + (w * CK + i) * 1024);
                dma16(vg + off, b + L::kKBytes + (w * CK + i) * 1024);
            }
        }
#pragma unroll
        for (int i = 0; i < CV; ++i) dma16(ktg + k0 * 2 + toff[i], b + 2 * L::kKBytes + (w * CV + i) * 1024);
    };

    FragAddr<HD> fa;
    fa.init();
    f32x16 dqt[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) dqt[db][r] = 0.f;

    const int kv_tiles = (int)(a.n_kv_pad / kTileN);
    issue(0, buf(0));
    wait_dma();
    __syncthreads();
    for (int t = 0; t < kv_tiles; ++t) {
        if (t + 1 < kv_tiles) issue(t + 1, buf(t + 1));
        const char* lk = buf(t);
        const char* lv = lk + L::kKBytes;
        const char* lkt = lk + 2 * L::kKBytes;
        // One stream of LDS fragments read two products ahead: the S^T and
        // dP^T operands (i = 2 KS kb + 2 ks + {0: K, 1: V}), then the K^T
        // operands of dQ^T (i = NA + 4 db + g).
        constexpr int PD = 2;
        constexpr int NA = 4 * KS, NT = NA + 4 * DB;
        auto frag = [&](int i) -> bf16x8 {
            if (i < NA) return k_frag<HD>((i & 1) ? lv : lk, fa, 2 * ((i >> 1) % KS) + i / (2 * KS));
            return t_frag<HD>(lkt, fa, i - NA);
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
        const int valid = (int)min<int64_t>(kTileN, a.n_kv - (int64_t)t * kTileN);
        bf16x8 sb[4];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], a.scale_log2, -lq2));
                if (tile_key(kb, r, hh) >= valid) p = 0.f;
                sb[2 * kb + (r >> 3)][r & 7] = (__bf16)(p * (dp[kb][r] - dq_d));
            }
#pragma unroll
        for (int c = 0; c < 4 * DB; ++c) {
            const int i = NA + c;
            dqt[c >> 2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[i % PD], sb[c & 3], dqt[c >> 2], 0, 0, 0);
            if (i + PD < NT) fr[i % PD] = frag(i + PD);
        }
        order_fragment_stream<PD, NT>();
        wait_dma();
        __syncthreads();
    }
    if (!qok) return;
    store_o<HD>(a.dq + query * rstride + head * HD, dqt, a.scale);
}

// fp32 path: one lane per (query, head) for dQ and one per (key, head) for
// dK and dV, walking the other side in order.  Meant for small problems.
template <int HD>
__global__ __launch_bounds__(64) void bwd_dq_fp32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                                                         const float* __restrict__ v, const float* __restrict__ d_o,
                                                         const float* __restrict__ lse,
                                                         const float* __restrict__ dd, int64_t n_q, int64_t n_kv,
                                                         int heads, float scale, float* __restrict__ dq) {
    const int head = blockIdx.y;
    const int64_t qi = (int64_t)blockIdx.x * 64 + threadIdx.x;
    if (qi >= n_q) return;
    const int64_t rs = (int64_t)heads * HD;
    float qv[HD], gv[HD], acc[HD];
#pragma unroll
    for (int d = 0; d < HD; ++d) {
        qv[d] = q[qi * rs + head * HD + d];
        gv[d] = d_o[qi * rs + head * HD + d];
        acc[d] = 0.f;
    }
    const float ls = lse[(int64_t)head * n_q + qi];
    const float dr = dd[(int64_t)head * n_q + qi];
    for (int64_t j = 0; j < n_kv; ++j) {
        const float* kr = k + j * rs + head * HD;
        const float* vr = v + j * rs + head * HD;
        float sdot = 0.f, gdot = 0.f;
#pragma unroll
        for (int d = 0; d < HD; ++d) {
            sdot = fmaf(qv[d], kr[d], sdot);
            gdot = fmaf(gv[d], vr[d], gdot);
        }
        const float ds = expf(sdot * scale - ls) * (gdot - dr);
#pragma unroll
        for (int d = 0; d < HD; ++d) acc[d] = fmaf(ds, kr[d], acc[d]);
    }
#pragma unroll
    for (int d = 0; d < HD; ++d) dq[qi * rs + head * HD + d] = acc[d] * scale;
}

template <int HD, bool DK>
__global__ __launch_bounds__(64) void bwd_dkdv_fp32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                                                           const float* __restrict__ v, const float* __restrict__ d_o,
                                                           const float* __restrict__ lse,
                                                           const float* __restrict__ dd, int64_t n_q, int64_t n_kv,
                                                           int heads, float scale, float* __restrict__ out) {
    const int head = blockIdx.y;
    const int64_t kj = (int64_t)blockIdx.x * 64 + threadIdx.x;
    if (kj >= n_kv) return;
    const int64_t rs = (int64_t)heads * HD;
    float kv[HD], acc[HD];
#pragma unroll
    for (int d = 0; d < HD; ++d) {
        kv[d] = k[kj * rs + head * HD + d];
        acc[d] = 0.f;
    }
    const float* vr = v + kj * rs + head * HD;
    for (int64_t i = 0; i < n_q; ++i) {
        const float* qr = q + i * rs + head * HD;
        const float* gr = d_o + i * rs + head * HD;
        float sdot = 0.f;
#pragma unroll
        for (int d = 0; d < HD; ++d) sdot = fmaf(qr[d], kv[d], sdot);
        const float p = expf(sdot * scale - lse[(int64_t)head * n_q + i]);
        if (DK) {   // dK_j += dS_ij q_i
            float gdot = 0.f;
#pragma unroll
            for (int d = 0; d < HD; ++d) gdot = fmaf(gr[d], vr[d], gdot);
            const float ds = p * (gdot - dd[(int64_t)head * n_q + i]);
#pragma unroll
            for (int d = 0; d < HD; ++d) acc[d] = fmaf(ds, qr[d], acc[d]);
        } else {    // dV_j += P_ij dO_i
#pragma unroll
            for (int d = 0; d < HD; ++d) acc[d] = fmaf(p, gr[d], acc[d]);
        }
    }
    const float mul = DK ? scale : 1.f;
#pragma unroll
    for (int d = 0; d < HD; ++d) out[kj * rs + head * HD + d] = acc[d] * mul;
}

}  // namespace

hipError_t launch_bwd_rowterm(const float* o, const void* d_o, int dtype, const float* lse, int64_t n_q,
                              int64_t n_q_pad, int heads, int hd, float* dd, float* ls2, hipStream_t s) {
    const int64_t rows = (int64_t)heads * n_q_pad;
    const unsigned blocks = (unsigned)((rows * 16 + 255) / 256);
    if (blocks == 0) return hipSuccess;
    if (dtype == MMDIT_BF16) {
        const __bf16* g = (const __bf16*)d_o;
        if (hd == 128)
            hipLaunchKernelGGL((bwd_rowterm_kernel<128, __bf16>), dim3(blocks), dim3(256), 0, s, o, g, lse, n_q,
                               n_q_pad, heads, dd, ls2);
        else
            hipLaunchKernelGGL((bwd_rowterm_kernel<64, __bf16>), dim3(blocks), dim3(256), 0, s, o, g, lse, n_q,
                               n_q_pad, heads, dd, ls2);
    } else {
        const float* g = (const float*)d_o;
        if (hd == 128)
            hipLaunchKernelGGL((bwd_rowterm_kernel<128, float>), dim3(blocks), dim3(256), 0, s, o, g, lse, n_q,
                               n_q_pad, heads, dd, ls2);
        else
            hipLaunchKernelGGL((bwd_rowterm_kernel<64, float>), dim3(blocks), dim3(256), 0, s, o, g, lse, n_q,
                               n_q_pad, heads, dd, ls2);
    }
    return hipGetLastError();
}

hipError_t launch_transpose(const __bf16* src, int64_t n, int64_t n_pad, int heads, int hd, __bf16* dst,
                            hipStream_t s) {
    if (n_pad == 0) return hipSuccess;
    dim3 grid((unsigned)(n_pad / kTileN), (unsigned)heads);
    if (hd == 128)
        hipLaunchKernelGGL(transpose_kernel<128>, grid, dim3(256), 0, s, src, n, n_pad, heads, dst);
    else
        hipLaunchKernelGGL(transpose_kernel<64>, grid, dim3(256), 0, s, src, n, n_pad, heads, dst);
    return hipGetLastError();
}

hipError_t launch_bwd_keys(const BwdArgs& a, int hd, hipStream_t s) {
    const int64_t kv_tiles = (a.n_kv + kBwdKvKeys - 1) / kBwdKvKeys;
    const unsigned blocks = (unsigned)((kv_tiles * a.heads + 7) / 8 * 8);
    const dim3 grid(blocks), block(kBwdKvWaves * kWave);
    if (hd == 128) {
        hipLaunchKernelGGL((bwd_key_kernel<128, false>), grid, block, 0, s, a);
        hipLaunchKernelGGL((bwd_key_kernel<128, true>), grid, block, 0, s, a);
    } else {
        hipLaunchKernelGGL((bwd_key_kernel<64, false>), grid, block, 0, s, a);
        hipLaunchKernelGGL((bwd_key_kernel<64, true>), grid, block, 0, s, a);
    }
    return hipGetLastError();
}

hipError_t launch_bwd_dq(const BwdArgs& a, int hd, hipStream_t s) {
    const int64_t q_tiles = (a.n_q + kBwdDqQueries - 1) / kBwdDqQueries;
    const unsigned blocks = (unsigned)((q_tiles * a.heads + 7) / 8 * 8);
    if (blocks == 0) return hipSuccess;
    if (hd == 128)
        hipLaunchKernelGGL(bwd_dq_kernel<128>, dim3(blocks), dim3(kBwdDqWaves * kWave), 0, s, a);
    else
        hipLaunchKernelGGL(bwd_dq_kernel<64>, dim3(blocks), dim3(kBwdDqWaves * kWave), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_bwd_fp32(const float* q, const float* k, const float* v, const float* d_o, const float* lse,
                           const float* dd, int64_t n_q, int64_t n_kv, int heads, int hd, float scale, float* dq,
                           float* dk, float* dv, hipStream_t s) {
    const dim3 gq((unsigned)((n_q + 63) / 64), (unsigned)heads), gk((unsigned)((n_kv + 63) / 64), (unsigned)heads);
    if (hd == 128) {
        if (n_q > 0)
            hipLaunchKernelGGL(bwd_dq_fp32_kernel<128>, gq, dim3(64), 0, s, q, k, v, d_o, lse, dd, n_q, n_kv, heads,
                               scale, dq);
        hipLaunchKernelGGL((bwd_dkdv_fp32_kernel<128, true>), gk, dim3(64), 0, s, q, k, v, d_o, lse, dd, n_q, n_kv,
                           heads, scale, dk);
        hipLaunchKernelGGL((bwd_dkdv_fp32_kernel<128, false>), gk, dim3(64), 0, s, q, k, v, d_o, lse, dd, n_q, n_kv,
                           heads, scale, dv);
    } else {
        if (n_q > 0)
            hipLaunchKernelGGL(bwd_dq_fp32_kernel<64>, gq, dim3(64), 0, s, q, k, v, d_o, lse, dd, n_q, n_kv, heads,
                               scale, dq);
        hipLaunchKernelGGL((bwd_dkdv_fp32_kernel<64, true>), gk, dim3(64), 0, s, q, k, v, d_o, lse, dd, n_q, n_kv,
                           heads, scale, dk);
        hipLaunchKernelGGL((bwd_dkdv_fp32_kernel<64, false>), gk, dim3(64), 0, s, q, k, v, d_o, lse, dd, n_q, n_kv,
                           heads, scale, dv);
    }
    return hipGetLastError();
}

}  // namespace mmdit
