// Dense softmax attention kernels.
//
//   O_i = sum_j softmax_j(s <q_i, k_j>) v_j   per head, no mask
//
// which the SkyReels-V4 pages use for the joint self-attention over
// [video | audio | text] tokens, for video queries against text embeddings
// and for both directions of the audio<->video cross-attention
// (paper.rainbus.top analysis, workflow step 3 and novelty 2; trdm.cn
// article, sections 2.1-2.2).
//
// bf16 path: 512-thread workgroups (8 waves x 32 queries = 256 queries, one
// workgroup and two waves per SIMD on a CU) walk the key range in 64-key
// tiles staged through LDS by direct global -> LDS copies; a K tile is shared
// by 256 queries, which halves copy traffic per FLOP against 128-query tiles.  When
// there are too few query tiles to fill 256 CUs (audio queries against video
// keys) the key range is split and a combine kernel merges the partial
// results by their log-sum-exp.  Workgroup ids are remapped so that the
// workgroups running on one XCD (ids congruent mod 8) take consecutive query
// tiles of the same head and share that head's K/V through their L2.
#include "attn_core.hpp"

namespace mmdit {

namespace {

// ---- V prescale: per-head largest magnitude -----------------------------------
// Workgroup (part, head) scans tokens [part * per, (part + 1) * per) of one
// head: each thread reads 16-byte chunks of a fixed column of the head's row.
template <int HD>
__global__ __launch_bounds__(256) void v_absmax_kernel(const __bf16* __restrict__ v, int64_t n, int heads,
                                                       uint32_t* __restrict__ vmax) {
    __shared__ uint32_t wmax[4];
    const int part = blockIdx.x, head = blockIdx.y;
    constexpr int CPR = HD / 8;          // 16-byte chunks per (token, head) row
    constexpr int RPI = 256 / CPR;       // rows per iteration
    const int64_t per = (n + kVmaxParts - 1) / kVmaxParts;
    const int64_t t0 = (int64_t)part * per;
    const int64_t t1 = t0 + per < n ? t0 + per : n;
    const int c = threadIdx.x % CPR;
    uint32_t m = 0u;
    for (int64_t t = t0 + threadIdx.x / CPR; t < t1; t += RPI) {
        const uint4 u = *reinterpret_cast<const uint4*>(v + (t * heads + head) * HD + c * 8);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t lo = w[i] & 0x7FFFu, hi = (w[i] >> 16) & 0x7FFFu;
            m = max(m, max(lo, hi));
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o));
    if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0)
        vmax[(int64_t)head * kVmaxParts + part] = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
}

// ---- V^T staging: [n_kv][heads][hd] bf16 -> [heads][hd][n_pad] fp16, x 2^e ----
template <int HD>
__global__ __launch_bounds__(256) void vt_dense_kernel(const __bf16* __restrict__ v, int64_t n_kv,
                                                       int64_t n_pad, int heads, const uint32_t* __restrict__ vmax,
                                                       _Float16* __restrict__ vt) {
    __shared__ _Float16 tile[kTileN][HD + 2];
    const int head = blockIdx.y;
    const float sc = __builtin_ldexpf(1.f, v_scale_exp(vmax, head));
    const int64_t k0 = (int64_t)blockIdx.x * kTileN;
    constexpr int CPR = HD / 8;                 // 16-byte chunks per row
    for (int u = threadIdx.x; u < kTileN * CPR; u += 256) {
        const int r = u / CPR, c = u % CPR;
        const int64_t key = k0 + r;
        const bf16x8 x = load_bf16x8(v + (key * heads + head) * HD + c * 8, key < n_kv);
#pragma unroll
        for (int i = 0; i < 8; ++i) tile[r][c * 8 + i] = (_Float16)((float)x[i] * sc);
    }
    __syncthreads();
    // each thread writes 8 consecutive keys of one d row
    for (int u = threadIdx.x; u < HD * (kTileN / 8); u += 256) {
        const int d = u / (kTileN / 8), c = u % (kTileN / 8);
        f16x8 y;
#pragma unroll
        for (int i = 0; i < 8; ++i) y[i] = tile[c * 8 + i][d];
        *reinterpret_cast<f16x8*>(vt + ((int64_t)head * HD + d) * n_pad + k0 + c * 8) = y;
    }
}

// The staging pass of the RoPE-fused joint attention: the same V^T tile as
// vt_dense_kernel, and the tile's 64 K rows of this head rotated into k_out
// (16 lanes per 256-byte row, one 8-element chunk each).
template <int HD>
__global__ __launch_bounds__(256) void vt_dense_rope_kernel(const __bf16* __restrict__ v, int64_t n_kv,
                                                            int64_t n_pad, int heads,
                                                            const uint32_t* __restrict__ vmax,
                                                            _Float16* __restrict__ vt, RopeFused r) {
    __shared__ _Float16 tile[kTileN][HD + 2];
    const int head = blockIdx.y;
    const float sc = __builtin_ldexpf(1.f, v_scale_exp(vmax, head));
    const int64_t k0 = (int64_t)blockIdx.x * kTileN;
    constexpr int CPR = HD / 8;
    for (int u = threadIdx.x; u < kTileN * CPR; u += 256) {
        const int rr = u / CPR, c = u % CPR;
        const int64_t key = k0 + rr;
        const int64_t off = (key * heads + head) * HD + c * 8;
        const bf16x8 x = load_bf16x8(v + off, key < n_kv);
#pragma unroll
        for (int i = 0; i < 8; ++i) tile[rr][c * 8 + i] = (_Float16)((float)x[i] * sc);
        if (key < n_kv) {
            const bf16x8 kx = load_bf16x8(r.k + off, true);
            *reinterpret_cast<bf16x8*>(r.k_out + off) = rope_chunk_bf16(kx, r.tab, rope_table_index(r.a, key, c * 8));
        }
    }
    __syncthreads();
    for (int u = threadIdx.x; u < HD * (kTileN / 8); u += 256) {
        const int d = u / (kTileN / 8), c = u % (kTileN / 8);
        f16x8 y;
#pragma unroll
        for (int i = 0; i < 8; ++i) y[i] = tile[c * 8 + i][d];
        *reinterpret_cast<f16x8*>(vt + ((int64_t)head * HD + d) * n_pad + k0 + c * 8) = y;
    }
}

// NW waves of QB blocks of 32 queries: a workgroup serves 32 NW QB queries.
// Four-wave workgroups run two per CU, so they must fit two waves per SIMD.
// With ROPE, each lane rotates its Q fragments as it loads them (the RoPE-
// fused joint attention) and the first key split stores them to r->q_out.
template <int HD, int QB, int NW, bool ROPE>
__device__ __forceinline__ void attn_bf16_body(const AttnArgs& a, const RopeFused* r) {
    using L = TileLayout<HD>;
    constexpr int QT = 32 * NW * QB;
    constexpr int KS = HD / 16;
    constexpr int KCH = kTileN * L::kKChunks / (kWave * NW);   // K copies per wave per tile
    constexpr int VCH = HD * 8 / (kWave * NW);                 // V^T copies per wave per tile
    constexpr bool kPin = QB == 1 && NW == 8;                   // fragment stream order pinned
    __shared__ __attribute__((aligned(16))) char lds[2 * L::kBytes];

    const int total = a.q_tiles * a.heads * a.splits;
    const int per_xcd = (total + 7) >> 3;
    const int logical = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
    if (logical >= total) return;
    const int qt = logical % a.q_tiles;
    const int hs = logical / a.q_tiles;
    const int split = hs % a.splits;
    const int head = hs / a.splits;
    const int tile0 = split * a.tiles_per_split;
    const int tile1 = min(a.kv_tiles, tile0 + a.tiles_per_split);

    const int w = wave_id();
    const int lane = threadIdx.x & 63;
    const int hh = lane >> 5;
    const int m = lane & 31;
    const int64_t rstride = (int64_t)a.heads * HD;
    const int64_t krb = rstride * 2;                            // bytes per key row

    // O^T accumulates V scaled by 2^ve; the epilogue scales back (exact)
    const int ve = v_scale_exp(a.vmax, head);
    // query row of this lane in query block qb: qrow0 + 32 qb
    const int64_t qrow0 = (int64_t)qt * QT + w * 32 * QB + m;
    bf16x8 qf[QB][KS];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int64_t qrow = qrow0 + 32 * qb;
            qf[qb][ks] = load_bf16x8(a.q + qrow * rstride + head * HD + 16 * ks + 8 * hh, qrow < a.n_q);
        }
    // Each lane's share of the tile copies, fixed for the whole key walk: the
    // byte offset (from the tile's first key row) of the 16-byte chunk that
    // belongs at its LDS position.
    // tile row (after the pi permutation) and chunk a lane copies in K copy i
    auto k_slot = [&](int i, int& krow, int& c) {
        int row;
        L::k_at((w * KCH + i) * kWave + lane, row, c);
        krow = (row & ~31) | perm_row(row & 31);
    };
    // Eight waves keep the offsets in registers; four waves (twice the copies
    // per wave) recompute them per tile rather than spill.
    constexpr bool kKeep = NW >= 8;
    auto k_off = [&](int i) {
        int krow, c;
        k_slot(i, krow, c);
        return (uint32_t)(krow * krb + c * 16);
    };
    auto v_off = [&](int i) {
        int d, c;
        L::v_at((w * VCH + i) * kWave + lane, d, c);
        return (uint32_t)((d * a.n_pad + c * 8) * 2);
    };
    uint32_t koff[kKeep ? KCH : 1], voff[kKeep ? VCH : 1];
    if constexpr (kKeep) {
#pragma unroll
        for (int i = 0; i < KCH; ++i) koff[i] = k_off(i);
#pragma unroll
        for (int i = 0; i < VCH; ++i) voff[i] = v_off(i);
    }
    const char* kg = reinterpret_cast<const char*>(a.k + head * HD);
    const char* vg = reinterpret_cast<const char*>(a.vt + (int64_t)head * HD * a.n_pad);

    // LDS: two K tiles and two V^T tiles.  The K ring runs one tile ahead of
    // the V ring: step t reads K(t+1) and V(t) while K(t+2) and V(t+1) land.
    auto kbuf = [&](int b) { return lds + b * L::kKBytes; };
    auto vbuf = [&](int b) { return lds + 2 * L::kKBytes + b * L::kVBytes; };
    auto issue_k = [&](int t, char* lb) {
        const int64_t kv0 = (int64_t)t * kTileN;
        const char* kt = kg + kv0 * krb;
        if (kv0 + kTileN <= a.n_kv) {
#pragma unroll
            for (int i = 0; i < KCH; ++i) dma16(kt + (kKeep ? koff[i] : k_off(i)), lb + (w * KCH + i) * 1024);
        } else {   // rows past n_kv re-read the last real row; their scores are masked
            const int last = (int)(a.n_kv - kv0) - 1;
#pragma unroll
            for (int i = 0; i < KCH; ++i) {
                int krow, c;
                k_slot(i, krow, c);
                dma16(kt + (int64_t)min(krow, last) * krb + c * 16, lb + (w * KCH + i) * 1024);
            }
        }
    };
    auto issue_v = [&](int t, char* lb) {
        const char* vt = vg + (int64_t)t * kTileN * 2;
#pragma unroll
        for (int i = 0; i < VCH; ++i) dma16(vt + (kKeep ? voff[i] : v_off(i)), lb + (w * VCH + i) * 1024);
    };

    FragAddr<HD> fa;
    fa.init();
    SoftmaxState<HD, QB> st;
    st.init();
    const int last_valid = (int)(a.n_kv - (int64_t)(tile1 - 1) * kTileN);   // 1..64
    const bool last_partial = last_valid < kTileN;

    issue_k(tile0, kbuf(0));
    issue_v(tile0, vbuf(0));
    if (tile0 + 1 < tile1) issue_k(tile0 + 1, kbuf(1));
    // RoPE-fused calls rotate the Q fragments here, while the first tiles'
    // copies are in flight (their table reads and the rotated rows' stores
    // overlap the copies).
    if constexpr (ROPE) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const int64_t qrow = qrow0 + 32 * qb;
            if (qrow >= a.n_q) continue;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int dim = 16 * ks + 8 * hh;
                qf[qb][ks] = rope_chunk_bf16(qf[qb][ks], r->tab, rope_table_index(r->a, qrow, dim));
                if (r->q_out && split == 0)
                    *reinterpret_cast<bf16x8*>(r->q_out + qrow * rstride + head * HD + dim) = qf[qb][ks];
            }
        }
    }

    wait_dma();
    __syncthreads();
    f32x16 sa[QB][2], sb[QB][2];
    qk_tile<HD, QB>(kbuf(0), fa, qf, sa);
    float mx[QB];
    if (last_partial && tile0 + 1 == tile1)
        tile_max<true, QB>(sa, a.scale_log2, last_valid, mx);
    else
        tile_max<false, QB>(sa, a.scale_log2, kTileN, mx);

    // Top of step t: K(t+1) and V(t) are published; every wave is done with
    // K(t) and V(t-1), whose buffers (b = (t - tile0) & 1) receive K(t+2) and V(t+1).
    auto top = [&](int t, int b) {
        wait_dma();
        __syncthreads();
        if (t + 2 < tile1) issue_k(t + 2, kbuf(b));
        if (t + 1 < tile1) issue_v(t + 1, vbuf(b ^ 1));
        maybe_rescale<HD, QB>(st, mx);
    };
    // Steps whose next tile is full, two per iteration: t - tile0 is even at
    // the first, so the buffer indices are constants (their LDS offsets fold
    // into the fragment reads' immediates).
    const int main_end = tile1 - 1 - (last_partial ? 1 : 0);
    int t = tile0;
    for (; t + 1 < main_end; t += 2) {
        top(t, 0);
        tile_step<HD, QB, true, false, kPin>(kbuf(1), vbuf(0), fa, qf, sa, sb, st, a.scale_log2, kTileN, mx);
        top(t + 1, 1);
        tile_step<HD, QB, true, false, kPin>(kbuf(0), vbuf(1), fa, qf, sb, sa, st, a.scale_log2, kTileN, mx);
    }
    if (t < main_end) {
        top(t, (t - tile0) & 1);
        tile_step<HD, QB, true, false, kPin>(kbuf((t + 1 - tile0) & 1), vbuf((t - tile0) & 1), fa, qf, sa, sb,
                                       st, a.scale_log2, kTileN, mx);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) sa[qb][kb] = sb[qb][kb];
        ++t;
    }
    if (t + 1 < tile1) {   // the next tile is the partial last one
        top(t, (t - tile0) & 1);
        tile_step<HD, QB, true, true, kPin>(kbuf((t + 1 - tile0) & 1), vbuf((t - tile0) & 1), fa, qf, sa, sb,
                                      st, a.scale_log2, last_valid, mx);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) sa[qb][kb] = sb[qb][kb];
        ++t;
    }
    top(t, (t - tile0) & 1);
    tile_step<HD, QB, false, false, kPin>(nullptr, vbuf((t - tile0) & 1), fa, qf, sa, sb, st, a.scale_log2, kTileN,
                                    mx);

#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const float l_tot = st.l_run[qb] + __shfl_xor(st.l_run[qb], 32);
        const int64_t qrow = qrow0 + 32 * qb;
        if (qrow >= a.n_q) continue;
        if (a.splits == 1) {
            store_o<HD>(a.o + qrow * rstride + head * HD, st.o[qb], __builtin_ldexpf(1.f / l_tot, -ve));
            // log-sum-exp of the scaled logits, natural log: the reference
            // maximum and the running sum are in the exp2 domain
            if (a.lse && hh == 0) a.lse[(int64_t)head * a.n_q + qrow] = (st.m_run[qb] + log2f(l_tot)) * kLn2;
        } else {
            const int64_t prow = ((int64_t)split * a.heads + head) * a.n_q_pad + qrow;
            store_o<HD>(a.part_o + prow * HD, st.o[qb], __builtin_ldexpf(1.f, -ve));
            if (hh == 0) *reinterpret_cast<float2*>(a.part_ml + prow * 2) = make_float2(st.m_run[qb], l_tot);
        }
    }
}

template <int HD, int QB, int NW>
__global__ __launch_bounds__(NW * kWave, 8 / NW) void attn_bf16_kernel(AttnArgs a) {
    attn_bf16_body<HD, QB, NW, false>(a, nullptr);
}

template <int HD, int QB, int NW>
__global__ __launch_bounds__(NW * kWave, 8 / NW) void attn_bf16_rope_kernel(AttnArgs a, RopeFused r) {
    attn_bf16_body<HD, QB, NW, true>(a, &r);
}

// Merge split partials: O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s.
template <int HD>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a) {
    const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    constexpr int C4 = HD / 4;
    const int64_t total = a.n_q * a.heads * C4;
    if (g >= total) return;
    const int c4 = (int)(g % C4);
    const int64_t qh = g / C4;
    const int head = (int)(qh % a.heads);
    const int64_t q = qh / a.heads;
    float M = -__builtin_inff();
    for (int s = 0; s < a.splits; ++s)
        M = fmaxf(M, a.part_ml[(((int64_t)s * a.heads + head) * a.n_q_pad + q) * 2]);
    float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
    float den = 0.f;
    for (int s = 0; s < a.splits; ++s) {
        const int64_t prow = ((int64_t)s * a.heads + head) * a.n_q_pad + q;
        const float2 ml = *reinterpret_cast<const float2*>(a.part_ml + prow * 2);
        const float w = __builtin_amdgcn_exp2f(ml.x - M);
        const float4 x = *reinterpret_cast<const float4*>(a.part_o + prow * HD + c4 * 4);
        num.x += w * x.x, num.y += w * x.y, num.z += w * x.z, num.w += w * x.w;
        den += w * ml.y;
    }
    const float inv = 1.f / den;
    *reinterpret_cast<float4*>(a.o + (q * a.heads + head) * HD + c4 * 4) =
        make_float4(num.x * inv, num.y * inv, num.z * inv, num.w * inv);
    if (a.lse && c4 == 0) a.lse[(int64_t)head * a.n_q + q] = (M + log2f(den)) * kLn2;
}

// fp32 path: one lane per (query, head), keys walked in order with an online
// softmax in fp32.  Meant for small problems (the fp32 parity workload).
template <int HD>
__global__ __launch_bounds__(64) void attn_fp32_kernel(const float* __restrict__ q, int64_t n_q,
                                                       const float* __restrict__ k,
                                                       const float* __restrict__ v, int64_t n_kv,
                                                       int heads, float scale, float* __restrict__ o,
                                                       float* __restrict__ lse) {
    const int head = blockIdx.y;
    const int64_t qi = (int64_t)blockIdx.x * 64 + threadIdx.x;
    if (qi >= n_q) return;
    const int64_t rs = (int64_t)heads * HD;
    float qv[HD], acc[HD];
#pragma unroll
    for (int d = 0; d < HD; ++d) {
        qv[d] = q[qi * rs + head * HD + d];
        acc[d] = 0.f;
    }
    float mr = -__builtin_inff(), l = 0.f;
    for (int64_t j = 0; j < n_kv; ++j) {
        const float* kr = k + j * rs + head * HD;
        const float* vr = v + j * rs + head * HD;
        float sdot = 0.f;
#pragma unroll
        for (int d = 0; d < HD; ++d) sdot = fmaf(qv[d], kr[d], sdot);
        const float x = sdot * scale;
        const float mn = fmaxf(mr, x);
        const float al = expf(mr - mn);
        const float p = expf(x - mn);
        l = l * al + p;
#pragma unroll
        for (int d = 0; d < HD; ++d) acc[d] = fmaf(p, vr[d], acc[d] * al);
        mr = mn;
    }
    const float inv = 1.f / l;
#pragma unroll
    for (int d = 0; d < HD; ++d) o[qi * rs + head * HD + d] = acc[d] * inv;
    if (lse) lse[(int64_t)head * n_q + qi] = mr + logf(l);
}

}  // namespace

hipError_t launch_v_absmax(const __bf16* v, int64_t n, int heads, int hd, uint32_t* vmax, hipStream_t s) {
    dim3 grid((unsigned)kVmaxParts, (unsigned)heads);
    if (hd == 128)
        hipLaunchKernelGGL(v_absmax_kernel<128>, grid, dim3(256), 0, s, v, n, heads, vmax);
    else
        hipLaunchKernelGGL(v_absmax_kernel<64>, grid, dim3(256), 0, s, v, n, heads, vmax);
    return hipGetLastError();
}

hipError_t launch_vt_dense(const __bf16* v, int64_t n_kv, int64_t n_pad, int heads, int hd,
                           const uint32_t* vmax, _Float16* vt, hipStream_t s) {
    dim3 grid((unsigned)(n_pad / kTileN), (unsigned)heads);
    if (hd == 128)
        hipLaunchKernelGGL(vt_dense_kernel<128>, grid, dim3(256), 0, s, v, n_kv, n_pad, heads, vmax, vt);
    else
        hipLaunchKernelGGL(vt_dense_kernel<64>, grid, dim3(256), 0, s, v, n_kv, n_pad, heads, vmax, vt);
    return hipGetLastError();
}

hipError_t launch_attn_bf16(const AttnArgs& a, int hd, hipStream_t s) {
    const int total = a.q_tiles * a.heads * a.splits;
    const unsigned blocks = (unsigned)(((total + 7) / 8) * 8);
    constexpr int QB = kDenseQB, NW = dense_threads(QB) / kWave, NS = kShortQ / 32;
    if (a.q_tile == kShortQ) {
        // two workgroups per CU: kShortQ queries each
        if (hd == 128)
            hipLaunchKernelGGL((attn_bf16_kernel<128, 1, NS>), dim3(blocks), dim3(NS * kWave), 0, s, a);
        else
            hipLaunchKernelGGL((attn_bf16_kernel<64, 1, NS>), dim3(blocks), dim3(NS * kWave), 0, s, a);
    } else if (hd == 128) {
        hipLaunchKernelGGL((attn_bf16_kernel<128, QB, NW>), dim3(blocks), dim3(dense_threads(QB)), 0, s, a);
    } else {
        hipLaunchKernelGGL((attn_bf16_kernel<64, QB, NW>), dim3(blocks), dim3(dense_threads(QB)), 0, s, a);
    }
    return hipGetLastError();
}

hipError_t launch_vt_dense_rope(const __bf16* v, int64_t n_kv, int64_t n_pad, int heads, int hd,
                                const uint32_t* vmax, _Float16* vt, const RopeFused& r, hipStream_t s) {
    dim3 grid((unsigned)(n_pad / kTileN), (unsigned)heads);
    if (hd == 128)
        hipLaunchKernelGGL(vt_dense_rope_kernel<128>, grid, dim3(256), 0, s, v, n_kv, n_pad, heads, vmax, vt, r);
    else
        hipLaunchKernelGGL(vt_dense_rope_kernel<64>, grid, dim3(256), 0, s, v, n_kv, n_pad, heads, vmax, vt, r);
    return hipGetLastError();
}

hipError_t launch_attn_bf16_rope(const AttnArgs& a, int hd, const RopeFused& r, hipStream_t s) {
    const int total = a.q_tiles * a.heads * a.splits;
    const unsigned blocks = (unsigned)(((total + 7) / 8) * 8);
    constexpr int QB = kDenseQB, NW = dense_threads(QB) / kWave, NS = kShortQ / 32;
    if (a.q_tile == kShortQ) {
        if (hd == 128)
            hipLaunchKernelGGL((attn_bf16_rope_kernel<128, 1, NS>), dim3(blocks), dim3(NS * kWave), 0, s, a, r);
        else
            hipLaunchKernelGGL((attn_bf16_rope_kernel<64, 1, NS>), dim3(blocks), dim3(NS * kWave), 0, s, a, r);
    } else if (hd == 128) {
        hipLaunchKernelGGL((attn_bf16_rope_kernel<128, QB, NW>), dim3(blocks), dim3(dense_threads(QB)), 0, s, a, r);
    } else {
        hipLaunchKernelGGL((attn_bf16_rope_kernel<64, QB, NW>), dim3(blocks), dim3(dense_threads(QB)), 0, s, a, r);
    }
    return hipGetLastError();
}

hipError_t launch_attn_combine(const AttnArgs& a, int hd, hipStream_t s) {
    const int64_t total = a.n_q * a.heads * (hd / 4);
    const unsigned blocks = (unsigned)((total + 255) / 256);
    if (hd == 128)
        hipLaunchKernelGGL(attn_combine_kernel<128>, dim3(blocks), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL(attn_combine_kernel<64>, dim3(blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_attn_fp32(const float* q, int64_t n_q, const float* k, const float* v,
                            int64_t n_kv, int heads, int hd, float scale, float* o, float* lse,
                            hipStream_t s) {
    dim3 grid((unsigned)((n_q + 63) / 64), (unsigned)heads);
    if (hd == 128)
        hipLaunchKernelGGL(attn_fp32_kernel<128>, grid, dim3(64), 0, s, q, n_q, k, v, n_kv, heads,
                           scale, o, lse);
    else
        hipLaunchKernelGGL(attn_fp32_kernel<64>, grid, dim3(64), 0, s, q, n_q, k, v, n_kv, heads,
                           scale, o, lse);
    return hipGetLastError();
}

}  // namespace mmdit
