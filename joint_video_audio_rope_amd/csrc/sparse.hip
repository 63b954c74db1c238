// Block-sparse video self-attention (Prism page, xyznot.com 2610.05416:
// "Ideas clave" macro-zones and hybrid top-k/top-p; "Metodo" section 3).
//
// Kernels, in launch order:
//   block_pool     fp64 means of each block's 64 query rows and 64 key rows,
//                  per head (HBM-bound: reads Q and K once); also records each
//                  block's first raster token.
//   vt_blocks      V of each block transposed to fp16 [d][64] for the P V^T
//                  matrix-core product (HBM-bound).
//   block_scores   fp64 logits Qbar Kbar^T * scale per head (fp64 FMA GEMM).
//   block_select   per (head, query block): fp64 softmax, sort by probability
//                  (ties to the lower block id), fp64 running sum, keep the
//                  longer of the top-k and top-p prefixes; emits the bitmask,
//                  the count and the selection bitmask.
//   sparse_attn    attention of each query block over its selected key blocks
//                  with the same online-softmax tile loop as the dense kernel.
// Selection runs in fp64 throughout: on smooth-field inputs the probability
// gaps and running-sum margins at the cut get down to ~1e-8, where fp32 flips
// rows.
#include <algorithm>

#include "attn_core.hpp"

namespace mmdit {

namespace {

// Offset of local token r (raster inside the block) from the block's first token.
__device__ __forceinline__ int64_t block_local(const SparseGeom& g, int r) {
    const int a = r / (g.BH * g.BW);
    const int rr = r - a * (g.BH * g.BW);
    const int b = rr / g.BW;
    const int c = rr - b * g.BW;
    return ((int64_t)a * g.H + b) * g.W + c;
}

// One workgroup per block: thread -> 8 consecutive channels of heads*hd.
// Sums of 64 bf16 values in fp64 are exact for any realistic spread of
// exponents, so the means do not depend on the summation order.
template <int HD>
__global__ __launch_bounds__(512) void block_pool_kernel(SparseGeom g, const __bf16* __restrict__ q,
                                                         const __bf16* __restrict__ k,
                                                         SparseWs w) {
    const int j = blockIdx.x;
    const int64_t base = block_token(g, j, 0);
    if (threadIdx.x == 0) w.base[j] = (int32_t)base;
    const int ncg = g.heads * HD / 8;
    const int64_t rs = (int64_t)g.heads * HD;
    const int vol = g.BT * g.BH * g.BW;
    for (int cg = threadIdx.x; cg < ncg; cg += blockDim.x) {
        double sq[8], sk[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) sq[i] = sk[i] = 0.0;
        for (int a = 0; a < g.BT; ++a)
            for (int b = 0; b < g.BH; ++b) {
                const int64_t row = base + ((int64_t)a * g.H + b) * g.W;
                for (int c = 0; c < g.BW; ++c) {
                    const int64_t tok = row + c;
                    const bf16x8 x = load_bf16x8(q + tok * rs + cg * 8, true);
                    const bf16x8 y = load_bf16x8(k + tok * rs + cg * 8, true);
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        sq[i] += (double)(float)x[i];
                        sk[i] += (double)(float)y[i];
                    }
                }
            }
        const int head = cg * 8 / HD, d = cg * 8 % HD;
        const int64_t o = ((int64_t)head * g.nb + j) * HD + d;
        const double inv = 1.0 / vol;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            w.qbar[o + i] = sq[i] * inv;
            w.kbar[o + i] = sk[i] * inv;
        }
    }
}

// One workgroup per (block, head): gather 64 rows of V, write fp16 [d][64].
template <int HD>
__global__ __launch_bounds__(256) void vt_blocks_kernel(SparseGeom g, const __bf16* __restrict__ v,
                                                        SparseWs w) {
    __shared__ _Float16 tile[kTileN][HD + 2];
    const int j = blockIdx.x, head = blockIdx.y;
    const int64_t base = block_token(g, j, 0);
    const int64_t rs = (int64_t)g.heads * HD;
    constexpr int CPR = HD / 8;
    for (int u = threadIdx.x; u < kTileN * CPR; u += 256) {
        const int r = u / CPR, c = u % CPR;
        const int64_t tok = base + block_local(g, r);
        const bf16x8 x = load_bf16x8(v + tok * rs + head * HD + c * 8, true);
#pragma unroll
        for (int i = 0; i < 8; ++i) tile[r][c * 8 + i] = (_Float16)(float)x[i];
    }
    __syncthreads();
    _Float16* dst = w.vt + ((int64_t)head * g.nb + j) * HD * kTileN;
    for (int u = threadIdx.x; u < HD * (kTileN / 8); u += 256) {
        const int d = u / (kTileN / 8), c = u % (kTileN / 8);
        f16x8 y;
#pragma unroll
        for (int i = 0; i < 8; ++i) y[i] = tile[c * 8 + i][d];
        *reinterpret_cast<f16x8*>(dst + d * kTileN + c * 8) = y;
    }
}

// fp64 GEMM: scores[h][i][j] = scale * <qbar[h][i], kbar[h][j]>.
// 256 threads compute a 128x128 tile, 8x8 per thread; d staged 16 at a time.
constexpr int kSB = 128, kSK = 16;
template <int HD>
__global__ __launch_bounds__(256) void block_scores_kernel(SparseGeom g, double scale, SparseWs w) {
    __shared__ double As[kSK][kSB + 1];
    __shared__ double Bs[kSK][kSB + 1];
    const int head = blockIdx.z;
    const int i0 = blockIdx.y * kSB, j0 = blockIdx.x * kSB;
    const int nb = g.nb;
    const double* A = w.qbar + (int64_t)head * nb * HD;
    const double* B = w.kbar + (int64_t)head * nb * HD;
    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
    double acc[8][8];
#pragma unroll
    for (int a = 0; a < 8; ++a)
#pragma unroll
        for (int b = 0; b < 8; ++b) acc[a][b] = 0.0;
    for (int d0 = 0; d0 < HD; d0 += kSK) {
        for (int u = threadIdx.x; u < kSB * kSK; u += 256) {
            const int r = u / kSK, c = u % kSK;
            As[c][r] = (i0 + r < nb) ? A[(int64_t)(i0 + r) * HD + d0 + c] : 0.0;
            Bs[c][r] = (j0 + r < nb) ? B[(int64_t)(j0 + r) * HD + d0 + c] : 0.0;
        }
        __syncthreads();
#pragma unroll
        for (int c = 0; c < kSK; ++c) {
            double av[8], bv[8];
#pragma unroll
            for (int a = 0; a < 8; ++a) av[a] = As[c][ty + 16 * a];
#pragma unroll
            for (int b = 0; b < 8; ++b) bv[b] = Bs[c][tx + 16 * b];
#pragma unroll
            for (int a = 0; a < 8; ++a)
#pragma unroll
                for (int b = 0; b < 8; ++b) acc[a][b] = fma(av[a], bv[b], acc[a][b]);
        }
        __syncthreads();
    }
    double* S = w.scores + (int64_t)head * nb * nb;
#pragma unroll
    for (int a = 0; a < 8; ++a) {
        const int i = i0 + ty + 16 * a;
        if (i >= nb) continue;
#pragma unroll
        for (int b = 0; b < 8; ++b) {
            const int j = j0 + tx + 16 * b;
            if (j < nb) S[(int64_t)i * nb + j] = acc[a][b] * scale;
        }
    }
}

constexpr int kSelThreads = 256;
constexpr int kSelMax = 4096;   // largest sortable row (power of two)

__device__ __forceinline__ double block_reduce_max(double x, double* red) {
    for (int o = 32; o > 0; o >>= 1) x = fmax(x, __shfl_xor(x, o));
    const int wv = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[wv] = x;
    __syncthreads();
    double r = red[0];
    for (int i = 1; i < kSelThreads / 64; ++i) r = fmax(r, red[i]);
    return r;
}

__device__ __forceinline__ double block_reduce_sum(double x, double* red) {
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
    const int wv = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[wv] = x;
    __syncthreads();
    double r = red[0];
    for (int i = 1; i < kSelThreads / 64; ++i) r += red[i];
    return r;
}

// a goes before b: larger probability first, equal probabilities by lower id.
__device__ __forceinline__ bool sel_before(double pa, int ja, double pb, int jb) {
    return pa > pb || (pa == pb && ja < jb);
}

__global__ __launch_bounds__(kSelThreads) void block_select_kernel(SparseGeom g, int top_k,
                                                                   double top_p, SparseWs w,
                                                                   uint32_t* __restrict__ sel_mask,
                                                                   int32_t* __restrict__ sel_count) {
    __shared__ double P[kSelMax];
    __shared__ uint16_t id[kSelMax];
    __shared__ double red[kSelThreads / 64];
    __shared__ double wsum[kSelThreads];
    __shared__ uint32_t words[kSelMax / 32];
    __shared__ int first_hit;

    const int nb = g.nb;
    const int row = blockIdx.x;                 // head * nb + i
    const double* L = w.scores + (int64_t)row * nb;
    int ns = 1;
    while (ns < nb) ns <<= 1;
    const int tid = threadIdx.x;

    // softmax over the row, fp64
    double mx = -__builtin_inf();
    for (int j = tid; j < nb; j += kSelThreads) mx = fmax(mx, L[j]);
    mx = block_reduce_max(mx, red);
    double se = 0.0;
    for (int j = tid; j < nb; j += kSelThreads) {
        const double e = exp(L[j] - mx);
        P[j] = e;
        se += e;
    }
    se = block_reduce_sum(se, red);
    for (int j = tid; j < ns; j += kSelThreads) {
        if (j < nb) {
            P[j] = P[j] / se;
            id[j] = (uint16_t)j;
        } else {
            P[j] = -1.0;
            id[j] = 0xffff;
        }
    }
    for (int wd = tid; wd < kSelMax / 32; wd += kSelThreads) words[wd] = 0u;
    if (tid == 0) first_hit = nb;
    __syncthreads();

    // bitonic sort, "before" order first
    for (int size = 2; size <= ns; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int t = tid; t < (ns >> 1); t += kSelThreads) {
                const int lo = 2 * t - (t & (stride - 1));
                const int hi = lo + stride;
                const bool up = (lo & size) == 0;
                const double pl = P[lo], ph = P[hi];
                const int jl = id[lo], jh = id[hi];
                const bool swap = up ? sel_before(ph, jh, pl, jl) : sel_before(pl, jl, ph, jh);
                if (swap) {
                    P[lo] = ph, P[hi] = pl;
                    id[lo] = (uint16_t)jh, id[hi] = (uint16_t)jl;
                }
            }
            __syncthreads();
        }
    }

    // running sum in sorted order: each thread owns a contiguous run
    int n_p = nb;
    if (top_p < 1.0) {
        const int per = ns / kSelThreads > 0 ? ns / kSelThreads : 1;
        const int r0 = tid * per;
        double part = 0.0;
        for (int r = r0; r < r0 + per && r < nb; ++r) part += P[r];
        wsum[tid] = part;
        __syncthreads();
        // exclusive prefix of the per-thread parts (sequential per thread: 256 adds)
        double pre = 0.0;
        for (int t = 0; t < tid; ++t) pre += wsum[t];
        double run = pre;
        for (int r = r0; r < r0 + per && r < nb; ++r) {
            run += P[r];
            if (run >= top_p) {
                atomicMin(&first_hit, r);
                break;
            }
        }
        __syncthreads();
        n_p = first_hit < nb ? first_hit + 1 : nb;
    }
    const int kk = top_k < nb ? top_k : nb;
    const int K = kk > n_p ? kk : n_p;

    for (int r = tid; r < K; r += kSelThreads) {
        const int j = id[r];
        atomicOr(&words[j >> 5], 1u << (j & 31));
    }
    __syncthreads();

    const int nw = (nb + 31) >> 5;
    if (tid == 0) {
        int acc = 0;
        for (int wd = 0; wd < nw; ++wd) acc += __popc(words[wd]);
        w.count[row] = acc;
        if (sel_count) sel_count[row] = acc;
    }
    for (int wd = tid; wd < nw; wd += kSelThreads) {
        w.mask[(int64_t)row * nw + wd] = words[wd];
        if (sel_mask) sel_mask[(int64_t)row * nw + wd] = words[wd];
    }
}

// Sparse attention.  A workgroup of 4 waves serves two query blocks of one
// head, 2p and 2p + 1 (neighbours along w inside a zone, whose selections
// largely coincide): waves 0-1 own block 2p, waves 2-3 block 2p + 1.  The
// workgroup walks the union of the two selections in ascending block id,
// staging each key block's K rows (gathered from the raster layout) and its
// fp16 V^T block in double-buffered LDS; a wave pair computes a tile only if
// its own block selected it.  Sharing a staged tile between two blocks cuts
// the gather traffic (the kernel is bound by it: a head's K and V^T are
// 88 MB, far beyond L2) at the price of idle waves on tiles only one block
// selected.  Dispatch keeps all XCDs on one head at a time (its K/V^T stay
// in the last-level cache) and gives each XCD a contiguous eighth of that
// head's blocks (spatial neighbours, similar selections).
template <int HD>
__global__ __launch_bounds__(256, 2) void sparse_attn_kernel(SparseGeom g, const __bf16* __restrict__ q,
                                                             const __bf16* __restrict__ k,
                                                             float scale_log2, SparseWs w,
                                                             float* __restrict__ o) {
    using L = TileLayout<HD>;
    constexpr int NW = 4;
    constexpr int KS = HD / 16;
    constexpr int KCH = kTileN * L::kKChunks / (kWave * NW);
    constexpr int VCH = HD * 8 / (kWave * NW);
    __shared__ __attribute__((aligned(16))) char lds[2 * L::kBytes];
    __shared__ uint32_t msk[2][kSelMax / 32];

    const int pairs = (g.nb + 1) >> 1;
    const int per = (pairs + 7) >> 3;
    const int slot = (int)(blockIdx.x >> 3);
    const int head = slot / per;
    const int pr = (int)(blockIdx.x & 7) * per + (slot - head * per);
    if (head >= g.heads || pr >= pairs) return;
    const int nw = (g.nb + 31) >> 5;
    const bool has_b = 2 * pr + 1 < g.nb;

    const uint32_t* mrow = w.mask + ((int64_t)head * g.nb + 2 * pr) * nw;
    for (int i = threadIdx.x; i < 2 * nw; i += 256) {
        const int sd = i / nw, wd = i - (i / nw) * nw;
        msk[sd][wd] = (sd == 0 || has_b) ? mrow[sd * nw + wd] : 0u;
    }

    const int wv = wave_id();
    const int side = wv >> 1;
    const int lane = threadIdx.x & 63;
    const int hh = lane >> 5;
    const int m = lane & 31;
    const int qb = min(2 * pr + side, g.nb - 1);
    const int64_t rstride = (int64_t)g.heads * HD;
    const int64_t krb = rstride * 2;

    const int64_t qtok = (int64_t)w.base[qb] + block_local(g, (wv & 1) * 32 + m);
    bf16x8 qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        qf[ks] = load_bf16x8(q + qtok * rstride + head * HD + 16 * ks + 8 * hh, true);

    uint32_t kbyte[KCH];   // < 2^32: checked on the host (block span * row bytes)
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
        int row, c;
        L::k_at((wv * KCH + i) * kWave + lane, row, c);
        kbyte[i] = (uint32_t)(block_local(g, (row & ~31) | perm_row(row & 31)) * krb + c * 16);
    }
    uint32_t voff[VCH];
#pragma unroll
    for (int i = 0; i < VCH; ++i) {
        int d, c;
        L::v_at((wv * VCH + i) * kWave + lane, d, c);
        voff[i] = (uint32_t)((d * kTileN + c * 8) * 2);
    }

    auto issue = [&](int j, char* lb) {
        const int64_t base = w.base[j];
        const char* kt = reinterpret_cast<const char*>(k + base * rstride + head * HD);
#pragma unroll
        for (int i = 0; i < KCH; ++i) dma16(kt + kbyte[i], lb + (wv * KCH + i) * 1024);
        const char* vt = reinterpret_cast<const char*>(w.vt + ((int64_t)head * g.nb + j) * HD * kTileN);
#pragma unroll
        for (int i = 0; i < VCH; ++i) dma16(vt + voff[i], lb + L::kKBytes + (wv * VCH + i) * 1024);
    };
    __syncthreads();

    // cursor over the union of both selections (uniform across the workgroup)
    int word = 0;
    uint32_t bits = __builtin_amdgcn_readfirstlane(msk[0][0] | msk[1][0]);
    auto advance = [&]() -> int {
        while (bits == 0u) {
            if (++word >= nw) return -1;
            bits = __builtin_amdgcn_readfirstlane(msk[0][word] | msk[1][word]);
        }
        const int b = __builtin_ctz(bits);
        bits &= bits - 1u;
        return word * 32 + b;
    };

    FragAddr<HD> fa;
    fa.init();
    f32x16 sc[2], sd[2];
    SoftmaxState<HD> st;
    st.init();
    int jc = advance();
    if (jc >= 0) issue(jc, lds);
    for (int it = 0; jc >= 0; ++it) {
        char* cur = lds + (it & 1) * L::kBytes;
        wait_dma();
        __syncthreads();
        const int jn = advance();
        if (jn >= 0) issue(jn, lds + ((it + 1) & 1) * L::kBytes);
        if ((msk[side][jc >> 5] >> (jc & 31)) & 1u) {
            qk_tile<HD>(cur, fa, qf, sc);
            maybe_rescale<HD>(st, tile_max<false>(sc, scale_log2, kTileN));
            tile_step<HD, false, false>(nullptr, cur + L::kKBytes, fa, qf, sc, sd, st, scale_log2, kTileN);
        }
        jc = jn;
    }

    if (2 * pr + side >= g.nb) return;
    const float l_tot = st.l_run + __shfl_xor(st.l_run, 32);
    store_o<HD>(o + qtok * rstride + head * HD, st, 1.f / l_tot);
}

}  // namespace

hipError_t launch_block_pool(const SparseGeom& g, const __bf16* q, const __bf16* k, int hd,
                             const SparseWs& w, hipStream_t s) {
    const int ncg = g.heads * 128 / 8;
    const int threads = std::min(512, (ncg + 63) / 64 * 64);
    hipLaunchKernelGGL(block_pool_kernel<128>, dim3(g.nb), dim3(threads), 0, s, g, q, k, w);
    (void)hd;
    return hipGetLastError();
}

hipError_t launch_vt_blocks(const SparseGeom& g, const __bf16* v, int hd, const SparseWs& w,
                            hipStream_t s) {
    hipLaunchKernelGGL(vt_blocks_kernel<128>, dim3(g.nb, g.heads), dim3(256), 0, s, g, v, w);
    (void)hd;
    return hipGetLastError();
}

hipError_t launch_block_scores(const SparseGeom& g, int hd, double scale, const SparseWs& w,
                               hipStream_t s) {
    const unsigned nt = (unsigned)((g.nb + kSB - 1) / kSB);
    hipLaunchKernelGGL(block_scores_kernel<128>, dim3(nt, nt, g.heads), dim3(256), 0, s, g, scale,
                       w);
    (void)hd;
    return hipGetLastError();
}

hipError_t launch_block_select(const SparseGeom& g, int top_k, double top_p, const SparseWs& w,
                               uint32_t* sel_mask, int32_t* sel_count, hipStream_t s) {
    hipLaunchKernelGGL(block_select_kernel, dim3(g.heads * g.nb), dim3(kSelThreads), 0, s, g, top_k,
                       top_p, w, sel_mask, sel_count);
    return hipGetLastError();
}

hipError_t launch_sparse_attn(const SparseGeom& g, const __bf16* q, const __bf16* k, int hd,
                              float scale_log2, const SparseWs& w, float* o, hipStream_t s) {
    const unsigned blocks = (unsigned)(8 * ((((g.nb + 1) / 2) + 7) / 8) * g.heads);
    hipLaunchKernelGGL(sparse_attn_kernel<128>, dim3(blocks), dim3(256), 0, s, g, q, k, scale_log2,
                       w, o);
    (void)hd;
    return hipGetLastError();
}

}  // namespace mmdit
