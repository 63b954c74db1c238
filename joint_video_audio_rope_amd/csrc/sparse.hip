// Block-sparse video self-attention (Prism page, xyznot.com 2610.05416:
// "Ideas clave" macro-zones and hybrid top-k/top-p; "Metodo" section 3).
//
// Kernels, in launch order:
//   block_pool     fp64 means of each block's 64 query rows and 64 key rows,
//                  per head (HBM-bound: reads Q and K once); also records each
//                  block's first raster token.
//   vt_blocks      each block's K rows (bf16) and V^T (fp16 [d][64]), each
//                  laid out as the image of its LDS tile (HBM-bound).
//   block_scores   fp64 logits Qbar Kbar^T * scale per head, on the fp64
//                  matrix cores, in chunks of query-block rows.
//   block_select   per (head, query block): fp64 softmax, then the top-p and
//                  top-k cuts found by bisection over the probabilities' bit
//                  patterns (ties to the lower block id), keeping the longer
//                  prefix; emits the bitmask and the count.
//   group_order    per head, the groups of query blocks ranked by estimated
//                  cost: the next kernel's dispatch order.
//   sparse_attn    attention of groups of query blocks over the union of
//                  their selected key blocks, fed through an LDS ring by
//                  producer waves, in half-tile steps of the dense kernel's
//                  online softmax.
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
// With adaptive blocks the workgroup of a block's first tile pools all of the
// block's tiles (up to 256 rows, still exact) and writes the block mean to
// every tile of the block; the other tiles' workgroups exit.
template <int HD>
__global__ __launch_bounds__(512) void block_pool_kernel(SparseGeom g, const __bf16* __restrict__ q,
                                                         const __bf16* __restrict__ k,
                                                         SparseWs w) {
    const int j = blockIdx.x;
    int ntile = 1;
    if (w.tdim) {
        if (w.lead[j] != j) return;
        while (ntile < 4 && j + ntile < g.nb && w.lead[j + ntile] == j) ++ntile;
    } else if (threadIdx.x == 0) {
        w.base[j] = (int32_t)block_token(g, j, 0);
    }
    const int ncg = g.heads * HD / 8;
    const int64_t rs = (int64_t)g.heads * HD;
    for (int cg = threadIdx.x; cg < ncg; cg += blockDim.x) {
        double sq[8], sk[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) sq[i] = sk[i] = 0.0;
        auto add = [&](int64_t tok) {
            const bf16x8 x = load_bf16x8(q + tok * rs + cg * 8, true);
            const bf16x8 y = load_bf16x8(k + tok * rs + cg * 8, true);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                sq[i] += (double)(float)x[i];
                sk[i] += (double)(float)y[i];
            }
        };
        if (w.tdim) {
            for (int u = 0; u < ntile; ++u) {
                const int64_t base = w.base[j + u];
                const uint32_t code = w.tdim[j + u];
                for (int r = 0; r < kTileN; ++r) add(base + tile_local(g, code, r));
            }
        } else {
            const int64_t base = block_token(g, j, 0);
            for (int a = 0; a < g.BT; ++a)
                for (int b = 0; b < g.BH; ++b) {
                    const int64_t row = base + ((int64_t)a * g.H + b) * g.W;
                    for (int c = 0; c < g.BW; ++c) add(row + c);
                }
        }
        const int head = cg * 8 / HD, d = cg * 8 % HD;
        const double inv = 1.0 / (kTileN * ntile);
        for (int u = 0; u < ntile; ++u) {
            const int64_t o = ((int64_t)head * g.nb + j + u) * HD + d;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                w.qbar[o + i] = sq[i] * inv;
                w.kbar[o + i] = sk[i] * inv;
            }
        }
    }
}

// LDS image of one staged key block for the sparse attention kernel: K (64
// rows x HD bf16) and then V^T (HD rows x 64 keys fp16), 16-byte chunks.  A
// wave reads 32 rows x 16 bytes per fragment: lane (m, hh) reads chunk hh of
// a 32-byte pair in row m.  Each pair of chunks of a row is stored
// contiguously, row after row, one 2 KB (K) or 4 KB (V^T) panel per pair;
// rows 8..15 of every 16 swap the two chunks of their pair, so the 16 lanes
// served together (16 rows, one chunk each) hit 16 different 16-byte slots of
// a 256-byte line.  Every fragment of a lane then sits at one per-lane offset
// plus a constant: no per-fragment address registers.
//   K chunk (row r, d chunk c):   (c >> 1) * 2048 + r * 32 + ((c & 1) ^ ((r >> 3) & 1)) * 16
//   V^T chunk (row d, key chunk c): kKBytes + (c >> 1) * 4096 + d * 32 + ((c & 1) ^ ((d >> 3) & 1)) * 16
template <int HD>
struct StreamTile {
    static constexpr int kKBytes = kTileN * HD * 2;
    static constexpr int kVBytes = HD * kTileN * 2;
    static constexpr int kBytes = kKBytes + kVBytes;
    static constexpr int kKPanel = kTileN * 32;    // one d-chunk pair of all 64 K rows
    static constexpr int kVPanel = HD * 32;        // one key-chunk pair of all HD V^T rows
    // inverse maps: which (row, chunk) a 16-byte chunk index u of the K or V^T part holds
    __host__ __device__ static void k_at(int u, int& row, int& c) {
        row = (u % (kKPanel / 16)) >> 1;
        c = 2 * (u / (kKPanel / 16)) + ((u & 1) ^ ((row >> 3) & 1));
    }
    __host__ __device__ static void v_at(int u, int& d, int& c) {
        d = (u % (kVPanel / 16)) >> 1;
        c = 2 * (u / (kVPanel / 16)) + ((u & 1) ^ ((d >> 3) & 1));
    }
    // lane (m, hh)'s offset inside a panel; fragment (step ks, key half kb)
    // of K and (row block db, key group gq) of V^T add constants to it
    __device__ static int lane_offset() {
        const int lane = threadIdx.x & 63, m = lane & 31, hh = lane >> 5;
        return m * 32 + ((hh ^ ((m >> 3) & 1)) << 4);
    }
    __device__ static bf16x8 k_frag(const char* tile, int lo, int ks, int kb) {
        return *reinterpret_cast<const bf16x8*>(tile + lo + ks * kKPanel + kb * 32 * 32);
    }
    __device__ static f16x8 v_frag(const char* tile, int lo, int db, int gq) {
        return *reinterpret_cast<const f16x8*>(tile + kKBytes + lo + gq * kVPanel + db * 32 * 32);
    }
};

// One workgroup per (block, head): gather the block's 64 rows of K and of V
// and write each as the exact image of its LDS tile (K rows in the MFMA row
// order, V transposed to fp16 [d][64] with the head's prescale 2^e applied,
// 16-byte chunks swizzled), so that the
// attention kernel stages a tile with two contiguous 16 KB copies instead of
// 64 scattered 256-byte rows.
template <int HD>
__global__ __launch_bounds__(256) void vt_blocks_kernel(SparseGeom g, const __bf16* __restrict__ k,
                                                        const __bf16* __restrict__ v, SparseWs w) {
    using L = StreamTile<HD>;
    __shared__ _Float16 tile[kTileN][HD + 2];
    const int j = blockIdx.x, head = blockIdx.y;
    const float sc = __builtin_ldexpf(1.f, v_scale_exp(w.vmax, head));   // the head's V prescale
    const int64_t base = w.tdim ? (int64_t)w.base[j] : block_token(g, j, 0);
    const uint32_t code = w.tdim ? w.tdim[j] : 0u;
    auto local = [&](int r) { return w.tdim ? tile_local(g, code, r) : block_local(g, r); };
    const int64_t rs = (int64_t)g.heads * HD;
    constexpr int CPR = HD / 8;
    for (int u = threadIdx.x; u < kTileN * CPR; u += 256) {
        const int r = u / CPR, c = u % CPR;
        const int64_t tok = base + local(r);
        const bf16x8 x = load_bf16x8(v + tok * rs + head * HD + c * 8, true);
#pragma unroll
        for (int i = 0; i < 8; ++i) tile[r][c * 8 + i] = (_Float16)((float)x[i] * sc);
    }
    // K image: LDS chunk index u holds (row, chunk) = k_at(u) of the tile,
    // row counted after the MFMA row permutation of each 32-row half
    __bf16* kdst = w.kimg + ((int64_t)head * g.nb + j) * (kTileN * HD);
    for (int u = threadIdx.x; u < kTileN * CPR; u += 256) {
        int row, c;
        L::k_at(u, row, c);
        const int64_t tok = base + local((row & ~31) | perm_row(row & 31));
        *reinterpret_cast<bf16x8*>(kdst + u * 8) = load_bf16x8(k + tok * rs + head * HD + c * 8, true);
    }
    __syncthreads();
    // V^T image: LDS chunk index u holds keys 8 c .. 8 c + 7 of d row d,
    // (d, c) = v_at(u)
    _Float16* dst = w.vt + ((int64_t)head * g.nb + j) * HD * kTileN;
    for (int u = threadIdx.x; u < HD * (kTileN / 8); u += 256) {
        int d, c;
        L::v_at(u, d, c);
        f16x8 y;
#pragma unroll
        for (int i = 0; i < 8; ++i) y[i] = tile[c * 8 + i][d];
        *reinterpret_cast<f16x8*>(dst + u * 8) = y;
    }
}

// fp64 GEMM for one chunk of query blocks: scores[h][i - row0][j] = scale *
// <qbar[h][i], kbar[h][j]> for i in [row0, row0 + rows), on the fp64 matrix
// cores.  v_mfma_f64_16x16x4_f64 multiplies a 16 x 4 block of A (lane l holds
// row l % 16, column l / 16) by a 4 x 16 block of B (lane l: row l / 16,
// column l % 16) into 16 x 16 sums (lane l: column l % 16, register r: row
// 4 r + l / 16).  A workgroup of four waves computes a 128 x 128 tile, each
// wave 64 x 64 (4 x 4 products per step of 4 along d), reading qbar and kbar
// straight from memory: each 128-byte line of a row serves four consecutive
// steps from L1.  Two workgroups share a CU.  Rows and columns past the chunk
// or the grid read row 0 and are not stored.  On the 24 x 64 x 112 grid: 1.36
// ms per call against 1.81 ms for a vector-FMA kernel with LDS-staged 8 x 8
// register blocks (32 rows x 64 columns per wave: 1.86 ms).
constexpr int kSB = 128;
typedef double f64x4 __attribute__((ext_vector_type(4)));
template <int HD>
__global__ __launch_bounds__(256, 2) void block_scores_kernel(SparseGeom g, double scale, SparseWs w, int row0,
                                                           int rows) {
    const int head = blockIdx.z;
    const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int i0 = row0 + blockIdx.y * kSB + (wv >> 1) * 64, j0 = blockIdx.x * kSB + (wv & 1) * 64;
    const int i_end = row0 + rows;
    const int nb = g.nb;
    const int li = lane & 15, lk = lane >> 4;
    const double* A = w.qbar + (int64_t)head * nb * HD;
    const double* B = w.kbar + (int64_t)head * nb * HD;
    const double* ar[4];
    const double* br[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int i = i0 + 16 * t + li, j = j0 + 16 * t + li;
        ar[t] = A + (int64_t)(i < i_end ? i : 0) * HD + lk;
        br[t] = B + (int64_t)(j < nb ? j : 0) * HD + lk;
    }
    f64x4 acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = (f64x4){0.0, 0.0, 0.0, 0.0};
#pragma unroll 4
    for (int k = 0; k < HD; k += 4) {
        double av[4], bv[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            av[t] = ar[t][k];
            bv[t] = br[t][k];
        }
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < 4; ++b) acc[a][b] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[a], bv[b], acc[a][b], 0, 0, 0);
    }
    double* S = w.scores + (int64_t)head * rows * nb;
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = i0 + 16 * a + 4 * r + lk;
            if (i >= i_end) continue;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const int j = j0 + 16 * b + li;
                if (j < nb) S[(int64_t)(i - row0) * nb + j] = acc[a][b][r] * scale;
            }
        }
}

constexpr int kSelWaves = 4;   // rows (one per wave) per selection workgroup of one-wave rows
// Sparse attention: LDS ring depth (tiles).  The query blocks per workgroup,
// kStreamGroup, are measured where they are declared.
constexpr int kStreamRing = 4;

// Wave-wide reductions.  The xor butterfly combines the same two partial
// results in every lane at every level (addition and max are commutative), so
// every lane ends with the same bits: decisions taken on them are uniform.
__device__ __forceinline__ double wave_sum(double x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
    return x;
}
__device__ __forceinline__ double wave_max(double x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = fmax(x, __shfl_xor(x, o));
    return x;
}

__device__ __forceinline__ double key_value(uint64_t key) { return __longlong_as_double((long long)key); }
__device__ __forceinline__ uint64_t value_key(double x) { return (uint64_t)__double_as_longlong(x); }

// Reductions over the W waves that share one selection row (W == 1: the
// wave alone).  Each wave reduces its lanes, writes its partial to LDS, and
// after a barrier every wave adds the W partials in wave order, so all waves
// hold the same bits and take the same decisions (every barrier is reached by
// all of them).  Slots alternate so one barrier per reduction suffices.
template <int W>
struct RowReduce {
    double* d;    // [2][W]
    int* c;       // [2][W]
    int flip = 0;
    __device__ double sum(double x) {
        x = wave_sum(x);
        if constexpr (W == 1) {
            return x;
        } else {
            if ((threadIdx.x & 63) == 0) d[flip * W + wave_id()] = x;
            __syncthreads();
            double t = 0.0;
#pragma unroll
            for (int k = 0; k < W; ++k) t += d[flip * W + k];
            flip ^= 1;
            return t;
        }
    }
    __device__ double max(double x) {
        x = wave_max(x);
        if constexpr (W == 1) {
            return x;
        } else {
            if ((threadIdx.x & 63) == 0) d[flip * W + wave_id()] = x;
            __syncthreads();
            double t = d[flip * W];
#pragma unroll
            for (int k = 1; k < W; ++k) t = fmax(t, d[flip * W + k]);
            flip ^= 1;
            return t;
        }
    }
    // wave-level count -> row count; with `below`, also the counts of the
    // waves before this one
    __device__ int count(int x, int* below = nullptr) {
        if constexpr (W == 1) {
            if (below) *below = 0;
            return x;
        } else {
            if ((threadIdx.x & 63) == 0) c[flip * W + wave_id()] = x;
            __syncthreads();
            int t = 0, b = 0;
            const int me = wave_id();
#pragma unroll
            for (int k = 0; k < W; ++k) {
                const int v = c[flip * W + k];
                b += k < me ? v : 0;
                t += v;
            }
            flip ^= 1;
            if (below) *below = b;
            return t;
        }
    }
};

// Selection of one row of block probabilities.  W == 1: one wave per row
// (kSelWaves rows per workgroup); W > 1: W waves per row, wave w holding the
// blocks w 64 EM .. (w + 1) 64 EM - 1.  Lane l of a wave holds its range's
// blocks l + 64 r.  The blocks in descending order of probability (equal
// probabilities by ascending id) are never sorted: for a non-negative double
// the bit pattern read as an unsigned integer orders like the value, so the
// row is searched by bisection over that integer range.
//   top-p: the element e at which the descending running sum first reaches p
//          is the largest key x with sum(P >= x) >= p; within a run of equal
//          values the running sum advances one element at a time.
//   top-k: the k-th element is the largest key x with count(P >= x) >= k.
// The selection is the longer of the two prefixes.  Slots past the row hold
// P = -1, which no threshold >= 0 admits.  Rows are the query blocks
// row0 .. row0 + rows - 1 of every head, whose scores hold the chunk.
template <int EM, int W, bool AD>   // EM: elements per lane per wave; AD: adaptive blocks (w.lead set)
__global__ __launch_bounds__(64 * (W == 1 ? kSelWaves : W)) void block_select_kernel(
        SparseGeom g, int top_k, double top_p, SparseWs w, int row0, int rows, uint32_t* __restrict__ sel_mask,
        int32_t* __restrict__ sel_count) {
    __shared__ double red_d[2 * W];
    __shared__ int red_c[2 * W];
    RowReduce<W> R{red_d, red_c};
    const int nb = g.nb;
    const int local = W == 1 ? (int)blockIdx.x * kSelWaves + wave_id() : (int)blockIdx.x;   // head * rows + i - row0
    if (local >= g.heads * rows) return;   // W == 1 only: a whole wave leaves, no barrier is skipped
    const int head = local / rows;
    const int row = head * nb + row0 + (local - head * rows);   // head * nb + i
    const int lane = threadIdx.x & 63;
    const int jbase = W == 1 ? 0 : wave_id() * 64 * EM;        // first block of this wave's range
    const double* L = w.scores + (int64_t)local * nb;

    // Columns that are blocks: every column with uniform blocks; with adaptive
    // blocks only each block's first tile (the other tiles of the block repeat
    // its logit and take its decision at the end).
    uint64_t okm = 0;
    int nv = nb;   // blocks in the row
    if constexpr (AD) {
#pragma unroll
        for (int r = 0; r < EM; ++r) {
            const int j = jbase + lane + 64 * r;
            if (j < nb && w.lead[j] == j) okm |= 1ull << r;
        }
        nv = 0;
#pragma unroll
        for (int r = 0; r < EM; ++r) nv += __popcll(__ballot((okm >> r) & 1ull));
        nv = R.count(nv);
    }
    auto col_ok = [&](int r) { return AD ? ((okm >> r) & 1ull) != 0 : jbase + lane + 64 * r < nb; };

    // softmax over the row's blocks, fp64
    double P[EM];
    double mx = -__builtin_inf();
#pragma unroll
    for (int r = 0; r < EM; ++r) {
        const int j = jbase + lane + 64 * r;
        P[r] = col_ok(r) ? L[j] : -__builtin_inf();
        mx = fmax(mx, P[r]);
    }
    mx = R.max(mx);
    double se = 0.0;
#pragma unroll
    for (int r = 0; r < EM; ++r) {
        if (col_ok(r)) {
            P[r] = exp(P[r] - mx);
            se += P[r];
        }
    }
    se = R.sum(se);
    double tot = 0.0;
#pragma unroll
    for (int r = 0; r < EM; ++r) {
        if (col_ok(r)) {
            P[r] = P[r] / se;
            tot += P[r];
        } else {
            P[r] = -1.0;
        }
    }
    tot = R.sum(tot);

    auto count_ge = [&](double t) {
        int c = 0;
#pragma unroll
        for (int r = 0; r < EM; ++r)
            c += __popcll(__ballot(P[r] >= t));
        return R.count(c);
    };
    auto count_eq = [&](double t) {
        int c = 0;
#pragma unroll
        for (int r = 0; r < EM; ++r)
            c += __popcll(__ballot(P[r] == t));
        return R.count(c);
    };
    auto sum_ge = [&](double t) {
        double x = 0.0;
#pragma unroll
        for (int r = 0; r < EM; ++r)
            if (P[r] >= t) x += P[r];
        return R.sum(x);
    };
    // sum and count of P >= t in one pass (the count from the compare masks)
    auto sum_count_ge = [&](double t, int& cnt) {
        double x = 0.0;
        int c = 0;
#pragma unroll
        for (int r = 0; r < EM; ++r) {
            const bool ge = P[r] >= t;
            c += __popcll(__ballot(ge));
            if (ge) x += P[r];
        }
        cnt = R.count(c);
        return R.sum(x);
    };
    // the one value left in [lo, hi) once the bisection stops
    auto value_in = [&](double lo, double hi) {
        double x = -1.0;
#pragma unroll
        for (int r = 0; r < EM; ++r)
            if (P[r] >= lo && P[r] < hi) x = fmax(x, P[r]);
        return R.max(x);
    };
    const uint64_t kInf = 0x7FF0000000000000ull;   // +inf: above every probability

    // top-p prefix: n_p elements, the last one of value vp, the mp-th of its run
    int n_p = nv;
    double vp = -1.0;
    int mp = 0;
    if (top_p < 1.0 && tot >= top_p) {
        if (top_p <= 0.0) {
            double x = P[0];
#pragma unroll
            for (int r = 1; r < EM; ++r) x = fmax(x, P[r]);
            vp = R.max(x);
            mp = 1;
            n_p = 1;
        } else {
            uint64_t lo = 0, hi = kInf;   // sum(P >= lo) >= p > sum(P >= hi)
            // count(P >= lo) and count(P >= hi): their difference is the
            // number of elements left in [lo, hi)
            int c_lo = nv, c_hi = 0;
            while (hi - lo > 1 && c_lo - c_hi > 1) {
                const uint64_t mid = lo + ((hi - lo) >> 1);
                int c;
                if (sum_count_ge(key_value(mid), c) >= top_p)
                    lo = mid, c_lo = c;
                else
                    hi = mid, c_hi = c;
            }
            vp = value_in(key_value(lo), key_value(hi));
            // within the run of elements equal to vp, in id order
            const uint64_t above = value_key(vp) + 1;
            double acc = sum_ge(key_value(above));
            const int c_above = count_ge(key_value(above));
            const int run = count_eq(vp);
            mp = 1;
            acc += vp;
            while (acc < top_p && mp < run) {
                acc += vp;
                ++mp;
            }
            n_p = c_above + mp;
        }
    }

    // top-k prefix, needed only when it is the longer one (the selection
    // below takes the top-p prefix whenever n_p >= k; every wave of a row
    // holds the same n_p, so all of them skip or run the search together)
    const int kk = top_k < nv ? top_k : nv;
    double vk = -1.0;
    int mk = 0;
    if (kk > 0 && kk < nv && kk > n_p) {
        uint64_t lo = 0, hi = kInf;   // count(P >= lo) >= k > count(P >= hi)
        int c_lo = nv, c_hi = 0;
        while (hi - lo > 1 && c_lo - c_hi > 1) {
            const uint64_t mid = lo + ((hi - lo) >> 1);
            const int c = count_ge(key_value(mid));
            if (c >= kk)
                lo = mid, c_lo = c;
            else
                hi = mid, c_hi = c;
        }
        vk = value_in(key_value(lo), key_value(hi));
        mk = kk - count_ge(key_value(value_key(vk) + 1));
    }

    // the longer prefix: every element above the last value, plus the first
    // m of that value's run in id order (all elements when it covers the row)
    const int K = kk > n_p ? kk : n_p;
    const bool all = K >= nv;
    const double v = kk > n_p ? vk : vp;
    const int mrun = kk > n_p ? mk : mp;
    // run elements (== v) in the waves before this one
    int before = 0;
    if constexpr (W > 1) {
        int c = 0;
#pragma unroll
        for (int r = 0; r < EM; ++r) c += __popcll(__ballot(P[r] >= 0.0 && P[r] == v));
        R.count(c, &before);
    }
    const int nw = (nb + 31) >> 5;
    uint32_t* mrow = w.mask + (int64_t)row * nw;
    uint32_t* srow = sel_mask ? sel_mask + (int64_t)row * nw : nullptr;
    // Adaptive blocks never straddle a zone (8 tiles), so every 64-column word
    // of a wave's range starts a block and a block's tiles share its word.
    uint64_t prev = 0, prev_starts = 0;   // block-start decisions and positions of the previous 64 columns
#pragma unroll
    for (int r = 0; r < EM; ++r) {
        const bool valid = P[r] >= 0.0;
        const uint64_t eq = __ballot(valid && P[r] == v);
        const int rank = before + __popcll(eq & ((1ull << lane) - 1ull));
        before += __popcll(eq);
        const bool sel = valid && (all || P[r] > v || (P[r] == v && rank < mrun));
        uint64_t b = __ballot(sel);
        if constexpr (AD) {
            // A block's later tiles copy the bit of its first tile: the
            // nearest block start at or below the column, in this word of 64
            // columns or, if none, the last one of the previous word.
            const uint64_t starts = __ballot(((okm >> r) & 1ull) != 0);
            const uint64_t upto = starts & (lane == 63 ? ~0ull : ((2ull << lane) - 1ull));
            const bool inh = upto ? ((b >> (63 - __clzll(upto))) & 1ull)
                                  : (prev_starts && ((prev >> (63 - __clzll(prev_starts))) & 1ull));
            prev = b;
            prev_starts = starts;
            b = __ballot(sel || (inh && jbase + lane + 64 * r < nb));
        }
        const int wd = (jbase >> 5) + 2 * r + lane;
        if (lane < 2 && wd < nw) {   // words past the row hold no bits
            const uint32_t word = lane ? (uint32_t)(b >> 32) : (uint32_t)b;
            mrow[wd] = word;
            if (srow) srow[wd] = word;
        }
    }
    if (lane == 0 && (W == 1 || wave_id() == 0)) {
        w.count[row] = K;
        if (sel_count) sel_count[row] = K;
    }
}

// One 32-key half KB of a staged 64-key tile for the wave's 32 queries:
// S^T = K_KB Q^T (8 MFMAs), the online softmax against the reference maximum,
// O^T += V_KB^T P^T (8 MFMAs).  The steps and key order of tile_step (exp2
// against the reference maximum, P and its row sums in fp16, fp32
// accumulation), with the lazy rescale checked per half, on half the
// registers: with 16 waves per workgroup a wave has 128.  lo is the lane's
// StreamTile offset.
//
// Each LDS fragment is read two MFMAs ahead of its use, in two alternating
// registers.  Left to itself the scheduler issued every K fragment read just
// before its MFMA and waited for it (lgkmcnt(0)), so a wave paid the LDS
// latency once per product; with few of a SIMD's waves selecting a tile,
// nothing hid it.  The QK phase's order is therefore pinned with
// sched_group_barrier: on the 24 x 64 x 112 grid the call went from 131.5 to
// 125.6 ms (results bitwise identical).  Three ahead no longer fits: the
// register allocator then spills Q fragments inside the walk.
template <int HD, int KB>
__device__ __forceinline__ void half_tile_step(const char* __restrict__ tile, int lo, const bf16x8 (&qf)[HD / 16],
                                               SoftmaxState<HD, 1>& st, float scale_log2) {
    using L = StreamTile<HD>;
    constexpr int NK = HD / 16;   // MFMA steps over d
    constexpr int PD = 2;         // fragments read ahead
    f32x16 s;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
    bf16x8 kf[PD];
#pragma unroll
    for (int j = 0; j < PD; ++j) kf[j] = L::k_frag(tile, lo, j, KB);
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks % PD], qf[ks], s, 0, 0, 0);
        if (ks + PD < NK) kf[ks % PD] = L::k_frag(tile, lo, ks + PD, KB);
    }
    order_fragment_stream<PD, NK>();
    float x = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) x = fmaxf(x, s[r]);
    const float mx[1] = {pair_max(x) * scale_log2};
    maybe_rescale<HD, 1>(st, mx);
    const float mneg = -st.m_run[0];
    // P in the B-operand order of the P V^T product: register r of the score
    // block is key 16 (r / 8) + 8 hh + r % 8 of this half
    f16x8 pf[2];
#pragma unroll
    for (int r = 0; r < 16; ++r)
        pf[r >> 3][r & 7] = (_Float16)__builtin_amdgcn_exp2f(__builtin_fmaf(s[r], scale_log2, mneg));
    // P V^T: products i = (key group u, row block db), V^T fragments PD ahead
    // (the scheduler keeps this order by itself and issues the first reads
    // during the exponentials)
    constexpr int NV = 2 * (HD / 32);
    f16x8 vf[PD];
#pragma unroll
    for (int j = 0; j < PD; ++j) vf[j] = L::v_frag(tile, lo, j % (HD / 32), 2 * KB + j / (HD / 32));
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        st.o[0][i % (HD / 32)] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf[i % PD], pf[i / (HD / 32)],
                                                                        st.o[0][i % (HD / 32)], 0, 0, 0);
        if (i + PD < NV) vf[i % PD] = L::v_frag(tile, lo, (i + PD) % (HD / 32), 2 * KB + (i + PD) / (HD / 32));
    }
    const f16x2 ones = {(_Float16)1.f, (_Float16)1.f};
    float ls = 0.f;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        const f16x2 pair = {pf[p >> 2][2 * (p & 3)], pf[p >> 2][2 * (p & 3) + 1]};
        ls = __builtin_amdgcn_fdot2(pair, ones, ls, false);
    }
    st.l_run[0] += ls;
}

// Dispatch order of the groups of a block-sparse walk kernel: G consecutive
// blocks of one head per workgroup (the forward's kStreamGroup query
// blocks, the backward's query or key blocks).  Workgroups go to the 8 XCDs
// round robin in blockIdx order and each XCD runs its share in that order.
// A fixed split of a head's groups over the XCDs leaves some XCDs more work
// than others (by the estimate below, on the 24 x 64 x 112 grid the XCD
// totals of the forward spread over 0.955-1.026 of their mean), and a costly
// group dispatched last ends the kernel late.  So per head this pass ranks
// the groups by an estimate of their time, costliest first (ties by group
// id), and the walk kernels deal the ranks to the XCDs in a snake
// (group_of_workgroup): rank 8 j + x to XCD x for even j, to XCD 7 - x for
// odd j.  On that grid the forward call went from 120.4 to 117.8 ms.  The
// estimate is 3 x (bits set in the group's rows of the bitmask) + 2 x (bits
// in their union): a selected pair costs the products of one wave pair, a
// union tile its copies and a step of every wave's walk.  Only the order of
// the workgroups changes, never what any of them computes.  One workgroup
// per head; the ranks are sorted in LDS (bitonic sort of 64-bit keys
// ~cost << 32 | group).
constexpr int kOrderMax = 8192;   // >= groups per head for G >= 4 and kSelMax blocks, a power of two
static_assert(kOrderMax >= (kSelMax + 3) / 4, "order table");

constexpr int kOrderThreads = 1024;   // one workgroup per head

template <int G>
__global__ __launch_bounds__(kOrderThreads) void group_order_kernel(SparseGeom g, const uint32_t* __restrict__ mask,
                                                                    int32_t* __restrict__ order) {
    constexpr int kWaves = kOrderThreads / kWave;
    __shared__ uint64_t key[kOrderMax];
    const int head = blockIdx.x;
    const int groups = (g.nb + G - 1) / G;
    const int nw = (g.nb + 31) >> 5;
    int n2 = 1;
    while (n2 < groups) n2 <<= 1;
    const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
    for (int gr = wv; gr < n2; gr += kWaves) {
        uint64_t k = ~0ull;   // padding sorts last
        if (gr < groups) {
            const int b0 = gr * G, nbk = min(G, g.nb - b0);
            const uint32_t* rows = mask + ((int64_t)head * g.nb + b0) * nw;
            int uni = 0, sel = 0;
            for (int wd = lane; wd < nw; wd += 64) {
                uint32_t u = 0u;
                for (int sd = 0; sd < nbk; ++sd) {
                    const uint32_t x = rows[(int64_t)sd * nw + wd];
                    u |= x;
                    sel += __popc(x);
                }
                uni += __popc(u);
            }
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) {
                uni += __shfl_xor(uni, o);
                sel += __shfl_xor(sel, o);
            }
            const uint32_t cost = 3u * (uint32_t)sel + 2u * (uint32_t)uni;
            k = ((uint64_t)(~cost) << 32) | (uint32_t)gr;
        }
        if (lane == 0) key[gr] = k;
    }
    __syncthreads();
    for (int size = 2; size <= n2; size <<= 1)
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = threadIdx.x; i < (n2 >> 1); i += kOrderThreads) {
                const int lo = 2 * i - (i & (stride - 1));   // bit `stride` clear
                const int hi = lo + stride;
                const bool up = (lo & size) == 0;             // ascending run
                const uint64_t a = key[lo], b = key[hi];
                if ((a > b) == up) {
                    key[lo] = b;
                    key[hi] = a;
                }
            }
            __syncthreads();
        }
    for (int r = threadIdx.x; r < groups; r += kOrderThreads)
        order[(int64_t)head * groups + r] = (int32_t)(uint32_t)key[r];
}

// Sparse attention with producer waves.  A workgroup serves G consecutive
// query blocks of one head with 2 G consumer waves, two per block (32
// queries each), and two producer waves.  The producers stream the union of
// the G selections, in ascending block id, into a ring of R LDS tiles (the
// block's K rows and fp16 V^T, one contiguous StreamTile image); producer p
// copies the tiles t with t % 2 == p.  Consumers follow the same walk and
// wait for, compute and release only the tiles their block selected.  There
// is no workgroup barrier in the walk: a producer publishes each tile through
// its slot's LDS flag and reuses a slot once the waves that use the tile in
// it have released it, so a wave waits on another's compute only through a
// full ring.  A producer publishes its previous tile as soon as its copies
// have landed, before it waits for the slot of its next tile: when
// publication waited behind that slot, a tile became visible only after the
// consumers had released the tiles ahead of it, which shrank the consumers'
// lead (4 % slower with one producer).  Two producers keep two tiles' copies
// in flight (one more 1.3 % on the 24 x 64 x 112 grid; three or four gain no
// more).  Larger groups share each staged tile among more blocks (a tile
// costs the same 32 KB however many blocks use it); G = 7 fills the 16 waves
// a workgroup can hold.
//
// Flags: ready[s] = t + 1 once tile t (slot s = t mod R) has landed (slots
// are written in increasing t: tile t + R is issued only after the users of
// tile t released it, which follows its publication); released[s] counts the
// releases of slot s over all its uses, and the producer owning the slot
// (s % 2) counts the releases its tiles are due: two per block that selected
// the tile.
typedef __attribute__((address_space(3))) int lds_int;

__device__ __forceinline__ int lds_load(lds_int* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Publish v into an LDS flag once at most N of this wave's copies are
// outstanding.  The compiler puts a full vmcnt(0) before any LDS store that
// follows global -> LDS copies (it cannot tell the flag from the copy
// target), which would also wait for the copies of the next tile; the wait
// and the store are therefore issued together.  A store has no result
// register, and an LDS operation the compiler does not see only makes its
// own lgkmcnt waits stricter.
template <int N>
__device__ __forceinline__ void publish_after(lds_int* flag, int v) {
    static_assert(N >= 0 && N < 64, "vmcnt immediate");
    __asm__ volatile("s_waitcnt vmcnt(%2)\n\tds_write_b32 %0, %1" ::"v"(flag), "v"(v), "n"(N) : "memory");
}

// Mark the workgroup broken and wait until the flag store has reached LDS
// (lgkmcnt(0); vmcnt and expcnt keep their no-wait maxima), so that anything
// this wave writes to LDS afterwards, a tile copy included, lands after it.
__device__ __forceinline__ void mark_broken(lds_int* broken) {
    __hip_atomic_store(broken, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __asm__ volatile("" ::: "memory");
}

// Wait until *p >= v.  After `limit` sleeps the wait gives up and marks the
// workgroup broken, which ends every later wait at once: a broken protocol
// costs one bounded wait per workgroup, never a hang, and the workgroup
// writes NaN instead of its results.
__device__ __forceinline__ void spin_ge(lds_int* p, int v, lds_int* broken, int limit) {
    for (int i = 0;; ++i) {
        if (__builtin_amdgcn_readfirstlane(lds_load(p)) >= v) break;
        if (__builtin_amdgcn_readfirstlane(lds_load(broken)) != 0) break;
        if (i >= limit) {
            mark_broken(broken);
            break;
        }
        __builtin_amdgcn_s_sleep(1);
    }
    __asm__ volatile("" ::: "memory");
}

template <int HD, int G, int R>
__global__ __launch_bounds__((2 * G + 2) * kWave, 1) void sparse_attn_stream_kernel(
        SparseGeom g, const __bf16* __restrict__ q, float scale_log2, SparseWs w, float* __restrict__ o,
        float* __restrict__ lse, int spin_limit) {
    using L = StreamTile<HD>;
    constexpr int NC = 2 * G;                          // consumer waves; waves NC, NC + 1 produce
    constexpr int KS = HD / 16;
    constexpr int KCP = L::kKBytes / (16 * kWave);     // producer copies per tile: K
    constexpr int VCP = L::kVBytes / (16 * kWave);     //                          V^T
    static_assert(R >= 2 && (R & (R - 1)) == 0, "ring of a power-of-two number of tiles");
    static_assert(KCP + VCP < 64, "vmcnt immediate");
    __shared__ __attribute__((aligned(16))) char lds[R * L::kBytes];
    __shared__ uint32_t msk[G][kSelMax / 32];
    __shared__ int ready[R], released[R], broken;

    static_assert(G == kStreamGroup, "group order table");
    const int groups = (int)stream_groups(g.nb);
    int head, grp;
    if (!group_of_workgroup(groups, g.heads, w.order, head, grp)) return;
    const int nw = (g.nb + 31) >> 5;
    const int b0 = G * grp;

    const uint32_t* mrow = w.mask + ((int64_t)head * g.nb + b0) * nw;
    for (int i = threadIdx.x; i < G * nw; i += (NC + 2) * kWave) {
        const int sd = i / nw, wd = i - (i / nw) * nw;
        msk[sd][wd] = (b0 + sd < g.nb) ? mrow[sd * nw + wd] : 0u;
    }
    if (threadIdx.x < R) {
        ready[threadIdx.x] = 0;
        released[threadIdx.x] = 0;
    }
    if (threadIdx.x == 0) broken = 0;
    __syncthreads();

    const int wv = wave_id();
    const int lane = threadIdx.x & 63;
    const int64_t rstride = (int64_t)g.heads * HD;

    // cursor over the union of the selections (the same walk in every wave)
    int word = 0;
    auto union_word = [&](int wd) {
        uint32_t u = 0u;
#pragma unroll
        for (int sd = 0; sd < G; ++sd) u |= msk[sd][wd];
        return __builtin_amdgcn_readfirstlane(u);
    };
    uint32_t bits = union_word(0);
    auto advance = [&]() -> int {
        while (bits == 0u) {
            if (++word >= nw) return -1;
            bits = union_word(word);
        }
        const int b = __builtin_ctz(bits);
        bits &= bits - 1u;
        return word * 32 + b;
    };
    auto ready_at = [&](int s) { return (lds_int*)&ready[s]; };
    // tile t is published once its slot's flag reaches t + 1
    auto wait_published = [&](int t) {
        for (int i = 0;; ++i) {
            if (__builtin_amdgcn_readfirstlane(lds_load(ready_at(t & (R - 1)))) >= t + 1) break;
            if (__builtin_amdgcn_readfirstlane(lds_load((lds_int*)&broken)) != 0) break;
            if (i >= spin_limit) {
                mark_broken((lds_int*)&broken);
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        __asm__ volatile("" ::: "memory");
    };
    auto released_at = [&](int s) { return (lds_int*)&released[s]; };
    lds_int* brk = (lds_int*)&broken;

    if (wv >= NC) {
        // ---- producers: wave NC + p copies the tiles t with t % 2 == p ----
        const int pp = wv - NC;
        int t = 0, last = -1;
        // releases of this producer's slots (sl % 2 == pp) that its tiles so
        // far will collect: two per block that selected the tile
        int due[R / 2];
#pragma unroll
        for (int i = 0; i < R / 2; ++i) due[i] = 0;
        for (int j = advance(); j >= 0; j = advance(), ++t) {
            if (t % 2 != pp) continue;
            const int sl = t & (R - 1);
            // publish this producer's previous tile once it has landed
            if (last >= 0) publish_after<0>(ready_at(last & (R - 1)), last + 1);
            int users = 0;
#pragma unroll
            for (int sd = 0; sd < G; ++sd) users += (msk[sd][j >> 5] >> (j & 31)) & 1u;
            users = __builtin_amdgcn_readfirstlane(users);
#pragma unroll
            for (int i = 0; i < R / 2; ++i) {
                if ((sl >> 1) != i) continue;
                // every user of tile t - R in this slot is done with it
                if (t >= R) spin_ge(released_at(sl), due[i], brk, spin_limit);
                due[i] += 2 * users;
            }
            char* lb = lds + sl * L::kBytes;
            const int64_t blk = (int64_t)head * g.nb + j;
            const char* kt = reinterpret_cast<const char*>(w.kimg + blk * (kTileN * HD)) + 16 * lane;
#pragma unroll
            for (int i = 0; i < KCP; ++i) dma16(kt + i * 1024, lb + i * 1024);
            const char* vt = reinterpret_cast<const char*>(w.vt + blk * (HD * kTileN)) + 16 * lane;
#pragma unroll
            for (int i = 0; i < VCP; ++i) dma16(vt + i * 1024, lb + L::kKBytes + i * 1024);
            last = t;
        }
        if (last >= 0) publish_after<0>(ready_at(last & (R - 1)), last + 1);
        return;
    }

    // ---- consumers: waves 2 b and 2 b + 1 hold the two halves of block b ----
    const int side = wv >> 1;
    const int hh = lane >> 5;
    const int m = lane & 31;
    const int qb = min(b0 + side, g.nb - 1);
    const int qr = (wv & 1) * 32 + m;
    const int64_t qtok = (int64_t)w.base[qb] + (w.tdim ? tile_local(g, w.tdim[qb], qr) : block_local(g, qr));
    bf16x8 qf[1][KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        qf[0][ks] = load_bf16x8(q + qtok * rstride + head * HD + 16 * ks + 8 * hh, true);

    const int lo = L::lane_offset();
    SoftmaxState<HD, 1> st;
    st.init();
    int t = 0;
    int own_word = -1;      // word of this block's mask held in own
    uint32_t own = 0u;
    for (int j = advance(); j >= 0; j = advance(), ++t) {
        const int sl = t & (R - 1);
        if ((j >> 5) != own_word) {
            own_word = j >> 5;
            own = __builtin_amdgcn_readfirstlane(msk[side][own_word]);
        }
        // Only the waves of blocks that selected a tile wait for it and
        // release it; the producer reuses the slot once those releases are
        // in.  A wave whose block skips a stretch of tiles therefore neither
        // waits for them nor holds their slots.
        if (!((own >> (j & 31)) & 1u)) continue;
        wait_published(t);
        const char* cur = lds + sl * L::kBytes;
        half_tile_step<HD, 0>(cur, lo, qf[0], st, scale_log2);
        __builtin_amdgcn_sched_barrier(0);
        half_tile_step<HD, 1>(cur, lo, qf[0], st, scale_log2);
        // this wave's reads of the slot are done (LDS serves a wave in order)
        __asm__ volatile("" ::: "memory");
        if (lane == 0) __hip_atomic_fetch_add(released_at(sl), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }

    if (b0 + side >= g.nb) return;
    // A wave that gave up on a wait, or whose tiles a producer that gave up
    // may have overwritten, finds the flag set here (the flag store completes
    // before any later copy of that producer lands): its rows become NaN.
    const bool bad = __builtin_amdgcn_readfirstlane(lds_load(brk)) != 0;
    const float l_tot = st.l_run[0] + __shfl_xor(st.l_run[0], 32);
    // O^T accumulated V scaled by 2^ve: scale back (exact)
    const int ve = v_scale_exp(w.vmax, head);
    store_o<HD>(o + qtok * rstride + head * HD, st.o[0],
                bad ? __builtin_nanf("") : __builtin_ldexpf(1.f / l_tot, -ve));
    // log-sum-exp over the selected keys, natural log (reference maximum and
    // running sum are in the exp2 domain)
    if (lse && hh == 0)
        lse[(int64_t)head * ((int64_t)g.T * g.H * g.W) + qtok] =
            bad ? __builtin_nanf("") : (st.m_run[0] + log2f(l_tot)) * kLn2;
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

hipError_t launch_vt_blocks(const SparseGeom& g, const __bf16* k, const __bf16* v, int hd, const SparseWs& w,
                            hipStream_t s) {
    hipLaunchKernelGGL(vt_blocks_kernel<128>, dim3(g.nb, g.heads), dim3(256), 0, s, g, k, v, w);
    (void)hd;
    return hipGetLastError();
}

hipError_t launch_block_scores(const SparseGeom& g, int hd, double scale, const SparseWs& w, int row0, int rows,
                               hipStream_t s) {
    const unsigned ct = (unsigned)((g.nb + kSB - 1) / kSB), rt = (unsigned)((rows + kSB - 1) / kSB);
    hipLaunchKernelGGL(block_scores_kernel<128>, dim3(ct, rt, g.heads), dim3(256), 0, s, g, scale, w, row0, rows);
    (void)hd;
    return hipGetLastError();
}

hipError_t launch_block_select(const SparseGeom& g, int top_k, double top_p, const SparseWs& w, int row0, int rows,
                               uint32_t* sel_mask, int32_t* sel_count, hipStream_t s) {
    const int em = (g.nb + 63) / 64;   // elements per lane with one wave per row
    const bool ad = w.lead != nullptr;
    auto go = [&](auto kernel, unsigned blocks, unsigned threads) {
        hipLaunchKernelGGL(kernel, dim3(blocks), dim3(threads), 0, s, g, top_k, top_p, w, row0, rows, sel_mask,
                           sel_count);
    };
    const unsigned one = (unsigned)((g.heads * rows + kSelWaves - 1) / kSelWaves), wide = (unsigned)(g.heads * rows);
    if (em <= 8)
        ad ? go(block_select_kernel<8, 1, true>, one, 64 * kSelWaves) : go(block_select_kernel<8, 1, false>, one, 64 * kSelWaves);
    else if (em <= 16)
        ad ? go(block_select_kernel<16, 1, true>, one, 64 * kSelWaves) : go(block_select_kernel<16, 1, false>, one, 64 * kSelWaves);
    else if (em <= 32)
        ad ? go(block_select_kernel<32, 1, true>, one, 64 * kSelWaves) : go(block_select_kernel<32, 1, false>, one, 64 * kSelWaves);
    else if (em <= 48)
        ad ? go(block_select_kernel<48, 1, true>, one, 64 * kSelWaves) : go(block_select_kernel<48, 1, false>, one, 64 * kSelWaves);
    else if (em <= 64)
        ad ? go(block_select_kernel<64, 1, true>, one, 64 * kSelWaves) : go(block_select_kernel<64, 1, false>, one, 64 * kSelWaves);
    // more than 4096 blocks: 2, 4 or 8 waves per row, 64 elements per lane
    else if (em <= 128)
        ad ? go(block_select_kernel<64, 2, true>, wide, 128) : go(block_select_kernel<64, 2, false>, wide, 128);
    else if (em <= 256)
        ad ? go(block_select_kernel<64, 4, true>, wide, 256) : go(block_select_kernel<64, 4, false>, wide, 256);
    else
        ad ? go(block_select_kernel<64, 8, true>, wide, 512) : go(block_select_kernel<64, 8, false>, wide, 512);
    return hipGetLastError();
}

hipError_t launch_group_order(const SparseGeom& g, int group, const uint32_t* mask, int32_t* order, hipStream_t s) {
    if (group == kStreamGroup)
        hipLaunchKernelGGL(group_order_kernel<kStreamGroup>, dim3(g.heads), dim3(kOrderThreads), 0, s, g, mask,
                           order);
    else if (group == kBwdGroup)
        hipLaunchKernelGGL(group_order_kernel<kBwdGroup>, dim3(g.heads), dim3(kOrderThreads), 0, s, g, mask, order);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_sparse_attn(const SparseGeom& g, const __bf16* q, int hd,
                              float scale_log2, const SparseWs& w, float* o, float* lse, int wait_limit,
                              hipStream_t s) {
    (void)hd;
    constexpr int G = kStreamGroup, R = kStreamRing;
    const unsigned blocks = (unsigned)group_workgroups(stream_groups(g.nb), g.heads);
    hipLaunchKernelGGL((sparse_attn_stream_kernel<128, G, R>), dim3(blocks), dim3((2 * G + 2) * kWave), 0, s, g, q,
                       scale_log2, w, o, lse, wait_limit);
    return hipGetLastError();
}

}  // namespace mmdit
