// Block-sparse video self-attention (Prism page, xyznot.com 2610.05416:
// "Ideas clave" macro-zones and hybrid top-k/top-p; "Metodo" section 3).
//
// Kernels, in launch order:
//   block_pool     fp64 means of each block's 64 query rows and 64 key rows,
//                  per head (HBM-bound: reads Q and K once); also records each
//                  block's first raster token.
//   vt_blocks      each block's K rows (bf16) and V^T (fp16 [d][64]), each
//                  laid out as the image of its LDS tile (HBM-bound).
//   block_scores   fp64 logits Qbar Kbar^T * scale per head (fp64 FMA GEMM).
//   block_select   per (head, query block): fp64 softmax, then the top-p and
//                  top-k cuts found by bisection over the probabilities' bit
//                  patterns (ties to the lower block id), keeping the longer
//                  prefix; emits the bitmask and the count.
//   sparse_attn    attention of groups of query blocks over the union of
//                  their selected key blocks, fed through an LDS ring by
//                  producer waves, with the dense kernel's online-softmax
//                  tile step.
// Selection runs in fp64 throughout: on smooth-field inputs the probability
// gaps and running-sum margins at the cut get down to ~1e-8, where fp32 flips
// rows.
#include <cstdlib>
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

// One workgroup per (block, head): gather the block's 64 rows of K and of V
// and write each as the exact image of its LDS tile (K rows in the MFMA row
// order, V transposed to fp16 [d][64], 16-byte chunks swizzled), so that the
// attention kernel stages a tile with two contiguous 16 KB copies instead of
// 64 scattered 256-byte rows.
template <int HD>
__global__ __launch_bounds__(256) void vt_blocks_kernel(SparseGeom g, const __bf16* __restrict__ k,
                                                        const __bf16* __restrict__ v, SparseWs w) {
    using L = TileLayout<HD>;
    __shared__ _Float16 tile[kTileN][HD + 2];
    const int j = blockIdx.x, head = blockIdx.y;
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
        for (int i = 0; i < 8; ++i) tile[r][c * 8 + i] = (_Float16)(float)x[i];
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

constexpr int kSelWaves = 4;   // rows (one per wave) per selection workgroup
// Sparse attention: query blocks per workgroup and LDS ring depth (tiles).
// Measured on the 24 x 64 x 112 grid (density 27.6 %): a group stages on
// average 0.73 (pairs), 0.62 (triples), 0.50 (4 blocks) of the tiles its
// blocks select; with workgroup barriers per tile, pairs (two workgroups per
// CU) took 164 ms and groups of 4 (idle waves on tiles only some blocks
// selected) 205 ms, while groups of 4 fed by producer waves take 132-134 ms.
constexpr int kStreamGroup = 4;
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

// Selection of one row of block probabilities, one wave per row.  Lane l
// holds blocks j = l + 64 r.  The blocks in descending order of probability
// (equal probabilities by ascending id) are never sorted: for a non-negative
// double the bit pattern read as an unsigned integer orders like the value,
// so the row is searched by bisection over that integer range.
//   top-p: the element e at which the descending running sum first reaches p
//          is the largest key x with sum(P >= x) >= p; within a run of equal
//          values the running sum advances one element at a time.
//   top-k: the k-th element is the largest key x with count(P >= x) >= k.
// The selection is the longer of the two prefixes.  Slots past the row hold
// P = -1, which no threshold >= 0 admits.
template <int EM, bool AD>   // elements per lane: nb <= 64 EM; AD: adaptive blocks (w.lead set)
__global__ __launch_bounds__(64 * kSelWaves) void block_select_kernel(SparseGeom g, int top_k,
                                                                      double top_p, SparseWs w,
                                                                      uint32_t* __restrict__ sel_mask,
                                                                      int32_t* __restrict__ sel_count) {
    const int nb = g.nb;
    const int row = (int)blockIdx.x * kSelWaves + wave_id();   // head * nb + i
    if (row >= g.heads * nb) return;
    const int lane = threadIdx.x & 63;
    const double* L = w.scores + (int64_t)row * nb;

    // Columns that are blocks: every column with uniform blocks; with adaptive
    // blocks only each block's first tile (the other tiles of the block repeat
    // its logit and take its decision at the end).
    uint64_t okm = 0;
    int nv = nb;   // blocks in the row
    if constexpr (AD) {
#pragma unroll
        for (int r = 0; r < EM; ++r) {
            const int j = lane + 64 * r;
            if (j < nb && w.lead[j] == j) okm |= 1ull << r;
        }
        nv = 0;
#pragma unroll
        for (int r = 0; r < EM; ++r) nv += __popcll(__ballot((okm >> r) & 1ull));
    }
    auto col_ok = [&](int r) { return AD ? ((okm >> r) & 1ull) != 0 : lane + 64 * r < nb; };

    // softmax over the row's blocks, fp64
    double P[EM];
    double mx = -__builtin_inf();
#pragma unroll
    for (int r = 0; r < EM; ++r) {
        const int j = lane + 64 * r;
        P[r] = col_ok(r) ? L[j] : -__builtin_inf();
        mx = fmax(mx, P[r]);
    }
    mx = wave_max(mx);
    double se = 0.0;
#pragma unroll
    for (int r = 0; r < EM; ++r) {
        if (col_ok(r)) {
            P[r] = exp(P[r] - mx);
            se += P[r];
        }
    }
    se = wave_sum(se);
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
    tot = wave_sum(tot);

    auto count_ge = [&](double t) {
        int c = 0;
#pragma unroll
        for (int r = 0; r < EM; ++r)
            c += __popcll(__ballot(P[r] >= t));
        return c;
    };
    auto count_eq = [&](double t) {
        int c = 0;
#pragma unroll
        for (int r = 0; r < EM; ++r)
            c += __popcll(__ballot(P[r] == t));
        return c;
    };
    auto count_in = [&](double lo, double hi) {
        int c = 0;
#pragma unroll
        for (int r = 0; r < EM; ++r)
            c += __popcll(__ballot(P[r] >= lo && P[r] < hi));
        return c;
    };
    auto sum_ge = [&](double t) {
        double x = 0.0;
#pragma unroll
        for (int r = 0; r < EM; ++r)
            if (P[r] >= t) x += P[r];
        return wave_sum(x);
    };
    // the one value left in [lo, hi) once the bisection stops
    auto value_in = [&](double lo, double hi) {
        double x = -1.0;
#pragma unroll
        for (int r = 0; r < EM; ++r)
            if (P[r] >= lo && P[r] < hi) x = fmax(x, P[r]);
        return wave_max(x);
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
            vp = wave_max(x);
            mp = 1;
            n_p = 1;
        } else {
            uint64_t lo = 0, hi = kInf;   // sum(P >= lo) >= p > sum(P >= hi)
            while (hi - lo > 1 && count_in(key_value(lo), key_value(hi)) > 1) {
                const uint64_t mid = lo + ((hi - lo) >> 1);
                if (sum_ge(key_value(mid)) >= top_p)
                    lo = mid;
                else
                    hi = mid;
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

    // top-k prefix
    const int kk = top_k < nv ? top_k : nv;
    double vk = -1.0;
    int mk = 0;
    if (kk > 0 && kk < nv) {
        uint64_t lo = 0, hi = kInf;   // count(P >= lo) >= k > count(P >= hi)
        while (hi - lo > 1 && count_in(key_value(lo), key_value(hi)) > 1) {
            const uint64_t mid = lo + ((hi - lo) >> 1);
            if (count_ge(key_value(mid)) >= kk)
                lo = mid;
            else
                hi = mid;
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
    const int nw = (nb + 31) >> 5;
    uint32_t* mrow = w.mask + (int64_t)row * nw;
    uint32_t* srow = sel_mask ? sel_mask + (int64_t)row * nw : nullptr;
    int before = 0;        // run elements with a lower id
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
            b = __ballot(sel || (inh && lane + 64 * r < nb));
        }
        const int wd = 2 * r + lane;
        if (lane < 2 && wd < nw) {   // words past the row hold no bits
            const uint32_t word = lane ? (uint32_t)(b >> 32) : (uint32_t)b;
            mrow[wd] = word;
            if (srow) srow[wd] = word;
        }
    }
    if (lane == 0) {
        w.count[row] = K;
        if (sel_count) sel_count[row] = K;
    }
}

// Sparse attention with producer waves.  A workgroup serves G consecutive
// query blocks of one head with 2 G consumer waves, two per block (which
// waves own which block is chosen for the SIMD placement described at the
// consumers), and two producer waves.  The producers stream the union of
// the G selections, in ascending block id, into a ring of R LDS tiles (the
// block's K rows and fp16 V^T, each one contiguous image); producer p copies
// the tiles t with t % 2 == p.  Consumers follow the same walk and compute
// only the tiles their block selected.  There is no workgroup barrier in the
// walk: a producer publishes each tile through its slot's LDS flag and reuses
// a slot once every consumer has released the tile in it, so the consumers
// run up to R - 1 tiles apart and none waits on another's compute except
// through a full ring.  A producer publishes its previous tile as soon as its
// copies have landed, before it waits for the slot of its next tile: when
// publication waited behind that slot, a tile became visible only after the
// consumers had released the tiles ahead of it, which shrank the consumers'
// lead (4 % slower with one producer).  Two producers keep two tiles' copies
// in flight (one more 1.3 % on the 24 x 64 x 112 grid; three or four gain no
// more).  Larger groups share each staged tile among more blocks (a tile
// costs the same 32 KB however many blocks use it), and the decoupled walk
// keeps the waves of blocks that did not select a tile from idling on it.
//
// Flags: ready[s] = t + 1 once tile t (slot s = t mod R) has landed (slots
// are written in increasing t: tile t + R is issued only after every consumer
// released tile t, which follows its publication); released[s] counts
// consumer waves done with slot s over all its uses.
constexpr int kSpinLimit = 1 << 18;
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

// Wait until *p >= v.  After `limit` sleeps (kSpinLimit unless the host
// lowers it) the wait gives up and marks the workgroup broken, which ends
// every later wait at once: a broken protocol costs one bounded wait per
// workgroup and wrong results, never a hang.
__device__ __forceinline__ void spin_ge(lds_int* p, int v, lds_int* broken, int limit) {
    for (int i = 0;; ++i) {
        if (__builtin_amdgcn_readfirstlane(lds_load(p)) >= v) break;
        if (__builtin_amdgcn_readfirstlane(lds_load(broken)) != 0) break;
        if (i >= limit) {
            __hip_atomic_store(broken, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            break;
        }
        __builtin_amdgcn_s_sleep(1);
    }
    __asm__ volatile("" ::: "memory");
}

template <int HD, int G, int R>
__global__ __launch_bounds__((2 * G + 2) * kWave, 1) void sparse_attn_stream_kernel(
        SparseGeom g, const __bf16* __restrict__ q, const __bf16* __restrict__ k, float scale_log2,
        SparseWs w, float* __restrict__ o, float* __restrict__ lse, int spin_limit) {
    using L = TileLayout<HD>;
    constexpr int NC = 2 * G;                          // consumer waves; waves NC, NC + 1 produce
    constexpr int KS = HD / 16;
    constexpr int KCP = kTileN * L::kKChunks / kWave;  // producer copies per tile: K
    constexpr int VCP = HD * 8 / kWave;                //                          V^T
    static_assert(R >= 2 && (R & (R - 1)) == 0, "ring of a power-of-two number of tiles");
    static_assert(KCP + VCP < 64, "vmcnt immediate");
    __shared__ __attribute__((aligned(16))) char lds[R * L::kBytes];
    __shared__ uint32_t msk[G][kSelMax / 32];
    __shared__ int ready[R], released[R], broken;

    const int groups = (g.nb + G - 1) / G;
    const int per = (groups + 7) >> 3;
    const int slot = (int)(blockIdx.x >> 3);
    const int head = slot / per;
    const int grp = (int)(blockIdx.x & 7) * per + (slot - head * per);
    if (head >= g.heads || grp >= groups) return;
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
                __hip_atomic_store((lds_int*)&broken, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
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
        for (int j = advance(); j >= 0; j = advance(), ++t) {
            if (t % 2 != pp) continue;
            const int sl = t & (R - 1);
            // publish this producer's previous tile once it has landed
            if (last >= 0) publish_after<0>(ready_at(last & (R - 1)), last + 1);
            if (t >= R) spin_ge(released_at(sl), NC * (t / R), brk, spin_limit);   // tile t - R is done
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

    // ---- consumers ----
    // Waves w and w + 4 share a SIMD.  Blocks of a group are a 2 x 2 (h, w)
    // square of neighbours; the selections of edge neighbours correlate most,
    // so each SIMD gets one wave of each block of a diagonal pair (blocks 0
    // and 3 on SIMDs 0-1, 1 and 2 on SIMDs 2-3) and concurrent work on edge
    // neighbours spreads over all four SIMDs.
    const int side = G == 4 ? (wv < 4 ? (wv >> 1) : 3 - ((wv - 4) >> 1)) : (wv >> 1);
    const int hh = lane >> 5;
    const int m = lane & 31;
    const int qb = min(b0 + side, g.nb - 1);
    const int qr = (wv & 1) * 32 + m;
    const int64_t qtok = (int64_t)w.base[qb] + (w.tdim ? tile_local(g, w.tdim[qb], qr) : block_local(g, qr));
    bf16x8 qf[1][KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        qf[0][ks] = load_bf16x8(q + qtok * rstride + head * HD + 16 * ks + 8 * hh, true);

    FragAddr<HD> fa;
    fa.init();
    f32x16 sc[1][2], sd[1][2];
    float mx[1];
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
        // Wait for the tile even when this block skips it: released[] counts
        // every use of a slot, so a wave may release tile t only once tile
        // t has been published, i.e. once every wave released tile t - R.
        // Otherwise a wave skipping ahead could release t and t + R before
        // a slower wave is done with t, and the producer would overwrite it.
        wait_published(t);
        if ((own >> (j & 31)) & 1u) {
            const char* cur = lds + sl * L::kBytes;
            qk_tile<HD, 1>(cur, fa, qf, sc);
            tile_max<false, 1>(sc, scale_log2, kTileN, mx);
            maybe_rescale<HD, 1>(st, mx);
            tile_step<HD, 1, false, false>(nullptr, cur + L::kKBytes, fa, qf, sc, sd, st, scale_log2, kTileN, mx);
        }
        // this wave's reads of the slot are done (LDS serves a wave in order)
        __asm__ volatile("" ::: "memory");
        if (lane == 0) __hip_atomic_fetch_add(released_at(sl), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }

    if (b0 + side >= g.nb) return;
    const float l_tot = st.l_run[0] + __shfl_xor(st.l_run[0], 32);
    store_o<HD>(o + qtok * rstride + head * HD, st.o[0], 1.f / l_tot);
    // log-sum-exp over the selected keys, natural log (reference maximum and
    // running sum are in the exp2 domain)
    if (lse && hh == 0)
        lse[(int64_t)head * ((int64_t)g.T * g.H * g.W) + qtok] = (st.m_run[0] + log2f(l_tot)) * kLn2;
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
    const unsigned blocks = (unsigned)((g.heads * g.nb + kSelWaves - 1) / kSelWaves);
    const dim3 grid(blocks), block(64 * kSelWaves);
    const int em = (g.nb + 63) / 64;
    auto go = [&](auto kernel) {
        hipLaunchKernelGGL(kernel, grid, block, 0, s, g, top_k, top_p, w, sel_mask, sel_count);
    };
    const bool ad = w.lead != nullptr;
    if (em <= 8)
        ad ? go(block_select_kernel<8, true>) : go(block_select_kernel<8, false>);
    else if (em <= 16)
        ad ? go(block_select_kernel<16, true>) : go(block_select_kernel<16, false>);
    else if (em <= 32)
        ad ? go(block_select_kernel<32, true>) : go(block_select_kernel<32, false>);
    else if (em <= 48)
        ad ? go(block_select_kernel<48, true>) : go(block_select_kernel<48, false>);
    else
        ad ? go(block_select_kernel<64, true>) : go(block_select_kernel<64, false>);
    return hipGetLastError();
}

// Bound of every wait in the stream kernel, in sleeps of about 64 cycles.
// MMDIT_SPARSE_SPIN_LIMIT (a non-negative integer) lowers it: tests set 0 to
// force the give-up path from the host and check that the kernel still ends.
static int stream_spin_limit() {
    const char* e = std::getenv("MMDIT_SPARSE_SPIN_LIMIT");
    if (!e || !*e) return kSpinLimit;
    char* end = nullptr;
    const long v = std::strtol(e, &end, 10);
    if (*end != '\0' || v < 0) return kSpinLimit;
    return (int)std::min<long>(v, kSpinLimit);
}

hipError_t launch_sparse_attn(const SparseGeom& g, const __bf16* q, const __bf16* k, int hd,
                              float scale_log2, const SparseWs& w, float* o, float* lse, hipStream_t s) {
    (void)hd;
    constexpr int G = kStreamGroup, R = kStreamRing;
    const unsigned blocks = (unsigned)(8 * ((((g.nb + G - 1) / G) + 7) / 8) * g.heads);
    hipLaunchKernelGGL((sparse_attn_stream_kernel<128, G, R>), dim3(blocks), dim3((2 * G + 2) * kWave), 0, s, g,
                       q, k, scale_log2, w, o, lse, stream_spin_limit());
    return hipGetLastError();
}

}  // namespace mmdit
