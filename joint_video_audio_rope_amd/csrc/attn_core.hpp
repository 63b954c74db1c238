// Shared inner loop of the bf16 attention kernels (dense and block-sparse).
//
// One wavefront owns QB blocks of 32 queries.  Per 64-key tile it computes the transposed
// score block S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (K from LDS as the A
// operand, the wave's Q rows held in registers as the B operand), runs the
// fp32 online softmax in the exp2 domain, and accumulates O^T += V^T P^T with
// v_mfma_f32_32x32x16_f16 (V^T from LDS as A, P from registers as B).
//
// Why transposed: in the 32x32 MFMA result, lane l holds column l % 32 for 16
// rows.  With queries as columns every lane owns exactly one query for both
// the score block and the O accumulator, so row max, row sum and the rescale
// of O need no data movement except one exchange with lane l ^ 32 (which
// holds the other half of the same query's keys).
//
// Key order inside a tile: MFMA row m of the score block holds key pi(m), pi
// swapping bits 2 and 3 of m.  Then register r of lane l (hh = l / 32) holds
// key 16 (r / 8) + 8 hh + r % 8, so the 8 registers of one 16-key group are 8
// consecutive keys: exactly the B-operand slot order of the P V^T product,
// whose A operand is then one contiguous 16-byte read of V^T.
//
// The softmax keeps a reference maximum per query and only moves it (and
// rescales O and the running sum) when a tile's maximum exceeds it by more
// than 2^8 in the exp2 domain.  Exponentials then stay <= 256, well inside
// fp16, and the O accumulators are touched by vector ALU instructions only on
// those rare tiles instead of every tile.
//
// LDS layouts XOR-swizzle the 16-byte chunks of each row so the 16 lanes
// that read one chunk column at a time hit 16 different bank groups.
// Tiles are copied global -> LDS with global_load_lds_dwordx4 (no register
// staging): one instruction moves 64 lanes x 16 bytes into 1 KiB of LDS, lane
// i landing at byte 16 i; each lane therefore fetches the global chunk that
// belongs at its LDS position.
#pragma once

#include "internal.hpp"

namespace mmdit {

#define MMDIT_LDS(p) ((__attribute__((address_space(3))) void*)(p))

__device__ __forceinline__ int perm_row(int m) {
    return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

// Key (0..63 inside the tile) held by register r of S block kb in lane half hh.
__device__ __forceinline__ int tile_key(int kb, int r, int hh) {
    return 32 * kb + 16 * (r >> 3) + 8 * hh + (r & 7);
}

template <int HD>
struct TileLayout {
    static constexpr int kKRowBytes = HD * 2;          // bf16 row of K
    static constexpr int kKChunks = HD / 8;            // 16-byte chunks per K row
    static constexpr int kKBytes = kTileN * HD * 2;
    static constexpr int kVRowBytes = kTileN * 2;      // fp16 row of V^T (64 keys)
    static constexpr int kVBytes = HD * kTileN * 2;
    static constexpr int kBytes = kKBytes + kVBytes;   // one K + V^T tile
    // XOR applied to the chunk index of a row.  gfx950 LDS serves a 16-byte
    // read of 16 consecutive lanes per cycle (256 B): those 16 lanes read one
    // chunk column of 16 consecutive rows and must land in 16 different
    // 16-byte slots of a 256-byte line.  256-byte rows: XOR with row & 15.
    // 128-byte rows (two per line, the line half given by row & 1): XOR with
    // (row ^ ((row & 31) >> 3)) & 7, which is distinct over 16 aligned rows
    // together with row & 1 and over any 8 aligned rows by itself, and repeats
    // every 32 rows (so 32-row blocks differ by a constant byte offset).
    __device__ static int swz(int row, int chunks) {
        return chunks >= 16 ? (row & 15) : ((row ^ ((row & 31) >> 3)) & 7);
    }
    __device__ static int k_off(int row, int chunk) {
        return row * kKRowBytes + ((chunk ^ swz(row, kKChunks)) << 4);
    }
    __device__ static int v_off(int d, int chunk) {
        return d * kVRowBytes + ((chunk ^ swz(d, 8)) << 4);
    }
    // Inverse maps: which (row, chunk) lives at LDS chunk index L.
    __device__ static void k_at(int L, int& row, int& chunk) {
        row = L / kKChunks;
        chunk = (L % kKChunks) ^ swz(row, kKChunks);
    }
    __device__ static void v_at(int L, int& d, int& chunk) {
        d = L >> 3;
        chunk = (L & 7) ^ swz(d, 8);
    }
};

// Online-softmax state of a wave's QB query blocks of 32 queries each; lane
// l owns query l % 32 of every block.
template <int HD, int QB = 1>
struct SoftmaxState {
    static constexpr int DB = HD / 32;
    f32x16 o[QB][DB];
    float m_run[QB];   // reference max of scaled logits (log2 domain)
    float l_run[QB];   // running sum over this lane's half of the keys
    __device__ void init() {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
            for (int i = 0; i < DB; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[qb][i][r] = 0.f;
            m_run[qb] = -__builtin_inff();
            l_run[qb] = 0.f;
        }
    }
};

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));


// Per-lane LDS byte offsets of the 16 K fragments (i = 2 ks + kb) and the 16
// V^T fragments (i = 4 db + g) of a tile, relative to the tile's K / V^T base.
template <int HD>
struct FragAddr {
    int k[HD / 16];   // K fragment of step ks for rows 0..31; rows 32..63 add 32 rows
    int v[4];         // V^T fragment of key group g for d rows 0..31; block db adds 32 db rows
    __device__ void init() {
        using L = TileLayout<HD>;
        const int lane = threadIdx.x & 63;
        const int hh = lane >> 5, m = lane & 31;
#pragma unroll
        for (int ks = 0; ks < HD / 16; ++ks) k[ks] = L::k_off(m, 2 * ks + hh);
#pragma unroll
        for (int g = 0; g < 4; ++g) v[g] = L::v_off(m, 2 * g + hh);
    }
};

// K fragment i = 2 ks + kb (the swizzle repeats every 16 rows, so rows
// 32..63 sit 32 rows further on).
template <int HD>
__device__ __forceinline__ bf16x8 k_frag(const char* lk, const FragAddr<HD>& fa, int i) {
    return *reinterpret_cast<const bf16x8*>(lk + fa.k[i >> 1] + (i & 1) * 32 * TileLayout<HD>::kKRowBytes);
}

// V^T fragment i = 4 db + g (the swizzle repeats every 32 rows).
template <int HD>
__device__ __forceinline__ f16x8 v_frag(const char* lv, const FragAddr<HD>& fa, int i) {
    return *reinterpret_cast<const f16x8*>(lv + fa.v[i & 3] + (i >> 2) * 32 * TileLayout<HD>::kVRowBytes);
}

// Instruction order for a chain of N MFMAs whose LDS fragments are read PD
// products ahead into PD alternating registers: PD reads, then (one MFMA,
// the next read) N - PD times, then the last PD MFMAs.  Left alone, the
// scheduler tends to issue each read right before its product and wait for
// it (lgkmcnt(0)), so the wave pays the LDS latency once per MFMA.  EXTRA
// further LDS reads of the region (say row statistics) join after pair i
// whenever i % PERIOD == AT.  Call once, after the code of the region it
// orders (a basic block; the groups are matched against its instructions).
template <int PD, int N, int PERIOD = 1, int AT = 0, int EXTRA = 0>
__device__ __forceinline__ void order_fragment_stream() {
    constexpr int kMfma = 0x008, kDsRead = 0x100;   // sched_group_barrier instruction classes
    __builtin_amdgcn_sched_group_barrier(kDsRead, PD, 0);
#pragma unroll
    for (int i = 0; i < N - PD; ++i) {
        __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kDsRead, 1, 0);
        if (EXTRA > 0 && i % PERIOD == AT) __builtin_amdgcn_sched_group_barrier(kDsRead, EXTRA, 0);
    }
    __builtin_amdgcn_sched_group_barrier(kMfma, PD, 0);
}

// Scores S^T = K Q^T of one tile (not overlapped; the first tile of a walk).
// Each K fragment read from LDS feeds the QB query blocks.
template <int HD, int QB>
__device__ __forceinline__ void qk_tile(const char* lk, const FragAddr<HD>& fa,
                                        const bf16x8 (&qf)[QB][HD / 16], f32x16 (&s)[QB][2]) {
    constexpr int NF = HD / 8;   // fragments per tile: 2 blocks x HD/16 steps
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) s[qb][kb][r] = 0.f;
#pragma unroll
    for (int i = 0; i < NF; ++i) {
        const bf16x8 kf = k_frag<HD>(lk, fa, i);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
            s[qb][i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[qb][i >> 1], s[qb][i & 1], 0, 0, 0);
    }
}

// Maximum of x over lanes l and l ^ 32 (the two halves of one query's keys).
// v_permlane32_swap with the same register as both operands returns the
// lower half's values in every lane (first result) and the upper half's in
// every lane (second result).
__device__ __forceinline__ float pair_max(float x) {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}

// Scaled (log2-domain) maximum of each query block's score tile over both
// halves of the lane pair; with MASK, keys >= valid are set to -inf first.
template <bool MASK, int QB>
__device__ __forceinline__ void tile_max(f32x16 (&s)[QB][2], float scale_log2, int valid, float (&mx)[QB]) {
    const int hh = (threadIdx.x & 63) >> 5;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        if (MASK) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (tile_key(kb, r, hh) >= valid) s[qb][kb][r] = -__builtin_inff();
        }
        float x = s[qb][0][0];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) x = fmaxf(x, s[qb][kb][r]);
        mx[qb] = pair_max(x) * scale_log2;
    }
}

// Move the reference max when a tile's max exceeds it by more than 2^8
// (wave-uniform branch, rare after the first tiles).
template <int HD, int QB>
__device__ __forceinline__ void maybe_rescale(SoftmaxState<HD, QB>& st, const float (&mx)[QB]) {
    bool up = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) up |= mx[qb] > st.m_run[qb] + 8.f;
    if (__any(up)) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const float m_new = fmaxf(st.m_run[qb], mx[qb]);
            const float alpha = __builtin_amdgcn_exp2f(st.m_run[qb] - m_new);
            st.m_run[qb] = m_new;
            st.l_run[qb] *= alpha;
#pragma unroll
            for (int db = 0; db < HD / 32; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) st.o[qb][db][r] *= alpha;
        }
    }
}

// One pipelined step for the wave's QB x 32 queries.
//   phase 1: P(t) = exp2(S(t) * scale - m) into fp16, interleaved with the
//            16 QB MFMAs of S(t+1) = K(t+1) Q^T (when NEXT);
//   phase 2: O^T += V(t)^T P(t)^T (16 QB MFMAs), interleaved with the row sum
//            of P(t) (fp16 pairs through v_dot2, i.e. exactly the values the
//            MFMA consumes) and, when NEXT, the maximum of S(t+1).
// Every fragment read from LDS feeds QB MFMAs.  Writes the scaled maximum of
// S(t+1) per query block to mx (untouched when !NEXT).  The vector work is
// left to the instruction scheduler (pinning each MFMA slot with its share of
// the softmax measured 2.4 % slower on the 35050-token joint attention).
// With PIN (QB = 1) the LDS reads and MFMAs of both phases keep the order of
// one fragment stream read PD ahead: 13.34 -> 13.08 ms on that attention
// (bitwise identical); 2, 3, 5 and 6 ahead were slower.  The 4-wave kernels
// leave it unpinned: there it spills.
template <int HD, int QB, bool NEXT, bool MASK_NEXT, bool PIN = false>
__device__ __forceinline__ void tile_step(const char* __restrict__ lk_next,
                                          const char* __restrict__ lv_cur, const FragAddr<HD>& fa,
                                          const bf16x8 (&qf)[QB][HD / 16], const f32x16 (&s_cur)[QB][2],
                                          f32x16 (&s_next)[QB][2], SoftmaxState<HD, QB>& st,
                                          float scale_log2, int valid_next, float (&mx)[QB]) {
    constexpr int NF = HD / 8;        // fragments per phase (K fragments = V^T fragments)
    constexpr int EP = 32 / NF;       // score elements per lane and query block per fragment
    constexpr int DP = 16 / NF;       // fp16 pairs summed per query block per fragment
    float mneg[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) mneg[qb] = -st.m_run[qb];

    // ---- phase 1 ----
    constexpr int PD = 4;             // LDS fragment prefetch depth
    bf16x8 kf[PD];
    if (NEXT) {
#pragma unroll
        for (int j = 0; j < PD; ++j) kf[j] = k_frag<HD>(lk_next, fa, j);
    }
    f16x8 pf[QB][4];
#pragma unroll
    for (int i = 0; i < NF; ++i) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            if (NEXT) {
                const int kb = i & 1;
                if (i < 2) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) s_next[qb][kb][r] = 0.f;
                }
                s_next[qb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i % PD], qf[qb][i >> 1],
                                                                         s_next[qb][kb], 0, 0, 0);
            }
#pragma unroll
            for (int e = i * EP; e < (i + 1) * EP; ++e) {
                const int kb = e >> 4, r = e & 15;
                const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s_cur[qb][kb][r], scale_log2, mneg[qb]));
                pf[qb][2 * kb + (r >> 3)][r & 7] = (_Float16)p;
            }
        }
        if (NEXT && i + PD < NF) kf[i % PD] = k_frag<HD>(lk_next, fa, i + PD);
    }

    // ---- phase 2 ----
    f16x8 vf[PD];
#pragma unroll
    for (int j = 0; j < PD; ++j) vf[j] = v_frag<HD>(lv_cur, fa, j);
    float ls[QB], mxl[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        ls[qb] = 0.f;
        mxl[qb] = -__builtin_inff();
    }
    const f16x2 ones = {(_Float16)1.f, (_Float16)1.f};
#pragma unroll
    for (int i = 0; i < NF; ++i) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            st.o[qb][i >> 2] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf[i % PD], pf[qb][i & 3], st.o[qb][i >> 2],
                                                                      0, 0, 0);
#pragma unroll
            for (int q = i * DP; q < (i + 1) * DP; ++q) {
                const f16x2 pair = {pf[qb][q >> 2][2 * (q & 3)], pf[qb][q >> 2][2 * (q & 3) + 1]};
                ls[qb] = __builtin_amdgcn_fdot2(pair, ones, ls[qb], false);
            }
            if (NEXT && !MASK_NEXT) {
#pragma unroll
                for (int e = i * EP; e < (i + 1) * EP; ++e) mxl[qb] = fmaxf(mxl[qb], s_next[qb][e >> 4][e & 15]);
            }
        }
        if (i + PD < NF) vf[i % PD] = v_frag<HD>(lv_cur, fa, i + PD);
    }
    if constexpr (PIN) {
        static_assert(QB == 1, "one MFMA per fragment");
        order_fragment_stream<PD, NEXT ? 2 * NF : NF>();
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) st.l_run[qb] += ls[qb];
    if (!NEXT) return;
    if (MASK_NEXT) {
        tile_max<true, QB>(s_next, scale_log2, valid_next, mx);
        return;
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) mx[qb] = pair_max(mxl[qb]) * scale_log2;
}

// 16-byte global load as a bf16 fragment (zero when !ok).
__device__ __forceinline__ bf16x8 load_bf16x8(const __bf16* p, bool ok) {
    uint4 u = make_uint4(0, 0, 0, 0);
    if (ok) u = *reinterpret_cast<const uint4*>(p);
    return __builtin_bit_cast(bf16x8, u);
}

// Asynchronous 16-byte global -> LDS copy for every lane of the wave; lane i
// writes lds_wave_base + 16 i.  lds_wave_base must be wave-uniform.
__device__ __forceinline__ void dma16(const void* g, char* lds_wave_base) {
    __builtin_amdgcn_global_load_lds(g, MMDIT_LDS(lds_wave_base), 16, 0, 0);
}

// Wait until this wave's global -> LDS copies have landed.  The copies count
// against vmcnt, but the compiler does not treat them as outstanding memory
// operations at a workgroup barrier, so every barrier that publishes copied
// tiles is preceded by this explicit wait (s_waitcnt vmcnt(0); the immediate
// keeps expcnt and lgkmcnt at their no-wait maxima).
__device__ __forceinline__ void wait_dma() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Wait until at most N of this wave's global -> LDS copies are outstanding
// (copies complete in issue order).  The 6-bit vmcnt field of the s_waitcnt
// immediate is split over bits 3:0 and 15:14; expcnt and lgkmcnt stay at
// their no-wait maxima.
template <int N>
__device__ __forceinline__ void wait_dma_upto() {
    static_assert(N >= 0 && N < 64, "vmcnt immediate");
    __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Wave index as a scalar (uniform) value.
__device__ __forceinline__ int wave_id() {
    return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}

// Store the normalised (or raw) O^T accumulators of one query block for this
// lane's query row.
template <int HD>
__device__ __forceinline__ void store_o(float* orow, const f32x16 (&o)[HD / 32], float mul) {
    const int hh = (threadIdx.x & 63) >> 5;
#pragma unroll
    for (int db = 0; db < HD / 32; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int d0 = 32 * db + 8 * g + 4 * hh;
            *reinterpret_cast<float4*>(orow + d0) =
                make_float4(o[db][4 * g] * mul, o[db][4 * g + 1] * mul,
                            o[db][4 * g + 2] * mul, o[db][4 * g + 3] * mul);
        }
}

}  // namespace mmdit
