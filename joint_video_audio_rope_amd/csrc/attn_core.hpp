// Shared inner loop of the bf16 attention kernels (dense and block-sparse).
//
// One wavefront owns 32 queries.  Per 64-key tile it computes the transposed
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
// LDS layouts use an XOR swizzle on 16-byte chunks (chunk ^ (row & 7)) so the
// 8 lanes that read one chunk column at a time hit 8 different bank groups.
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
    __device__ static int k_off(int row, int chunk) {
        return row * kKRowBytes + ((chunk ^ (row & 7)) << 4);
    }
    __device__ static int v_off(int d, int chunk) {
        return d * kVRowBytes + ((chunk ^ (d & 7)) << 4);
    }
    // Inverse maps: which (row, chunk) lives at LDS chunk index L.
    __device__ static void k_at(int L, int& row, int& chunk) {
        row = L / kKChunks;
        chunk = (L % kKChunks) ^ (row & 7);
    }
    __device__ static void v_at(int L, int& d, int& chunk) {
        d = L >> 3;
        chunk = (L & 7) ^ (d & 7);
    }
};

template <int HD>
struct SoftmaxState {
    static constexpr int DB = HD / 32;
    f32x16 o[DB];
    float m_run;   // reference max of scaled logits (log2 domain)
    float l_run;   // running sum over this lane's half of the keys
    __device__ void init() {
#pragma unroll
        for (int i = 0; i < DB; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[i][r] = 0.f;
        m_run = -__builtin_inff();
        l_run = 0.f;
    }
};

// One 64-key tile.  `valid` keys (<= 64) of the tile are real; with MASK the
// rest are masked out.  qf: the wave's Q fragments (B operand), one per 16-d
// step.  scale_log2 = softmax scale * log2(e) > 0.
template <int HD, bool MASK>
__device__ __forceinline__ void attn_tile(const char* __restrict__ lk, const char* __restrict__ lv,
                                          const bf16x8 (&qf)[HD / 16], SoftmaxState<HD>& st,
                                          float scale_log2, int valid) {
    using L = TileLayout<HD>;
    constexpr int KS = HD / 16;
    constexpr int DB = HD / 32;
    const int lane = threadIdx.x & 63;
    const int hh = lane >> 5;
    const int m = lane & 31;

    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const bf16x8 a =
                *reinterpret_cast<const bf16x8*>(lk + L::k_off(32 * kb + m, 2 * ks + hh));
            s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s[kb], 0, 0, 0);
        }
    }

    if (MASK) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (tile_key(kb, r, hh) >= valid) s[kb][r] = -__builtin_inff();
    }
    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32)) * scale_log2;

    if (__any(mx > st.m_run + 8.f)) {
        const float m_new = fmaxf(st.m_run, mx);
        const float alpha = __builtin_amdgcn_exp2f(st.m_run - m_new);
        st.m_run = m_new;
        st.l_run *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) st.o[db][r] *= alpha;
    }
    const float mneg = -st.m_run;

    float ls = 0.f;
    f16x8 pf[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], scale_log2, mneg));
            ls += p;
            pf[2 * kb + (r >> 3)][r & 7] = (_Float16)p;
        }
    st.l_run += ls;

#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const f16x8 a = *reinterpret_cast<const f16x8*>(lv + L::v_off(32 * db + m, 2 * g + hh));
            st.o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pf[g], st.o[db], 0, 0, 0);
        }
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

// Wave index as a scalar (uniform) value.
__device__ __forceinline__ int wave_id() {
    return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}

// Store the normalised (or raw) O^T accumulators of this lane's query row.
template <int HD>
__device__ __forceinline__ void store_o(float* orow, const SoftmaxState<HD>& st, float mul) {
    const int hh = (threadIdx.x & 63) >> 5;
#pragma unroll
    for (int db = 0; db < HD / 32; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int d0 = 32 * db + 8 * g + 4 * hh;
            *reinterpret_cast<float4*>(orow + d0) =
                make_float4(st.o[db][4 * g] * mul, st.o[db][4 * g + 1] * mul,
                            st.o[db][4 * g + 2] * mul, st.o[db][4 * g + 3] * mul);
        }
}

}  // namespace mmdit
