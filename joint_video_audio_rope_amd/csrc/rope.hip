// Time-shifted 3D rotary embedding, applied in place to Q and K.
//
// Positions follow the SkyReels-V4 pages (paper.rainbus.top analysis,
// workflow step 1 and novelties 4-5; trdm.cn article section 2.2): video
// tokens turn their t | h | w slices by their frame, row and column, with
// conditioning frames at negative t; audio token j turns only the temporal
// slice, at position j * t_scale; text is left alone.  The host builds the
// (cos, sin) table in fp64 and rounds it to fp32; this kernel only looks it up.
//
// HBM-bound: one thread per 16-byte chunk of Q and the same chunk of K, so a
// wavefront reads and writes 1 KiB contiguous per tensor and the table
// (tens of KiB) stays in cache.  Bytes per rotated token = heads * head_dim *
// elem * 2 tensors * (read + write).
#include "internal.hpp"

namespace mmdit {

namespace {

template <int EPC>
struct Chunk;

template <>
struct Chunk<8> {  // 8 bf16
    __device__ static void load(const void* p, float (&x)[8]) {
        const uint4 u = *reinterpret_cast<const uint4*>(p);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = __uint_as_float(w[i] << 16);
            x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
    __device__ static void store(void* p, const float (&x)[8]) {
        bf16x8 v;
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = (__bf16)x[i];
        *reinterpret_cast<bf16x8*>(p) = v;
    }
    static constexpr int kBytes = 2;
};

template <>
struct Chunk<4> {  // 4 fp32
    __device__ static void load(const void* p, float (&x)[4]) {
        const float4 u = *reinterpret_cast<const float4*>(p);
        x[0] = u.x, x[1] = u.y, x[2] = u.z, x[3] = u.w;
    }
    __device__ static void store(void* p, const float (&x)[4]) {
        *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
    }
    static constexpr int kBytes = 4;
};

template <int EPC>
__global__ __launch_bounds__(256) void rope_kernel(RopeArgs a, const float2* __restrict__ tab,
                                                   char* __restrict__ q, char* __restrict__ k) {
    const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (g >= a.total_chunks) return;
    int s = 0;
    while (s + 1 < a.n_segs && g >= a.seg[s].chunk_end) ++s;
    const RopeSeg& sg = a.seg[s];
    const int c = (int)(g - sg.chunk_begin);
    const int tok = c / a.chunks_per_token;
    const int e = (c - tok * a.chunks_per_token) * EPC;   // element inside the token row
    const int dim = e % a.head_dim;

    int t_idx;                // float2 index of this chunk's first pair
    if (dim < a.d_t) {
        const int p = sg.kind == MMDIT_SEG_VIDEO ? tok / (sg.H * sg.W) : tok;
        t_idx = sg.tab_t + p * (a.d_t >> 1) + (dim >> 1);
    } else if (sg.kind != MMDIT_SEG_VIDEO) {
        return;               // audio: h and w slices sit at position 0
    } else if (dim < a.d_t + a.d_h) {
        const int p = (tok / sg.W) % sg.H;
        t_idx = sg.tab_h + p * (a.d_h >> 1) + ((dim - a.d_t) >> 1);
    } else {
        const int p = tok % sg.W;
        t_idx = sg.tab_w + p * (a.d_w >> 1) + ((dim - a.d_t - a.d_h) >> 1);
    }
    float2 cs[EPC / 2];
#pragma unroll
    for (int i = 0; i < EPC / 2; ++i) cs[i] = tab[t_idx + i];

    const int64_t off =
        ((sg.offset + tok) * (int64_t)(a.heads * a.head_dim) + e) * Chunk<EPC>::kBytes;
    float xq[EPC], xk[EPC];
    Chunk<EPC>::load(q + off, xq);
    Chunk<EPC>::load(k + off, xk);
#pragma unroll
    for (int i = 0; i < EPC / 2; ++i) {
        rope_pair(xq[2 * i], xq[2 * i + 1], cs[i].x, cs[i].y, xq[2 * i], xq[2 * i + 1]);
        rope_pair(xk[2 * i], xk[2 * i + 1], cs[i].x, cs[i].y, xk[2 * i], xk[2 * i + 1]);
    }
    Chunk<EPC>::store(q + off, xq);
    Chunk<EPC>::store(k + off, xk);
}

}  // namespace

hipError_t launch_rope(const RopeArgs& a, const float* table, void* q, void* k, int dtype,
                       hipStream_t s) {
    if (a.total_chunks == 0) return hipSuccess;
    const int threads = 256;
    const int64_t blocks = (a.total_chunks + threads - 1) / threads;
    const float2* tab = reinterpret_cast<const float2*>(table);
    if (dtype == MMDIT_BF16)
        hipLaunchKernelGGL(rope_kernel<8>, dim3((unsigned)blocks), dim3(threads), 0, s, a, tab,
                           (char*)q, (char*)k);
    else
        hipLaunchKernelGGL(rope_kernel<4>, dim3((unsigned)blocks), dim3(threads), 0, s, a, tab,
                           (char*)q, (char*)k);
    return hipGetLastError();
}

}  // namespace mmdit
