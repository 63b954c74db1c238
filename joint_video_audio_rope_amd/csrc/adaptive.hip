// Content-adaptive 3D block shapes for the block-sparse video attention
// (Prism page, xyznot.com 2610.05416: "Ideas clave", the dual-guidance
// variation indicator and the 16 candidate shapes; "Metodo" sections 1 and 2).
//
//   zone_stats   one pass over V (and the audio norms a): for every 8x8x8
//                macro-zone and channel, the mean of V over the other two axes
//                at each of the 8 positions along t, h and w, and the variance
//                of those means; summed over a chunk of channels (HBM-bound:
//                reads V once).
//   zone_shapes  one workgroup: per zone the variance shares r_{v,d}, the
//                density rho (zone energy over the largest), the volume B from
//                rho against 0.5 and 0.25, the audio coupling abar and shares
//                vhat_{a,d}, g_d = r_{v,d} + abar vhat_{a,d} + eps, the log2
//                optimum l*_d and the nearest candidate of volume B; then the
//                tile tables the sparse kernels read.
//
// Blocks stay 64-token tiles inside the sparse kernels: a block of B tokens is
// B / 64 consecutive tiles that share its pooled means and its selection, so
// the uniform tile machinery runs unchanged.  Inside a block, tiles halve the
// longest edge (the first of t, h, w among equals) once per factor of two;
// tiles are numbered in raster order of their position in the block, blocks
// in raster order of their position in the zone, zones in raster order.
//
// Readings where the page leaves a step open: candidates are the boxes with
// edges in {2, 4, 8} and volume 64, 128 or 256 (exactly 16), ordered by
// volume then (b_T, b_H, b_W), ties to the first; D counts every channel
// (heads x head_dim); rho = E / max E with E = sum_d sigma2_{v,d}; abar = zone
// mean of a over the largest zone mean; vhat the directional variance of a
// over its sum; shares of a zero total are 0; eps = 1e-6.  All of it is fp64,
// so the discrete choices (volume, shape) are taken in the same precision as
// the double-precision reference.
#include "internal.hpp"

namespace mmdit {

namespace {

constexpr double kTau128 = 0.5;
constexpr double kTau256 = 0.25;
constexpr double kEps = 1e-6;

__device__ __forceinline__ int64_t zone_origin(const SparseGeom& g, int m) {
    const int zt = m / (g.nzh * g.nzw);
    const int zr = m - zt * (g.nzh * g.nzw);
    const int zh = zr / g.nzw;
    const int zw = zr - zh * g.nzw;
    return ((int64_t)(zt * kZoneEdge) * g.H + zh * kZoneEdge) * g.W + zw * kZoneEdge;
}

// Sum over 8 positions of (mean at the position - zone mean)^2, / 8.
__device__ __forceinline__ double axis_var(const double (&s)[8], double mu) {
    double acc = 0.0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const double d = s[i] * (1.0 / 64.0) - mu;
        acc += d * d;
    }
    return acc * 0.125;
}

// Grid (zones, chunks + 1): workgroup (m, y < chunks) covers channel pairs
// 256 y .. 256 y + 255 of zone m; (m, chunks) covers the audio norms.
// part[(m * chunks + y) * 3 + d] = sum over the chunk's channels of
// (1 / 8) sum_i (Vbar_{i}^{(d)} - mu)^2.  Sums of 64 and 512 bf16 values are
// exact in fp64, so the means do not depend on the summation order.
template <int HD>
__global__ __launch_bounds__(kStatPairs) void zone_stats_kernel(SparseGeom g, const __bf16* __restrict__ v,
                                                                const float* __restrict__ a, int chunks,
                                                                double* __restrict__ part,
                                                                double* __restrict__ audio) {
#pragma clang fp contract(off)
    __shared__ double red[3][kStatPairs];
    __shared__ double av[512];
    __shared__ double axs[3][8];
    const int m = blockIdx.x, y = blockIdx.y, tid = threadIdx.x;
    const int64_t org = zone_origin(g, m);
    if (y < chunks) {
        const int D = g.heads * HD;
        const int cp = y * kStatPairs + tid;
        double var[3] = {0.0, 0.0, 0.0};
        if (2 * cp < D) {
            double sT[2][8], sH[2][8], sW[2][8];
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int i = 0; i < 8; ++i) sT[c][i] = sH[c][i] = sW[c][i] = 0.0;
            const uint32_t* src = reinterpret_cast<const uint32_t*>(v) + cp;
            const int64_t rs = D / 2;   // uint32 words per token
#pragma unroll
            for (int t = 0; t < 8; ++t)
#pragma unroll
                for (int h = 0; h < 8; ++h) {
                    uint32_t u[8];
#pragma unroll
                    for (int w = 0; w < 8; ++w)
                        u[w] = __builtin_nontemporal_load(src + (org + ((int64_t)t * g.H + h) * g.W + w) * rs);
#pragma unroll
                    for (int w = 0; w < 8; ++w) {
                        const double x0 = (double)__uint_as_float(u[w] << 16);
                        const double x1 = (double)__uint_as_float(u[w] & 0xFFFF0000u);
                        sT[0][t] += x0, sH[0][h] += x0, sW[0][w] += x0;
                        sT[1][t] += x1, sH[1][h] += x1, sW[1][w] += x1;
                    }
                }
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                double tot = 0.0;
#pragma unroll
                for (int i = 0; i < 8; ++i) tot += sT[c][i];
                const double mu = tot * (1.0 / 512.0);
                var[0] += axis_var(sT[c], mu);
                var[1] += axis_var(sH[c], mu);
                var[2] += axis_var(sW[c], mu);
            }
        }
#pragma unroll
        for (int d = 0; d < 3; ++d) red[d][tid] = var[d];
        __syncthreads();
        for (int o = kStatPairs / 2; o > 0; o >>= 1) {
            if (tid < o)
#pragma unroll
                for (int d = 0; d < 3; ++d) red[d][tid] += red[d][tid + o];
            __syncthreads();
        }
        if (tid < 3) part[((int64_t)m * chunks + y) * 3 + tid] = red[tid][0];
        return;
    }
    // audio norms: 512 values of the zone, raster (t, h, w) inside it
    for (int i = tid; i < 512; i += kStatPairs)
        av[i] = a ? (double)a[org + ((int64_t)(i >> 6) * g.H + ((i >> 3) & 7)) * g.W + (i & 7)] : 0.0;
    __syncthreads();
    if (tid < 24) {
        const int d = tid >> 3, idx = tid & 7;
        double s = 0.0;
        for (int j = 0; j < 64; ++j) {
            // the j-th of the 64 tokens whose coordinate along d is idx
            const int p = j >> 3, q = j & 7;
            const int i = d == 0 ? (idx << 6) | (p << 3) | q : d == 1 ? (p << 6) | (idx << 3) | q
                                                                      : (p << 6) | (q << 3) | idx;
            s += av[i];
        }
        axs[d][idx] = s;
    }
    __syncthreads();
    if (tid == 0) {
        double tot = 0.0;
        for (int i = 0; i < 8; ++i) tot += axs[0][i];
        const double mu = tot * (1.0 / 512.0);
        audio[m * 4 + 0] = mu;
        for (int d = 0; d < 3; ++d) {
            double s[8];
            for (int i = 0; i < 8; ++i) s[i] = axs[d][i];
            audio[m * 4 + 1 + d] = axis_var(s, mu);
        }
    }
}

// One workgroup of 1024 threads; zones <= kMaxZones, up to four per thread.
__global__ __launch_bounds__(1024) void zone_shapes_kernel(SparseGeom g, int chunks, int channels,
                                                           AdaptiveWs w) {
#pragma clang fp contract(off)
    __shared__ double emax_s[16], amax_s[16];
    __shared__ int nbz[kMaxZones], zbase[kMaxZones];
    __shared__ uint8_t zcode[kMaxZones];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int nz = g.nb / kZoneTiles;
    // per-axis variance sums of zone m (channel means), their total E and the
    // zone's audio norm
    auto zone_energy = [&](int m, double (&s2)[3], double& E, double& am) {
        s2[0] = s2[1] = s2[2] = 0.0;
        for (int y = 0; y < chunks; ++y)
#pragma unroll
            for (int d = 0; d < 3; ++d) s2[d] += w.part[((int64_t)m * chunks + y) * 3 + d];
#pragma unroll
        for (int d = 0; d < 3; ++d) s2[d] /= (double)channels;
        E = (s2[0] + s2[1]) + s2[2];
        am = w.audio[m * 4];
    };
    double e = 0.0, x = 0.0;
    for (int m = tid; m < nz; m += 1024) {
        double s2[3], E, am;
        zone_energy(m, s2, E, am);
        e = fmax(e, E);
        x = fmax(x, am);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        e = fmax(e, __shfl_xor(e, o));
        x = fmax(x, __shfl_xor(x, o));
    }
    if (lane == 0) emax_s[wv] = e, amax_s[wv] = x;
    __syncthreads();
    double emax = 0.0, amax = 0.0;
    for (int i = 0; i < 16; ++i) emax = fmax(emax, emax_s[i]), amax = fmax(amax, amax_s[i]);
    for (int m = tid; m < nz; m += 1024) {
        double s2[3], E, am;
        zone_energy(m, s2, E, am);
        const double rho = emax > 0.0 ? E / emax : 0.0;
        const int lb = rho >= kTau128 ? 6 : rho >= kTau256 ? 7 : 8;   // log2 B
        const double abar = amax > 0.0 ? am / amax : 0.0;
        const double sa[3] = {w.audio[m * 4 + 1], w.audio[m * 4 + 2], w.audio[m * 4 + 3]};
        const double st = (sa[0] + sa[1]) + sa[2];
        double lg[3];
#pragma unroll
        for (int d = 0; d < 3; ++d) {
            const double r = E > 0.0 ? s2[d] / E : 0.0;
            const double vh = st > 0.0 ? sa[d] / st : 0.0;
            lg[d] = log2((r + abar * vh) + kEps);
        }
        const double c3 = ((double)lb + 0.5 * ((lg[0] + lg[1]) + lg[2])) / 3.0;
        // first candidate of the volume; stays the choice if every distance is
        // NaN (non-finite inputs)
        int best = lb == 6 ? 0 : lb == 7 ? 7 : 13;
        double bd = __builtin_inf();
        for (int i = 0; i < 16; ++i) {
            int ed[3];
            adaptive_candidate(i, ed[0], ed[1], ed[2]);
            if (ed[0] + ed[1] + ed[2] != lb) continue;
            double dist = 0.0;
#pragma unroll
            for (int d = 0; d < 3; ++d) {
                const double diff = (double)ed[d] - (-0.5 * lg[d] + c3);
                dist += diff * diff;
            }
            if (dist < bd) bd = dist, best = i;
        }
        zcode[m] = (uint8_t)best;
        nbz[m] = 1 << (9 - lb);
        w.code[m] = (uint8_t)best;
    }
    __syncthreads();
    if (tid == 0) {
        int acc = 0;
        for (int i = 0; i < nz; ++i) zbase[i] = acc, acc += nbz[i];
        *w.nblocks = acc;
    }
    __syncthreads();
    for (int s = tid; s < nz * kZoneTiles; s += 1024) {
        const int zm = s / kZoneTiles;
        const TileGeom tg = tile_geom(g, s, zcode[zm]);
        w.base[s] = (int32_t)tg.base;
        w.tdim[s] = (uint8_t)tg.dims;
        w.lead[s] = s - tg.sub;
        w.tblock[s] = zbase[zm] + tg.blk;
    }
}

// First raster token and log2 edges of every tile: one thread per tile.
// Codes outside 0..15 are clamped (they come from a forward call of this
// library).
__global__ __launch_bounds__(256) void tile_table_kernel(SparseGeom g, const uint8_t* __restrict__ codes,
                                                         int32_t* __restrict__ tbase, uint8_t* __restrict__ tdim) {
    const int s = (int)(blockIdx.x * 256 + threadIdx.x);
    if (s >= g.nb) return;
    const TileGeom tg = tile_geom(g, s, min((int)codes[s / kZoneTiles], 15));
    tbase[s] = (int32_t)tg.base;
    tdim[s] = (uint8_t)tg.dims;
}


// out[t] = sqrt(sum_c x[t][c]^2), one workgroup of 256 threads per token,
// float4 loads, fp32 sums in a fixed tree order.
__global__ __launch_bounds__(256) void token_norms_kernel(const float* __restrict__ x, int64_t width,
                                                          float* __restrict__ out) {
    __shared__ float red[256];
    const int64_t t = blockIdx.x;
    const float* row = x + t * width;
    float acc = 0.f;
    for (int64_t c = 4 * (int64_t)threadIdx.x; c < width; c += 4 * 256) {
        typedef float f32x4 __attribute__((ext_vector_type(4)));
        const f32x4 u = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(row + c));
        acc += u[0] * u[0] + u[1] * u[1] + u[2] * u[2] + u[3] * u[3];
    }
    red[threadIdx.x] = acc;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
        if ((int)threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
        __syncthreads();
    }
    if (threadIdx.x == 0) out[t] = sqrtf(red[0]);
}

}  // namespace

hipError_t launch_token_norms(const float* x, int64_t n, int64_t width, float* out, hipStream_t s) {
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(token_norms_kernel, dim3((uint32_t)n), dim3(256), 0, s, x, width, out);
    return hipGetLastError();
}

int zone_stat_chunks(int heads, int hd) { return (heads * hd / 2 + kStatPairs - 1) / kStatPairs; }

hipError_t launch_tile_table(const SparseGeom& g, const uint8_t* codes, int32_t* tbase, uint8_t* tdim,
                             hipStream_t s) {
    hipLaunchKernelGGL(tile_table_kernel, dim3((unsigned)((g.nb + 255) / 256)), dim3(256), 0, s, g, codes, tbase,
                       tdim);
    return hipGetLastError();
}

hipError_t launch_zone_stats(const SparseGeom& g, const __bf16* v, const float* a, int hd, const AdaptiveWs& w,
                             hipStream_t s) {
    if (hd != 128) return hipErrorInvalidValue;
    const int chunks = zone_stat_chunks(g.heads, hd);
    const int nz = g.nb / kZoneTiles;
    hipLaunchKernelGGL(zone_stats_kernel<128>, dim3(nz, chunks + 1), dim3(kStatPairs), 0, s, g, v, a, chunks,
                       w.part, w.audio);
    return hipGetLastError();
}

hipError_t launch_zone_shapes(const SparseGeom& g, int hd, const AdaptiveWs& w, hipStream_t s) {
    if (g.nb / kZoneTiles > kMaxZones) return hipErrorInvalidValue;
    hipLaunchKernelGGL(zone_shapes_kernel, dim3(1), dim3(1024), 0, s, g, zone_stat_chunks(g.heads, hd),
                       g.heads * hd, w);
    return hipGetLastError();
}

}  // namespace mmdit
